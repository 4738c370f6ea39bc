// Fused RoPE + append for one layer.
//
// q is rotated in place; k is rotated and written with v into the staging slot of its
// stream-batch element ([NEWS] method, algorithm item 1: the new frames' KV enter the rolling
// cache; [WT] adaptive sink and RoPE refresh: keys and queries carry the RoPE phase of their
// frame index relative to the current base).  RoPE: interleaved pairs; the first pt pairs turn
// by the temporal angle (per element, from the host), the next ph by the row angle and the last
// pw by the column angle of the token (tables in device memory).
//
// One workgroup per (frame of the chunk, 64-token tile of the frame, head, element); 16-byte
// loads and stores throughout, the stores with the non-temporal hint (the attention reads the
// rows later, from HBM).  K rows go to the cache as [token][d]; V goes through LDS and
// leaves transposed as [d][token] rows of the tile, so the attention kernel can read V^T
// fragments contiguously.  Frame t of element b has its own slot and temporal angle.
#include "common.h"

#include <type_traits>

namespace sdv2 {

// m: a factor on the rotated values before their rounding (the cache's key scale for k, 1 for
// q: a product by 1 is exact).
template <bool BF16>
__device__ __forceinline__ void rotate16(uint4& w, const float2* cs, float m = 1.f) {
  if constexpr (BF16) {
    uint32_t* u = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = bf16_bits_to_f32(u[j] & 0xffffu), y = bf16_bits_to_f32(u[j] >> 16);
      u[j] = pack_bf16x2((x * cs[j].x - y * cs[j].y) * m, (x * cs[j].y + y * cs[j].x) * m);
    }
  } else {
    float* f = reinterpret_cast<float*>(&w);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float x = f[2 * j], y = f[2 * j + 1];
      f[2 * j] = x * cs[j].x - y * cs[j].y;
      f[2 * j + 1] = x * cs[j].y + y * cs[j].x;
    }
  }
}

// The 8 values of a 16-byte bf16 chunk rotated in fp32 (pairs as in rotate16), for the e4m3 path
// which rounds once from fp32.
__device__ __forceinline__ void rotate8_f32(const uint4& w, const float2* cs, float* out) {
  const uint32_t* u = reinterpret_cast<const uint32_t*>(&w);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x = bf16_bits_to_f32(u[j] & 0xffffu), y = bf16_bits_to_f32(u[j] >> 16);
    out[2 * j] = x * cs[j].x - y * cs[j].y;
    out[2 * j + 1] = x * cs[j].y + y * cs[j].x;
  }
}

// KV: cache element type (kKvF32, kKvBF16, kKvFP8); q, k, v are fp32 for kKvF32, else bf16.
// TILE: tokens per workgroup, 64 (a key tile) or 32 (half of one, for grids that would leave
// CUs idle; not for e4m3, whose V^T byte order spans a whole key tile).
template <int KV, int D, int TILE>
__global__ __launch_bounds__(256) void rope_append_kernel(const AppendArgs a) {
  constexpr bool BF16 = KV != kKvF32;
  using T = typename std::conditional<BF16, uint16_t, float>::type;   // activations
  using TC = typename std::conditional<KV == kKvFP8, uint8_t, T>::type;  // cache elements
  constexpr int VEC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int CH = D / VEC;                // chunks per row
  constexpr int ROWS = 256 / CH;             // token rows per pass
  static_assert(TILE == kTileKeys || (TILE == kTileKeys / 2 && KV != kKvFP8), "tile");
  constexpr int VSTR = D + (BF16 ? 2 : 1);   // LDS row stride (elements): breaks bank aliasing
  __shared__ T vs[TILE * VSTR];

  const int tiles = (a.N + kTileKeys - 1) / kTileKeys * (kTileKeys / TILE);   // padding included
  const int t = blockIdx.x / tiles;                // frame of the chunk
  const int n0 = (blockIdx.x - t * tiles) * TILE, head = blockIdx.y, b = blockIdx.z;
  const int fr = b * a.T + t;                      // frame index within the call
  const int tid = threadIdx.x;

  const int c = tid % CH;
  const int64_t kdst = a.k_layer_off + (int64_t)a.dst_slot[fr] * a.slot_stride +
                       (int64_t)head * a.head_stride;
  constexpr int PASSES = TILE / ROWS;
  // Every global load of the tile is issued before the first store (q is rotated in place, so
  // loads placed after a store could not be hoisted by the compiler and each pass would cost a
  // full memory round trip), and the q, k, v rows before the (cos, sin) values, which come
  // straight from the arguments and tables: nothing waits before the rows are requested.
  uint4 qv[PASSES], kv[PASSES], vv[PASSES];
  float2 cs[PASSES][VEC / 2];
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int n = n0 + pass * ROWS + tid / CH;
    if (n < a.N) {
      const int64_t off = ((int64_t)(fr * a.N + n) * a.H + head) * D + c * VEC;
      qv[pass] = *(const uint4*)((const T*)a.q + off);
      kv[pass] = *(const uint4*)((const T*)a.k + off);
      vv[pass] = *(const uint4*)((const T*)a.v + off);
    } else {                                   // padding tokens of V^T stay zero
      vv[pass] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int n = n0 + pass * ROWS + tid / CH;
    if (n < a.N) {
      const int hr = n / a.grid_w, wc = n - hr * a.grid_w;
#pragma unroll
      for (int j = 0; j < VEC / 2; ++j) {
        const int p = c * (VEC / 2) + j;
        cs[pass][j] = p < a.pt ? a.tcs[fr][p]
                      : p < a.pt + a.ph ? a.tab_h[hr * a.ph + (p - a.pt)]
                                        : a.tab_w[wc * a.pw + (p - a.pt - a.ph)];
      }
    }
  }
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int row = pass * ROWS + tid / CH;
    const int n = n0 + row;
    uint32_t* vrow = reinterpret_cast<uint32_t*>(vs + row * VSTR + c * VEC);
    vrow[0] = vv[pass].x; vrow[1] = vv[pass].y; vrow[2] = vv[pass].z; vrow[3] = vv[pass].w;
    if (n < a.N) {
      const int64_t off = ((int64_t)(fr * a.N + n) * a.H + head) * D + c * VEC;
      rotate16<BF16>(qv[pass], cs[pass]);
      store16_nt((T*)a.q + off, qv[pass]);
      if constexpr (KV == kKvFP8) {            // 8 dims -> one 8-byte unit at its e4m3 position
        float kr[8];
        rotate8_f32(kv[pass], cs[pass], kr);
#pragma unroll
        for (int j = 0; j < 8; ++j) kr[j] *= a.kmul;   // the cache's key factor, before the rounding
        const uint2 w = make_uint2(pack_fp8x4(kr[0], kr[1], kr[2], kr[3]),
                                   pack_fp8x4(kr[4], kr[5], kr[6], kr[7]));
        *(uint2*)((TC*)a.kv + kdst + (int64_t)n * D + fp8_pos(c * VEC)) = w;
      } else {
        rotate16<BF16>(kv[pass], cs[pass], a.kmul);
        store16_nt((TC*)a.kv + kdst + (int64_t)n * D + c * VEC, kv[pass]);
      }
    }
  }
  __syncthreads();

  // V^T rows: d-major, the tile's 64 tokens contiguous (e4m3: in fp8_pos order)
  constexpr int TVEC = 16 / (int)sizeof(TC);  // cache elements per 16-byte store
  constexpr int TCH = TILE / TVEC;            // 16-byte chunks per V^T row of the tile
  TC* vdst = (TC*)a.kv + a.v_layer_off + (int64_t)a.dst_slot[fr] * a.slot_stride +
             (int64_t)head * a.head_stride + n0;
  for (int idx = tid; idx < D * TCH; idx += 256) {
    const int drow = idx / TCH, kc = idx % TCH;
    uint4 w;
    if constexpr (KV == kKvFP8) {
      float f[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) f[j] = bf16_bits_to_f32(vs[fp8_pos(kc * 16 + j) * VSTR + drow]);
      w = make_uint4(pack_fp8x4(f[0], f[1], f[2], f[3]), pack_fp8x4(f[4], f[5], f[6], f[7]),
                     pack_fp8x4(f[8], f[9], f[10], f[11]), pack_fp8x4(f[12], f[13], f[14], f[15]));
    } else {
      T vals[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) vals[j] = vs[(kc * VEC + j) * VSTR + drow];
      __builtin_memcpy(&w, vals, sizeof(w));
    }
    store16_nt(vdst + (int64_t)drow * a.Npad + kc * TVEC, w);
  }
}

hipError_t launch_rope_append(const AppendArgs& a, int head_dim, int kv, hipStream_t s) {
  // Every workgroup loads its whole tile before storing, so one round of workgroups runs as a
  // load phase then a store phase: a grid under two rounds of the 256 CUs takes half tiles.
  const int tiles64 = (a.N + kTileKeys - 1) / kTileKeys;
  const bool half = kv != kKvFP8 && (int64_t)a.T * tiles64 * a.H * a.nbatch < 2 * 256;
  const dim3 grid(a.T * tiles64 * (half ? 2 : 1), a.H, a.nbatch);
#define SDV2_APPEND(KV_, D_)                                                                          \
  do {                                                                                               \
    if (half) hipLaunchKernelGGL((rope_append_kernel<KV_, D_, kTileKeys / 2>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((rope_append_kernel<KV_, D_, kTileKeys>), grid, dim3(256), 0, s, a);     \
  } while (0)
  if (kv == kKvFP8) {
    if (head_dim == 128)
      hipLaunchKernelGGL((rope_append_kernel<kKvFP8, 128, kTileKeys>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((rope_append_kernel<kKvFP8, 64, kTileKeys>), grid, dim3(256), 0, s, a);
  } else if (kv == kKvBF16) {
    if (head_dim == 128) SDV2_APPEND(kKvBF16, 128); else SDV2_APPEND(kKvBF16, 64);
  } else {
    if (head_dim == 128) SDV2_APPEND(kKvF32, 128); else SDV2_APPEND(kKvF32, 64);
  }
#undef SDV2_APPEND
  return hipGetLastError();
}

}  // namespace sdv2
