// Chunk attention over [sinks | window | own chunk] for gfx950.
//
// For every stream-batch element b and head: O = softmax(scale * Q_rot K^T) V over the keys of
// the present sink frames, the window frames and the element's own (staged) frame.  This is the
// attention of the causal DiT over the sink + rolling KV cache ([NEWS] method, algorithm item 1;
// [REPO] core components: ring-buffer KV cache with sliding-window attention); the walkthrough
// ([WT] SLO-aware batching scheduler) names FlashAttention as the exact tiled evaluation of it.
//
// bf16 path (split-KV, flash-style):
//  * workgroup = 4 waves x 32 query rows of one (element, head); grid = heads x splits x
//    elements x query tiles, remapped so that the workgroups sharing one head's K/V run on one
//    XCD (one L2);
//  * K tile [64 keys][d] and V^T tile [d][64 keys] (V is stored transposed in the cache) are
//    staged through LDS, double-buffered: the next tile's global loads are in flight while
//    the current tile is consumed;
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K as the A operand from LDS, Q^T as the B
//    operand held in registers for the whole kernel).  K rows are placed in LDS with bits 2
//    and 3 of the key index swapped so that the accumulator layout of S^T is already the B
//    operand layout of the P V product: every lane holds 8 consecutive keys of one query per
//    16-key step, so P never leaves registers;
//  * online softmax in base 2: one row max per 64-key tile (within the lane, then one lane
//    swap across the two 32-lane halves), exponentials by v_exp_f32, row sums kept per lane
//    and merged once at the end;
//  * O^T += V^T P^T with the same MFMA (V^T rows from LDS as the A operand);
//  * with several splits each workgroup writes (O/l, m, l) in fp32 and a combine kernel merges
//    them by log-sum-exp weights; with one split the output is normalised and written in bf16.
// fp32 path: a plain per-query-row kernel in fp32 (no reduced-precision matrix instructions).
#include "common.h"

#include <math.h>

namespace sdv2 {

constexpr float kLazy = 8.0f;   // lazy-rescale margin of the running max (log2 units)

// LDS row of key `key` within a 64-key tile: swap bits 2 and 3 of the key index.
__device__ __forceinline__ int perm_key(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const AttnArgs a) {
  constexpr int KSTR = D + 8;            // LDS row stride of the K tile (elements)
  constexpr int VSTR = kTileKeys + 8;    // LDS row stride of the V^T tile
  constexpr int K_ELEMS = kTileKeys * KSTR;
  constexpr int V_ELEMS = D * VSTR;
  constexpr int BUF = K_ELEMS + V_ELEMS;
  constexpr int NLD = D / 32;            // 16-byte chunks per thread per tile (K and V each)
  static_assert(NLD == 2 || NLD == 4, "head_dim 64 or 128");
  constexpr int KCH = D / 8;             // 16-byte chunks per K row
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BUF];

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int qtile = w % a.qtiles;
  int rest = w / a.qtiles;
  const int elem = rest % a.nbatch;
  rest /= a.nbatch;
  const int split = rest % a.nsplit;
  const int head = rest / a.nsplit;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r = lane & 31;
  const int qrow = qtile * kQTile + wave * 32 + r;
  const bool qvalid = qrow < a.N;

  // Q^T operand: lane (g, r) holds Q[row r][kd*16 + 8g .. +7] for every 16-wide k step.
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = (const uint16_t*)a.q +
                         ((int64_t)(elem * a.N + (qvalid ? qrow : 0)) * a.H + head) * D + g * 8;
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      const uint4 v = qvalid ? *(const uint4*)(qp + kd * 16) : make_uint4(0, 0, 0, 0);
      qf[kd] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int t_begin = (int)((int64_t)split * a.total_tiles / a.nsplit);
  const int t_end = (int)((int64_t)(split + 1) * a.total_tiles / a.nsplit);
  const uint16_t* kvb = (const uint16_t*)a.kv;

  // Prefetch registers for one K tile and one V^T tile (16-byte chunks c = i*256 + tid).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 rk0, rk1, rk2, rk3, rv0, rv1, rv2, rv3;
#define SDV2_LOAD_TILE(tile_)                                                                  \
  do {                                                                                         \
    const int f_ = (tile_) / a.tiles_per_frame;                                                \
    const int n0_ = ((tile_) - f_ * a.tiles_per_frame) * kTileKeys;                            \
    const int slot_ = f_ < a.nshared ? a.slots[f_] : a.own_slot0 + elem;                       \
    const int64_t sh_ = (int64_t)slot_ * a.slot_stride + (int64_t)head * a.head_stride;        \
    const uint16_t* kp_ = kvb + a.k_layer_off + sh_ + (int64_t)n0_ * D;                        \
    const uint16_t* vp_ = kvb + a.v_layer_off + sh_ + n0_;                                     \
    rk0 = *(const u32x4*)(kp_ + ((0 * 256 + tid) / KCH) * D + ((0 * 256 + tid) % KCH) * 8);    \
    rk1 = *(const u32x4*)(kp_ + ((1 * 256 + tid) / KCH) * D + ((1 * 256 + tid) % KCH) * 8);    \
    rv0 = *(const u32x4*)(vp_ + (int64_t)((0 * 256 + tid) / 8) * a.Npad + (tid % 8) * 8);      \
    rv1 = *(const u32x4*)(vp_ + (int64_t)((1 * 256 + tid) / 8) * a.Npad + (tid % 8) * 8);      \
    if constexpr (NLD == 4) {                                                                  \
      rk2 = *(const u32x4*)(kp_ + ((2 * 256 + tid) / KCH) * D + ((2 * 256 + tid) % KCH) * 8);  \
      rk3 = *(const u32x4*)(kp_ + ((3 * 256 + tid) / KCH) * D + ((3 * 256 + tid) % KCH) * 8);  \
      rv2 = *(const u32x4*)(vp_ + (int64_t)((2 * 256 + tid) / 8) * a.Npad + (tid % 8) * 8);    \
      rv3 = *(const u32x4*)(vp_ + (int64_t)((3 * 256 + tid) / 8) * a.Npad + (tid % 8) * 8);    \
    }                                                                                          \
  } while (0)
#define SDV2_STORE_TILE(buf_)                                                                  \
  do {                                                                                         \
    uint16_t* kt_ = lds + (buf_) * BUF;                                                        \
    uint16_t* vt_ = kt_ + K_ELEMS;                                                             \
    *(u32x4*)(kt_ + perm_key((0 * 256 + tid) / KCH) * KSTR + ((0 * 256 + tid) % KCH) * 8) = rk0; \
    *(u32x4*)(kt_ + perm_key((1 * 256 + tid) / KCH) * KSTR + ((1 * 256 + tid) % KCH) * 8) = rk1; \
    *(u32x4*)(vt_ + ((0 * 256 + tid) / 8) * VSTR + (tid % 8) * 8) = rv0;                       \
    *(u32x4*)(vt_ + ((1 * 256 + tid) / 8) * VSTR + (tid % 8) * 8) = rv1;                       \
    if constexpr (NLD == 4) {                                                                  \
      *(u32x4*)(kt_ + perm_key((2 * 256 + tid) / KCH) * KSTR + ((2 * 256 + tid) % KCH) * 8) = rk2; \
      *(u32x4*)(kt_ + perm_key((3 * 256 + tid) / KCH) * KSTR + ((3 * 256 + tid) % KCH) * 8) = rk3; \
      *(u32x4*)(vt_ + ((2 * 256 + tid) / 8) * VSTR + (tid % 8) * 8) = rv2;                     \
      *(u32x4*)(vt_ + ((3 * 256 + tid) / 8) * VSTR + (tid % 8) * 8) = rv3;                     \
    }                                                                                          \
  } while (0)

  const float sl = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;

  SDV2_LOAD_TILE(t_begin);
  SDV2_STORE_TILE(0);
  __syncthreads();

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int buf = (tile - t_begin) & 1;
    const bool more = tile + 1 < t_end;
    if (more) SDV2_LOAD_TILE(tile + 1);
    const uint16_t* kt = lds + buf * BUF;
    const uint16_t* vt = kt + K_ELEMS;

    // S^T for keys [0,32) and [32,64) of the tile (rows permuted, see perm_key)
    f32x16 s0, s1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      const bf16x8 a0 = *(const bf16x8*)(kt + r * KSTR + kd * 16 + g * 8);
      const bf16x8 a1 = *(const bf16x8*)(kt + (32 + r) * KSTR + kd * 16 + g * 8);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kd], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kd], s1, 0, 0, 0);
    }
    // lane (g, r), accumulator v holds key 16*(v/8) + 8g + v%8 (+32 for s1) of query r

    const int f = tile / a.tiles_per_frame;
    const int nvalid = a.N - (tile - f * a.tiles_per_frame) * kTileKeys;
    if (nvalid < kTileKeys) {                       // ragged last tile of a frame
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 16 * (v >> 3) + 8 * g + (v & 7);
        if (key >= nvalid) s0[v] = -INFINITY;
        if (key + 32 >= nvalid) s1[v] = -INFINITY;
      }
    }

    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescale: the running max m_run only moves when the tile max exceeds it by more than
    // kLazy (log2 units), so exponentials stay <= 2^kLazy and O/l is unchanged (both use m_run).
    // Once the max has settled no tile rescales O.
    const float m_tile = mx * sl;
    const bool grow = m_tile > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {          // wave-uniform branch
      const float m_new = grow ? m_tile : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    }
    const float m_new = m_run;

    uint32_t pw0[8], pw1[8];
    float ps = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[v], sl, -m_new));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s0[v + 1], sl, -m_new));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(s1[v], sl, -m_new));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(s1[v + 1], sl, -m_new));
      ps += (p0 + p1) + (p2 + p3);
      pw0[v / 2] = pack_bf16x2(p0, p1);
      pw1[v / 2] = pack_bf16x2(p2, p3);
    }
    l_run += ps;

    // P^T operands: 16-key step kk of key block kb covers accumulator entries 8kk..8kk+7
    const bf16x8 pb00 = __builtin_bit_cast(bf16x8, make_uint4(pw0[0], pw0[1], pw0[2], pw0[3]));
    const bf16x8 pb01 = __builtin_bit_cast(bf16x8, make_uint4(pw0[4], pw0[5], pw0[6], pw0[7]));
    const bf16x8 pb10 = __builtin_bit_cast(bf16x8, make_uint4(pw1[0], pw1[1], pw1[2], pw1[3]));
    const bf16x8 pb11 = __builtin_bit_cast(bf16x8, make_uint4(pw1[4], pw1[5], pw1[6], pw1[7]));
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const uint16_t* vr = vt + (i * 32 + r) * VSTR + g * 8;
      o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vr + 0), pb00, o[i], 0, 0, 0);
      o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vr + 16), pb01, o[i], 0, 0, 0);
      o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vr + 32), pb10, o[i], 0, 0, 0);
      o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vr + 48), pb11, o[i], 0, 0, 0);
    }

    if (more) SDV2_STORE_TILE(buf ^ 1);
    __syncthreads();
  }

  // lane (g, r), accumulator v of o[i] holds O^T[d = 32i + 8(v/4) + 4g + v%4][query r]
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  if (a.nsplit == 1) {
    uint16_t* op = (uint16_t*)a.out + ((int64_t)(elem * a.N + qrow) * a.H + head) * D + 4 * g;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        uint2 w2;
        w2.x = pack_bf16x2(o[i][4 * a4 + 0] * inv, o[i][4 * a4 + 1] * inv);
        w2.y = pack_bf16x2(o[i][4 * a4 + 2] * inv, o[i][4 * a4 + 3] * inv);
        *(uint2*)(op + 32 * i + 8 * a4) = w2;
      }
  } else {
    const int64_t prow = (((int64_t)split * a.nbatch + elem) * a.H + head) * a.N + qrow;
    float* po = a.part_o + prow * D + 4 * g;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        *(float4*)(po + 32 * i + 8 * a4) =
            make_float4(o[i][4 * a4] * inv, o[i][4 * a4 + 1] * inv, o[i][4 * a4 + 2] * inv,
                        o[i][4 * a4 + 3] * inv);
    if (g == 0) a.part_ml[prow] = make_float2(m_run, l_tot);
  }
#undef SDV2_LOAD_TILE
#undef SDV2_STORE_TILE
}

// Merge split-KV partials: O = sum_s w_s O_s / sum_s w_s, w_s = l_s 2^(m_s - max m).
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  constexpr int TPR = D / 4;                        // threads per output row
  const int64_t rows = (int64_t)a.nbatch * a.H * a.N;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int d0 = (threadIdx.x % TPR) * 4;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[s * rows + row].x);
  float W = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < a.nsplit; ++s) {
    const float2 ml = a.part_ml[s * rows + row];
    const float wgt = ml.y * __builtin_amdgcn_exp2f(ml.x - M);
    const float4 v = *(const float4*)(a.part_o + (s * rows + row) * D + d0);
    W += wgt;
    acc.x = fmaf(wgt, v.x, acc.x);
    acc.y = fmaf(wgt, v.y, acc.y);
    acc.z = fmaf(wgt, v.z, acc.z);
    acc.w = fmaf(wgt, v.w, acc.w);
  }
  const float inv = 1.f / W;
  const int n = (int)(row % a.N);
  const int eh = (int)(row / a.N);
  const int head = eh % a.H, elem = eh / a.H;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)(elem * a.N + n) * a.H + head) * D + d0;
  uint2 w2;
  w2.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  w2.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *(uint2*)op = w2;
}

// fp32: one query row per lane, 32-key tiles through LDS, online softmax per row.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnArgs a) {
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const int qtiles = (a.N + 63) / 64;
  const int qtile = blockIdx.x % qtiles;
  const int head = (blockIdx.x / qtiles) % a.H;
  const int elem = blockIdx.x / (qtiles * a.H);
  const int lane = threadIdx.x;
  const int n = qtile * 64 + lane;
  const bool valid = n < a.N;

  float q[D], o[D];
  const float* qp = (const float*)a.q + ((int64_t)(elem * a.N + (valid ? n : 0)) * a.H + head) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* kvb = (const float*)a.kv;
  for (int f = 0; f <= a.nshared; ++f) {
    const int slot = f < a.nshared ? a.slots[f] : a.own_slot0 + elem;
    const int64_t sh = (int64_t)slot * a.slot_stride + (int64_t)head * a.head_stride;
    const float* kp = kvb + a.k_layer_off + sh;
    const float* vp = kvb + a.v_layer_off + sh;
    for (int n0 = 0; n0 < a.N; n0 += KT) {
      __syncthreads();
      for (int idx = lane; idx < KT * D; idx += 64) {
        ks[idx / D][idx % D] = kp[(int64_t)(n0 + idx / D) * D + idx % D];
        vs[idx % KT][idx / KT] = vp[(int64_t)(idx / KT) * a.Npad + n0 + idx % KT];
      }
      __syncthreads();
      const int nv = min(KT, a.N - n0);
      float s[KT];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[j][d], acc);
        s[j] = j < nv ? acc * a.scale : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      const float alpha = expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        const float p = expf(s[j] - m_new);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(p, vs[j][d], o[d]);
      }
      m = m_new;
    }
  }
  if (!valid) return;
  float* op = (float*)a.out + ((int64_t)(elem * a.N + n) * a.H + head) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, bool bf16, hipStream_t s) {
  if (bf16) {
    const int grid = a.H * a.nsplit * a.nbatch * a.qtiles;
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  } else {
    const int grid = a.nbatch * a.H * ((a.N + 63) / 64);
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)a.nbatch * a.H * a.N;
  const int rows_per_block = 256 / (head_dim / 4);
  const int grid = (int)((rows + rows_per_block - 1) / rows_per_block);
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdv2
