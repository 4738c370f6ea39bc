// Cache maintenance kernels: slot copies (commit, sink replacement), RoPE rebase, the sink
// similarity decision and the per-frame motion reduction.
#include "common.h"

#include <math.h>

namespace sdv2 {

// ---- slot copy: K and V of one slot into another, every layer --------------------------------
// Commit ([NEWS] algorithm item 1, [REPO] ring-buffer KV cache): the finished element's staged
// frame enters slot S + f mod W (or sink slot f).  Sink replacement ([WT] adaptive sink and RoPE
// refresh): the committed frame enters the chosen sink slot, read from the device decision.
__global__ __launch_bounds__(256) void copy_slots_kernel(const CopyArgs a) {
  int dst = a.dst_slot;
  if (a.dst_from != nullptr) {
    dst = *a.dst_from;
    if (dst < 0) return;
  }
  const int layer = blockIdx.y >> 1, which = blockIdx.y & 1;
  char* base = a.kv + layer * a.layer_stride_bytes + which * a.v_block_bytes;
  const uint4* src = (const uint4*)(base + a.src_slot * a.slot_bytes);
  uint4* out = (uint4*)(base + dst * a.slot_bytes);
  const int64_t n = a.slot_bytes / 16;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = src[i];
}

hipError_t launch_copy_slots(const CopyArgs& a, hipStream_t s) {
  const int64_t n = a.slot_bytes / 16;
  int gx = (int)((n + 256 * 8 - 1) / (256 * 8));
  gx = gx < 1 ? 1 : gx > 512 ? 512 : gx;
  hipLaunchKernelGGL(copy_slots_kernel, dim3(gx, 2 * a.L), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- RoPE rebase: rotate the temporal pairs of cached K by the rebase angle -----------------
// [WT] adaptive sink and RoPE refresh: the RoPE phase is reset once the frame index passes the
// threshold; rotating every cached key by -delta on the temporal pairs (queries are rotated at
// the new base by the append) keeps every score unchanged.
template <int KV>
__global__ __launch_bounds__(256) void rebase_kernel(const RebaseArgs a, int D) {
  __shared__ float2 cs[kMaxTPairs];
  if ((int)threadIdx.x < a.pt) cs[threadIdx.x] = a.cs[threadIdx.x];
  __syncthreads();
  const int si = blockIdx.y / a.L, layer = blockIdx.y % a.L;
  const int64_t slot = a.slots[si];
  const int64_t npairs = (int64_t)a.H * a.N * a.pt;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < npairs;
       i += (int64_t)gridDim.x * 256) {
    const int p = (int)(i % a.pt);
    const int64_t rowi = i / a.pt;
    const int n = (int)(rowi % a.N), h = (int)(rowi / a.N);
    // dims 2p, 2p+1 stay adjacent in the e4m3 order (fp8_pos keeps bits 0-2)
    const int dpos = KV == kKvFP8 ? fp8_pos(2 * p) : 2 * p;
    const int64_t off = layer * a.layer_stride + slot * a.slot_stride + h * a.head_stride +
                        (int64_t)n * D + dpos;
    const float c = cs[p].x, sn = cs[p].y;
    if constexpr (KV == kKvFP8) {
      uint16_t* ptr = (uint16_t*)((uint8_t*)a.kv + off);
      const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)*ptr, false);
      *ptr = (uint16_t)(pack_fp8x4(v.x * c - v.y * sn, v.x * sn + v.y * c, 0.f, 0.f) & 0xffffu);
    } else if constexpr (KV == kKvBF16) {
      uint32_t* ptr = (uint32_t*)((uint16_t*)a.kv + off);
      const uint32_t w = *ptr;
      const float x = bf16_bits_to_f32(w & 0xffffu), y = bf16_bits_to_f32(w >> 16);
      *ptr = pack_bf16x2(x * c - y * sn, x * sn + y * c);
    } else {
      float2* ptr = (float2*)((float*)a.kv + off);
      const float2 v = *ptr;
      *ptr = make_float2(v.x * c - v.y * sn, v.x * sn + v.y * c);
    }
  }
}

hipError_t launch_rebase(const RebaseArgs& a, int head_dim, int kv, hipStream_t s) {
  const int64_t npairs = (int64_t)a.H * a.N * a.pt;
  int gx = (int)((npairs + 256 * 4 - 1) / (256 * 4));
  gx = gx < 1 ? 1 : gx > 1024 ? 1024 : gx;
  const dim3 grid(gx, a.nslots * a.L);
  if (kv == kKvFP8)
    hipLaunchKernelGGL(rebase_kernel<kKvFP8>, grid, dim3(256), 0, s, a, head_dim);
  else if (kv == kKvBF16)
    hipLaunchKernelGGL(rebase_kernel<kKvBF16>, grid, dim3(256), 0, s, a, head_dim);
  else
    hipLaunchKernelGGL(rebase_kernel<kKvF32>, grid, dim3(256), 0, s, a, head_dim);
  return hipGetLastError();
}

// ---- fp64 block reduction helpers -------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// ---- sink decision ------------------------------------------------------------------------------
// [WT] adaptive sink and RoPE refresh: cosine similarity of the new chunk embedding against each
// sink's embedding, in fp64 with a fixed reduction order; the least similar sink (lowest index on
// ties; similarity 0 when a norm is 0) is replaced when its similarity is below tau.  One block.
__global__ __launch_bounds__(256) void sink_decide_kernel(const SinkArgs a) {
  __shared__ double red[4][1 + 2 * kMaxSinks];
  __shared__ int dec;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.store_slot >= 0) {
    for (int i = tid; i < a.D; i += 256) a.embeds[(int64_t)a.store_slot * a.D + i] = a.h[i];
    if (tid == 0) {
      a.decision[0] = -1;
      a.alpha[0] = 1.0;
    }
    return;
  }
  double hh = 0.0, ee[kMaxSinks], he[kMaxSinks];
#pragma unroll
  for (int j = 0; j < kMaxSinks; ++j) { ee[j] = 0.0; he[j] = 0.0; }
  for (int i = tid; i < a.D; i += 256) {
    const double x = a.h[i];
    hh = fma(x, x, hh);
#pragma unroll
    for (int j = 0; j < kMaxSinks; ++j)
      if (j < a.S) {
        const double e = a.embeds[(int64_t)j * a.D + i];
        ee[j] = fma(e, e, ee[j]);
        he[j] = fma(x, e, he[j]);
      }
  }
  hh = wave_sum(hh);
#pragma unroll
  for (int j = 0; j < kMaxSinks; ++j)
    if (j < a.S) { ee[j] = wave_sum(ee[j]); he[j] = wave_sum(he[j]); }
  if (lane == 0) {
    red[wave][0] = hh;
#pragma unroll
    for (int j = 0; j < kMaxSinks; ++j)
      if (j < a.S) { red[wave][1 + j] = ee[j]; red[wave][1 + kMaxSinks + j] = he[j]; }
  }
  __syncthreads();
  if (tid == 0) {
    const double h2 = ((red[0][0] + red[1][0]) + red[2][0]) + red[3][0];
    int best = -1;
    double best_alpha = 0.0;
    for (int j = 0; j < a.S; ++j) {
      const double e2 = ((red[0][1 + j] + red[1][1 + j]) + red[2][1 + j]) + red[3][1 + j];
      const double he2 = ((red[0][1 + kMaxSinks + j] + red[1][1 + kMaxSinks + j]) +
                          red[2][1 + kMaxSinks + j]) + red[3][1 + kMaxSinks + j];
      const double al = (h2 == 0.0 || e2 == 0.0) ? 0.0 : he2 / (sqrt(h2) * sqrt(e2));
      if (best < 0 || al < best_alpha) { best = j; best_alpha = al; }
    }
    const int d = best_alpha < a.tau ? best : -1;
    a.decision[0] = d;
    a.alpha[0] = best_alpha;
    dec = d;
  }
  __syncthreads();
  if (dec >= 0)
    for (int i = tid; i < a.D; i += 256) a.embeds[(int64_t)dec * a.D + i] = a.h[i];
}

hipError_t launch_sink_decide(const SinkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sink_decide_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- motion: d_t = sqrt(sum (x_t - x_{t-1})^2 / n), fp64 ----------------------------------
// [NEWS] algorithm item 2 / [WT] motion-aware noise scheduler: the distance between consecutive
// latent frames.  Pass 1: each block sums one 16384-element part of one frame pair; pass 2 adds
// the parts of a frame in order - a fixed reduction order, so results are run-to-run identical.
constexpr int kMotionChunk = 16384;

int motion_parts(int64_t elems) { return (int)((elems + kMotionChunk - 1) / kMotionChunk); }

template <bool VEC4>
__global__ __launch_bounds__(256) void motion_partial_kernel(const float* x, int64_t n,
                                                             double* partials, int parts) {
  __shared__ double red[4];
  const int t = blockIdx.y + 1, p = blockIdx.x;
  const float* cur = x + (int64_t)t * n;
  const float* prev = cur - n;
  const int64_t lo = (int64_t)p * kMotionChunk;
  const int64_t hi = lo + kMotionChunk < n ? lo + kMotionChunk : n;
  double acc = 0.0;
  if constexpr (VEC4) {
    for (int64_t i = lo + 4 * threadIdx.x; i < hi; i += 4 * 256) {
      const float4 a = *(const float4*)(cur + i), b = *(const float4*)(prev + i);
      const double d0 = (double)a.x - (double)b.x, d1 = (double)a.y - (double)b.y;
      const double d2 = (double)a.z - (double)b.z, d3 = (double)a.w - (double)b.w;
      acc = fma(d0, d0, acc);
      acc = fma(d1, d1, acc);
      acc = fma(d2, d2, acc);
      acc = fma(d3, d3, acc);
    }
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
      const double d = (double)cur[i] - (double)prev[i];
      acc = fma(d, d, acc);
    }
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0)
    partials[(int64_t)(t - 1) * parts + p] = ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ __launch_bounds__(256) void motion_final_kernel(const double* partials, int parts,
                                                           int F, int64_t n, double* dist) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= F) return;
  double s = 0.0;
  for (int p = 0; p < parts; ++p) s += partials[(int64_t)t * parts + p];
  dist[t] = sqrt(s / (double)n);
}

hipError_t launch_motion(const float* frames, int nframes, int64_t elems, double* dist,
                         double* partials, int parts, hipStream_t s) {
  const int F = nframes - 1;
  const bool vec4 = (elems % 4 == 0) && (((uintptr_t)frames & 15) == 0);
  if (vec4)
    hipLaunchKernelGGL(motion_partial_kernel<true>, dim3(parts, F), dim3(256), 0, s, frames, elems,
                       partials, parts);
  else
    hipLaunchKernelGGL(motion_partial_kernel<false>, dim3(parts, F), dim3(256), 0, s, frames,
                       elems, partials, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(motion_final_kernel, dim3((F + 255) / 256), dim3(256), 0, s, partials, parts,
                     F, elems, dist);
  return hipGetLastError();
}

}  // namespace sdv2
