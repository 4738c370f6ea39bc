// Cache maintenance kernels: the sink-replacement copy, the RoPE rebase, the fused chunk
// statistics (motion distance and sink similarity) with the sink decision, and the batched
// motion reduction.
#include "common.h"

#include <math.h>

namespace sdv2 {

// ---- slot copy: K and V of one slot into another, every layer --------------------------------
// Sink replacement ([WT] adaptive sink and RoPE refresh): the committed frame's K and V (in its
// ring slot) enter the chosen sink slot, read from the device decision; nothing is copied when
// the decision is -1.  (The commit itself moves no data: the append wrote element 0's frames to
// the ring slots they keep.)
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
// Work item = one 16-byte chunk of a key row among the first a.cpr chunks, which hold every
// temporal pair and fill whole 128-byte lines (the other dims are written back unchanged);
// consecutive threads take consecutive chunks of a row, then the next row; each thread has
// four chunks in flight; stores carry the non-temporal hint.
template <int KV>
__device__ __forceinline__ void rebase_chunk(uint4& w, int c, const float2* cs, int pt) {
  if constexpr (KV == kKvBF16) {
    uint32_t* u = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = 4 * c + j;
      if (p < pt) {
        const float x = bf16_bits_to_f32(u[j] & 0xffffu), y = bf16_bits_to_f32(u[j] >> 16);
        u[j] = pack_bf16x2(x * cs[p].x - y * cs[p].y, x * cs[p].y + y * cs[p].x);
      }
    }
  } else if constexpr (KV == kKvF32) {
    float* f = reinterpret_cast<float*>(&w);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = 2 * c + j;
      if (p < pt) {
        const float x = f[2 * j], y = f[2 * j + 1];
        f[2 * j] = x * cs[p].x - y * cs[p].y;
        f[2 * j + 1] = x * cs[p].y + y * cs[p].x;
      }
    }
  } else {
    // e4m3: the byte pair at positions 16c + 2k holds dims fp8_pos(16c + 2k) and the next one
    // (fp8_pos keeps bits 0-2), i.e. pair fp8_pos(16c + 2k) / 2
    uint32_t* u = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int p = fp8_pos(16 * c + 2 * k) >> 1;
      if (p < pt) {
        const uint32_t word = u[k >> 1];
        const int half = (k & 1) * 16;
        const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)(word >> half), false);
        const uint32_t r = pack_fp8x4(v.x * cs[p].x - v.y * cs[p].y, v.x * cs[p].y + v.y * cs[p].x, 0.f, 0.f) & 0xffffu;
        u[k >> 1] = (word & ~(0xffffu << half)) | (r << half);
      }
    }
  }
}

template <int KV>
__global__ __launch_bounds__(256) void rebase_kernel(const RebaseArgs a, int D) {
  constexpr int EB = KV == kKvF32 ? 4 : KV == kKvBF16 ? 2 : 1;
  constexpr int U = 4;                             // chunks in flight per thread
  __shared__ float2 cs[kMaxTPairs];
  if ((int)threadIdx.x < a.pt) cs[threadIdx.x] = a.cs[threadIdx.x];
  __syncthreads();
  const int si = blockIdx.y / a.L, layer = blockIdx.y % a.L;
  char* const base = (char*)a.kv + (layer * a.layer_stride + (int64_t)a.slots[si] * a.slot_stride) * EB;
  const int64_t nwork = (int64_t)a.H * a.N * a.cpr;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i0 < nwork; i0 += (int64_t)gridDim.x * 256 * U) {
    uint4 w[U];
    uint4* ptr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * 256;
      ptr[u] = nullptr;
      if (i < nwork) {
        const int c = (int)(i % a.cpr);
        const int64_t row = i / a.cpr;
        const int n = (int)(row % a.N), h = (int)(row / a.N);
        ptr[u] = (uint4*)(base + ((int64_t)h * a.head_stride + (int64_t)n * D) * EB + 16 * c);
        w[u] = *ptr[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ptr[u]) {
        rebase_chunk<KV>(w[u], (int)((i0 + u * 256) % a.cpr), cs, a.pt);
        store16_nt(ptr[u], w[u]);
      }
  }
}

hipError_t launch_rebase(const RebaseArgs& a, int head_dim, int kv, hipStream_t s) {
  const int64_t nwork = (int64_t)a.H * a.N * a.cpr;
  int gx = (int)((nwork + 256 * 4 - 1) / (256 * 4));
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

// ---- fused chunk statistics, pass 1 -----------------------------------------------------------
// Per block: sum (cur - prev)^2 over latent elements [b*lpb, (b+1)*lpb) and h.h, e_j.e_j, h.e_j
// over embedding elements [b*epb, (b+1)*epb), all in fp64, reduced in a fixed order (lane
// strides, a butterfly inside each wave, then the four waves in order).
template <bool VEC4>
__global__ __launch_bounds__(256) void chunk_stats_kernel(const StatsArgs a) {
  __shared__ double red[4][kStatsQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
  double mo = 0.0, hh = 0.0, ee[kMaxSinks], he[kMaxSinks];
#pragma unroll
  for (int j = 0; j < kMaxSinks; ++j) { ee[j] = 0.0; he[j] = 0.0; }
  if (a.n_lat > 0) {
    const int64_t lo = (int64_t)b * a.lat_per_block;
    const int64_t hi = lo + a.lat_per_block < a.n_lat ? lo + a.lat_per_block : a.n_lat;
    if constexpr (VEC4) {
#pragma unroll 2
      for (int64_t i = lo + 4 * tid; i < hi; i += 4 * 256) {
        const float4 x = *(const float4*)(a.cur + i), y = *(const float4*)(a.prev + i);
        const double d0 = (double)x.x - (double)y.x, d1 = (double)x.y - (double)y.y;
        const double d2 = (double)x.z - (double)y.z, d3 = (double)x.w - (double)y.w;
        mo = fma(d0, d0, mo);
        mo = fma(d1, d1, mo);
        mo = fma(d2, d2, mo);
        mo = fma(d3, d3, mo);
      }
    } else {
      for (int64_t i = lo + tid; i < hi; i += 256) {
        const double d = (double)a.cur[i] - (double)a.prev[i];
        mo = fma(d, d, mo);
      }
    }
  }
  if (a.D > 0) {
    const int lo = b * a.emb_per_block;
    const int hi = lo + a.emb_per_block < a.D ? lo + a.emb_per_block : a.D;
#pragma unroll 4
    for (int i = lo + tid; i < hi; i += 256) {
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
  }
  mo = wave_sum(mo);
  hh = wave_sum(hh);
#pragma unroll
  for (int j = 0; j < kMaxSinks; ++j)
    if (j < a.S) { ee[j] = wave_sum(ee[j]); he[j] = wave_sum(he[j]); }
  if (lane == 0) {
    red[wave][0] = mo;
    red[wave][1] = hh;
#pragma unroll
    for (int j = 0; j < kMaxSinks; ++j)
      if (j < a.S) { red[wave][2 + j] = ee[j]; red[wave][2 + kMaxSinks + j] = he[j]; }
  }
  __syncthreads();
  const int q = tid;   // quantity: 0 motion, 1 h.h, 2 + j e_j.e_j, 2 + kMaxSinks + j h.e_j
  const bool used = q < 2 || (q >= 2 && q < 2 + a.S) || (q >= 2 + kMaxSinks && q < 2 + kMaxSinks + a.S);
  if (q < kStatsQ && used)
    a.part[(int64_t)b * kStatsQ + q] = ((red[0][q] + red[1][q]) + red[2][q]) + red[3][q];
}

hipError_t launch_chunk_stats(const StatsArgs& a, int blocks, hipStream_t s) {
  const bool vec4 = a.n_lat > 0 && (a.n_lat % 4 == 0) && (((uintptr_t)a.prev | (uintptr_t)a.cur) & 15) == 0;
  if (vec4)
    hipLaunchKernelGGL(chunk_stats_kernel<true>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(chunk_stats_kernel<false>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- fused chunk statistics, pass 2: statistics, sink decision, embedding stores ---------------
// [WT] adaptive sink and RoPE refresh: cosine similarity of the new chunk embedding against each
// sink's embedding; the least similar sink (lowest index on ties; similarity 0 when a norm is 0)
// is replaced when its similarity is below tau.  A sink stored by this call (a chunk frame below
// S) has h as its embedding.  One block.
__global__ __launch_bounds__(256) void sink_decide_kernel(const SinkArgs a) {
  __shared__ double tot[kStatsQ];
  __shared__ int dec;
  const int tid = threadIdx.x;
  if (tid < kStatsQ) {
    double sum = 0.0;
    for (int b = 0; b < a.blocks; ++b) sum += a.part[(int64_t)b * kStatsQ + tid];
    tot[tid] = sum;
  }
  __syncthreads();
  if (tid == 0) {
    const double nan = __builtin_nan("");
    const double h2 = tot[1];
    int best = -1;
    double best_alpha = 1.0;
    if (a.decide) {
      for (int j = 0; j < a.S; ++j) {
        const bool stored = j >= a.store_lo && j < a.store_hi;
        const double e2 = stored ? h2 : tot[2 + j], he2 = stored ? h2 : tot[2 + kMaxSinks + j];
        const double al = (h2 == 0.0 || e2 == 0.0) ? 0.0 : he2 / (sqrt(h2) * sqrt(e2));
        if (best < 0 || al < best_alpha) { best = j; best_alpha = al; }
      }
    }
    const int d = (a.decide && best_alpha < a.tau) ? best : -1;
    a.decision[0] = d;
    a.alpha[0] = best_alpha;
    dec = d;
    if (a.stats) {
      a.stats[0] = a.n_lat > 0 ? tot[0] : nan;
      a.stats[1] = a.n_lat > 0 ? sqrt(tot[0] / (double)a.n_lat) : nan;
      a.stats[2] = a.D > 0 ? h2 : nan;
      for (int j = 0; j < a.S; ++j) {
        const bool stored = j >= a.store_lo && j < a.store_hi;
        a.stats[3 + j] = a.D > 0 ? (stored ? h2 : tot[2 + j]) : nan;
        a.stats[3 + a.S + j] = a.D > 0 ? (stored ? h2 : tot[2 + kMaxSinks + j]) : nan;
      }
      a.stats[3 + 2 * a.S] = a.decide ? best_alpha : nan;
    }
  }
  __syncthreads();
  if (a.D > 0 && (a.store_hi > a.store_lo || dec >= 0))
    for (int i = tid; i < a.D; i += 256) {
      const float x = a.h[i];
      for (int j = a.store_lo; j < a.store_hi; ++j) a.embeds[(int64_t)j * a.D + i] = x;
      if (dec >= 0) a.embeds[(int64_t)dec * a.D + i] = x;
    }
}

hipError_t launch_sink_decide(const SinkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sink_decide_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- motion: d_t = sqrt(sum (x_t - x_{t-1})^2 / n), fp64 ----------------------------------
// [NEWS] algorithm item 2 / [WT] motion-aware noise scheduler: the distance between consecutive
// latent frames.  Pass 1: a block walks kMotionRun consecutive frame pairs over one part of
// kMotionChunk elements, so every frame of the run is read once; each thread keeps the frames
// of the next kMotionDepth pairs in flight in a ring of registers.  The run is unrolled and
// branch-free, so every pair waits only for its own frame: tail elements read one fixed element
// in every frame (difference zero), frames past the run repeat its last frame, and each lane
// stores its wave's pair sum (lanes other than 0 into a slot of their own).  Per pair the sum of
// (x_t - x_{t-1})^2 is taken in fp64 (lane strides, a butterfly in each wave, the four waves in
// order), into partials[part][pair].  Pass 2 adds the parts of a frame in order.  A fixed
// reduction order: results are run-to-run identical.
constexpr int kMotionChunk = 4096;   // elements of a part: 16 per thread
constexpr int kMotionRun = 32;       // frame pairs per block
constexpr int kMotionDepth = 3;      // frames in flight per thread (with 4 blocks per CU)

int motion_parts(int64_t elems) { return (int)((elems + kMotionChunk - 1) / kMotionChunk); }

// One run of pairs over one part.  TAIL: the part reaches past the frame's end; an
// out-of-range load reads element 0 of the series in every frame, so its difference is zero.
template <bool VEC4, bool TAIL>
__device__ __forceinline__ void motion_run(const float* x, int64_t n, int t0, int pairs,
                                           int64_t lo, double* red) {
  constexpr int E = kMotionChunk / 256;            // elements per thread
  constexpr int L = VEC4 ? E / 4 : E;              // loads per frame
  // frame slots (frame t0 + i lives in slot i % NS); the scalar path, with 16 loads per frame,
  // keeps one frame in flight
  constexpr int NS = (VEC4 ? kMotionDepth : 1) + 1;
  const int last = t0 + pairs;                     // last frame of the run
  float f[NS][E];
  auto load = [&](int t, float* v) {
    const int64_t fb = (int64_t)(t < last ? t : last) * n + lo;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int r = VEC4 ? 4 * ((int)threadIdx.x + 256 * j) : (int)threadIdx.x + 256 * j;
      // (the multiplier form keeps the tail's choice arithmetic: no branch around the load)
      const float* ptr = TAIL ? x + (fb + r) * (int64_t)(lo + r < n) : x + fb + r;
      if constexpr (VEC4) {                        // n % 4 == 0 and 16-byte aligned frames
        const float4 w = *(const float4*)ptr;
        v[4 * j] = w.x; v[4 * j + 1] = w.y; v[4 * j + 2] = w.z; v[4 * j + 3] = w.w;
      } else {
        v[j] = *ptr;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NS; ++i) load(t0 + i, f[i]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < kMotionRun; ++k) {           // pair k: frames in slots k and k + 1 (mod NS)
    const float* prev = f[k % NS];
    const float* cur = f[(k + 1) % NS];
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const double df = (double)cur[j] - (double)prev[j];
      acc = fma(df, df, acc);
    }
    if (k + NS <= kMotionRun) load(t0 + k + NS, f[k % NS]);   // the slot's frame is done
    // the scheduler keeps each pair's arithmetic between the refills (else it computes as early
    // as possible and waits for every load right after it is issued)
    __builtin_amdgcn_sched_barrier(0);
    const double v = wave_sum(acc);
    red[lane == 0 && k < pairs ? wave * kMotionRun + k : 4 * kMotionRun + threadIdx.x] = v;
  }
}

template <bool VEC4>
__global__ __launch_bounds__(256, 4) void motion_partial_kernel(const float* x, int64_t n, int F,
                                                                double* partials, int parts) {
  // per-wave pair sums; every lane stores (the others into a slot of their own), so the store
  // is not a branch the compiler could hoist the next pairs' arithmetic over
  __shared__ double red[4 * kMotionRun + 256];
  const int p = blockIdx.x, t0 = blockIdx.y * kMotionRun;   // pairs (t0 + k, t0 + k + 1)
  const int pairs = F - t0 < kMotionRun ? F - t0 : kMotionRun;
  const int64_t lo = (int64_t)p * kMotionChunk;
  if (lo + kMotionChunk <= n) motion_run<VEC4, false>(x, n, t0, pairs, lo, red);
  else motion_run<VEC4, true>(x, n, t0, pairs, lo, red);
  __syncthreads();
  if ((int)threadIdx.x < pairs) {
    const double* r = red + threadIdx.x;
    partials[(int64_t)p * F + t0 + threadIdx.x] =
        ((r[0] + r[kMotionRun]) + r[2 * kMotionRun]) + r[3 * kMotionRun];
  }
}

// partials[p][t]: one thread per frame pair adds the parts in order, eight loads in flight.
__global__ __launch_bounds__(256) void motion_final_kernel(const double* partials, int parts,
                                                           int F, int64_t n, double* dist) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= F) return;
  double s = 0.0;
  int p = 0;
  for (; p + 8 <= parts; p += 8) {
    double v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = partials[(int64_t)(p + i) * F + t];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  for (; p < parts; ++p) s += partials[(int64_t)p * F + t];
  dist[t] = sqrt(s / (double)n);
}

hipError_t launch_motion(const float* frames, int nframes, int64_t elems, double* dist,
                         double* partials, int parts, hipStream_t s) {
  const int F = nframes - 1;
  const bool vec4 = (elems % 4 == 0) && (((uintptr_t)frames & 15) == 0);
  const dim3 grid(parts, (F + kMotionRun - 1) / kMotionRun);
  if (vec4)
    hipLaunchKernelGGL(motion_partial_kernel<true>, grid, dim3(256), 0, s, frames, elems, F, partials, parts);
  else
    hipLaunchKernelGGL(motion_partial_kernel<false>, grid, dim3(256), 0, s, frames, elems, F, partials, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(motion_final_kernel, dim3((F + 255) / 256), dim3(256), 0, s, partials, parts,
                     F, elems, dist);
  return hipGetLastError();
}

}  // namespace sdv2
