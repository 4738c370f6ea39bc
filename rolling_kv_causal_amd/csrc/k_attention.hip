// Chunk attention over [sinks | window | own chunk] for gfx950.
//
// For every stream-batch element b and head: O = softmax(scale * Q_rot K^T) V over the keys of
// the present sink frames, the window frames and the element's own (staged) frame.  This is the
// attention of the causal DiT over the sink + rolling KV cache ([NEWS] method, algorithm item 1;
// [REPO] core components: ring-buffer KV cache with sliding-window attention); the walkthrough
// ([WT] SLO-aware batching scheduler) names FlashAttention as the exact tiled evaluation of it.
//
// Kernels here (the head_dim-128 bf16 and e4m3 cache kernel is in k_attention_w64.hip):
//  * attn_bf16_kernel, bf16 cache with head_dim 64 (split-KV, flash-style): workgroup = 8 waves
//    x 32 query rows of one (element, head), a 256-row query tile; the grid follows the work
//    plan (query tiles dealt to the XCDs in contiguous runs, so the workgroups sharing one
//    head's K/V run on one XCD and one L2; only an XCD's last round of tiles split).  K tile
//    [64 keys][d] and V^T tile [d][64 keys] (V is stored transposed in the cache) are staged
//    through LDS, double-buffered.  S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K as the A
//    operand from LDS, Q^T as the B operand held in registers); K rows sit in LDS with bits 2
//    and 3 of the key index swapped so that the S^T accumulator layout is already the B
//    operand layout of O^T += V^T P^T, and P never leaves registers.  Online softmax in base 2.
//  * combine_kernel: merges the split-KV partials (bf16 O/l of each split, fp32 m and l) by
//    log-sum-exp weights into the bf16 output.
//  * attn_f32_kernel, fp32 cache: a plain per-query-row kernel in fp32 (no reduced-precision
//    matrix instructions).
#include "common.h"
#include "attn_tiles.h"

#include <math.h>

namespace sdv2 {

// Ping-pong schedule.  A workgroup is 8 waves = 2 groups of 4 (wave w runs on SIMD w % 4, so
// every SIMD holds one wave of each group); every wave owns 32 query rows, so the 256 rows of
// the workgroup share each K/V tile staged in LDS.  Per tile k a wave runs an MFMA phase
// M(k) = {O^T += V^T(k-1) P^T(k-1); S^T(k) = K(k) Q^T} and a VALU phase V(k) = {row max,
// exponentials, row sums of S(k) -> P(k)}.  Group B runs half a tile behind group A and
// workgroup barriers separate the phases, so while one wave of a SIMD issues MFMAs the other
// issues the softmax: phase 2m is {A: M(m), B: V(m-1)}, phase 2m+1 is {A: V(m), B: M(m)}.
// LDS rings of two K and two V^T tiles: K(m+1) and V(m) stream in during phases 2m and 2m+1
// (direct global->LDS loads issued by all waves at the start of phase 2m, awaited before the
// barrier that ends phase 2m+1), into slots whose previous tiles were last read in phase 2m-1.
// bf16 cache.  The 64-row kernel (k_attention_w64.hip) serves head_dim 128; this kernel serves
// head_dim 64.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const AttnArgs a) {
  constexpr int EB = 2;                       // bytes per cache element in HBM
  constexpr int KD = D / 16;                  // 16-wide k steps over d (QK)
  constexpr int DB = D / 32;                  // 32-row d blocks of O^T (PV)
  constexpr int KRB = D * 2;                  // bytes per K row in LDS (bf16)
  constexpr int VRB = kTileKeys * 2;          // bytes per V^T row of a tile in LDS (bf16)
  constexpr int K_BYTES = kTileKeys * KRB;
  constexpr int V_BYTES = D * VRB;
  constexpr int KG_BYTES = kTileKeys * D * EB;   // bytes of a K (V^T) tile in HBM
  constexpr int NW = 8;                       // waves per workgroup
  constexpr int KLD = KG_BYTES / 1024 / NW;   // 1 KB wave loads per wave per K tile
  constexpr int VLD = KLD;
  static_assert(KLD >= 1 && (D == 64 || D == 128), "head_dim 64 or 128");
  __shared__ __attribute__((aligned(1024))) char lds[2 * K_BYTES + 2 * V_BYTES];
  char* const ldsK = lds;
  char* const ldsV = lds + 2 * K_BYTES;
  typedef __attribute__((address_space(3))) void lds_void;

  WorkItem wi;
  if (!plan_item(a.plan, a.qtiles, a.nbatch, blockIdx.x, wi)) return;   // past its XCD's share
  const int qtile = wi.qtile, elem = wi.elem, head = wi.head, split = wi.split, nsplit = wi.nsplit;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                  // 0 = group A, 1 = group B
  const int g = lane >> 5, r = lane & 31;
  const int R = a.T * a.N;                    // query rows per element (T frames of N tokens)
  const int qrow = qtile * kQTile + wave * 32 + r;
  const bool qvalid = qrow < R;
  const int tq = qrow / a.N;                  // the row's frame within the chunk
  const int tq_wave = (qtile * kQTile + wave * 32) / a.N;   // lowest frame of the wave's rows

  // Q^T operand: lane (g, r) holds Q[row r][kd*16 + 8g .. +7] for every 16-wide k step.
  bf16x8 qf[KD];
  {
    const uint16_t* qp = (const uint16_t*)a.q +
                         ((int64_t)(elem * R + (qvalid ? qrow : 0)) * a.H + head) * D + g * 8;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const uint4 v = qvalid ? *(const uint4*)(qp + kd * 16) : make_uint4(0, 0, 0, 0);
      qf[kd] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Block-causal chunk: the walk [shared frames..., own frames 0..T-1] ends with the last own
  // frame a row of this query tile sees; the host keeps nsplit <= (nshared + 1) tiles per frame,
  // so every split has a tile.
  const int tq_hi = min(a.T - 1, (qtile * kQTile + kQTile - 1) / a.N);
  const int tiles_q = (a.nshared + tq_hi + 1) * a.tiles_per_frame;
  const int t_begin = (int)((int64_t)split * tiles_q / nsplit);
  const int t_end = (int)((int64_t)(split + 1) * tiles_q / nsplit);
  const int ntiles = t_end - t_begin;         // >= 1
  const int last = ntiles - 1;
  const char* kvb = (const char*)a.kv;
  const int64_t head_off = (int64_t)head * a.head_stride;
  // Slot of frame f in lane f (shared frames, then the T own frames; the host keeps
  // S + W + T <= 64), read back with readlane: the tile walk issues no scalar memory load,
  // whose wait would also drain the LDS queue.
  const int own_i = min(max(lane - a.nshared, 0), a.T - 1);
  const int slot_lane = lane < a.nshared ? a.slots[lane] : a.own_slot[elem * a.T + own_i];
  const char* const kblk = kvb + (a.k_layer_off + head_off) * EB;
  const char* const vblk = kvb + (a.v_layer_off + head_off) * EB;
  const int64_t slot_bytes = a.slot_stride * EB;
  auto frame_at = [&](TileCursor& c) {
    const int slot = __builtin_amdgcn_readlane(slot_lane, c.f & 63);
    c.kp = kblk + slot * slot_bytes + (int64_t)c.k * (kTileKeys * D * EB);
    c.vp = vblk + slot * slot_bytes + c.k * (kTileKeys * EB);
  };
  auto cursor_at = [&](int tile) -> TileCursor {
    TileCursor c;
    c.f = tile / a.tiles_per_frame;
    c.k = tile - c.f * a.tiles_per_frame;
    frame_at(c);
    return c;
  };
  auto advance = [&](TileCursor& c) {
    if (++c.k == a.tiles_per_frame) {
      c.k = 0;
      ++c.f;
      frame_at(c);
    } else {
      c.kp += kTileKeys * D * EB;
      c.vp += kTileKeys * EB;
    }
  };

  // Per-lane byte offsets of the tile fills (loop invariant): LDS row R of a K tile holds key
  // perm_key(R), its chunks placed by lds_chunk.
  uint32_t koff[KLD], voff[VLD];
#pragma unroll
  for (int i = 0; i < KLD; ++i) {
    int R, c;
    lds_chunk_inv<KRB>((wave * KLD + i) * 64 + lane, R, c);
    koff[i] = (uint32_t)(perm_key(R) * D * EB + c * 16);
  }
#pragma unroll
  for (int i = 0; i < VLD; ++i) {
    int R, c;
    lds_chunk_inv<VRB>((wave * VLD + i) * 64 + lane, R, c);
    voff[i] = (uint32_t)(R * a.Npad * EB + c * 16);
  }
  char* const kdst = ldsK;
  char* const vdst = ldsV;
  constexpr int KDST = K_BYTES, VDST = V_BYTES;   // per ring slot
  auto fill_k = [&](const TileCursor& c, int buf) {
    const char* src = c.kp;
#pragma unroll
    for (int i = 0; i < KLD; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + koff[i]),
                                       (lds_void*)(kdst + buf * KDST + (wave * KLD + i) * 1024), 16, 0, 0);
  };
  auto fill_v = [&](const TileCursor& c, int buf) {
    const char* src = c.vp;
#pragma unroll
    for (int i = 0; i < VLD; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + voff[i]),
                                       (lds_void*)(vdst + buf * VDST + (wave * VLD + i) * 1024), 16, 0, 0);
  };
  // Per-lane LDS read offsets (loop invariant): one 16-byte chunk per fragment.
  int kro[KD], vro[4];
#pragma unroll
  for (int kd = 0; kd < KD; ++kd) kro[kd] = lds_chunk<KRB>(r, 2 * kd + g);   // + 32 rows for kb = 1
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) vro[ch] = lds_chunk<VRB>(r, 2 * ch + g);   // + 32 rows per d block

  const float sl = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  f32x16 s0, s1;                              // S^T of the current tile: keys [0,32), [32,64)
  bf16x8 pb00 = {}, pb01 = {}, pb10 = {}, pb11 = {};   // P^T operands of the previous tile

  // MFMA phase of tile k: 16 PV fragments (d block t/4, key step t%4) then 16 QK fragments
  // (k step u/2, key block u%2), one MFMA each.  Fragment reads run kAhead fragments ahead of
  // their MFMA, and sched_group_barrier fixes the interleave (one MFMA, one LDS read), so each
  // MFMA waits only for its own operand instead of the whole LDS queue.
  constexpr int NPV = DB * 4, NQK = KD * 2, NF = NPV + NQK, kAhead = 8;
#define SDV2_FRAG(t_)                                                                          \
  ((t_) < NPV ? *(const bf16x8*)(vt + ((t_) / 4) * 32 * VRB + vro[(t_) % 4])                   \
              : *(const bf16x8*)(kt + (((t_) - NPV) % 2) * 32 * KRB + kro[((t_) - NPV) / 2]))
#define SDV2_FRAG_MFMA(t_, f_)                                                                 \
  do {                                                                                         \
    if ((t_) < NPV) {                                                                          \
      const bf16x8 pb_ = ((t_) % 4 == 0) ? pb00 : ((t_) % 4 == 1) ? pb01 : ((t_) % 4 == 2) ? pb10 : pb11; \
      o[(t_) / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f_, pb_, o[(t_) / 4], 0, 0, 0);    \
    } else if ((((t_) - NPV) % 2) == 0) {                                                      \
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f_, qf[((t_) - NPV) / 2],                   \
                                                   (t_) - NPV < 2 ? f32x16{} : s0, 0, 0, 0);   \
    } else {                                                                                   \
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f_, qf[((t_) - NPV) / 2],                   \
                                                   (t_) - NPV < 2 ? f32x16{} : s1, 0, 0, 0);   \
    }                                                                                          \
  } while (0)
  // fragments t in [T0, T1) of tile k's phase.  Every phase runs all of them, which keeps a
  // single code path (and the accumulators in place): M(0) adds V^T P^T with P = 0 over a
  // zeroed V^T slot, and the S^T of M(n) is never used.
#define SDV2_MFMA_RUN(k_, T0, T1)                                                              \
  do {                                                                                         \
    const char* vt = ldsV + (((k_) - 1) & 1) * V_BYTES;                                        \
    const char* kt = ldsK + ((k_) & 1) * K_BYTES;                                              \
    (void)vt; (void)kt;                                                                        \
    bf16x8 fr_[NF];                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    _Pragma("unroll") for (int t_ = T0; t_ < T0 + kAhead && t_ < T1; ++t_) fr_[t_] = SDV2_FRAG(t_); \
    _Pragma("unroll") for (int t_ = T0; t_ < T1; ++t_) {                                       \
      SDV2_FRAG_MFMA(t_, fr_[t_]);                                                             \
      if (t_ + kAhead < T1) fr_[t_ + kAhead] = SDV2_FRAG(t_ + kAhead);                         \
    }                                                                                          \
    __builtin_amdgcn_sched_group_barrier(0x100, (T1 - T0) < kAhead ? (T1 - T0) : kAhead, 0);   \
    _Pragma("unroll") for (int t_ = T0; t_ < T1; ++t_) {                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                       \
      if (t_ + kAhead < T1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  } while (0)
#define SDV2_MFMA_PHASE(k_) SDV2_MFMA_RUN(k_, 0, NF)

  // VALU phase of the current tile: masked row max, lazy rescale, exponentials -> P^T, row
  // sums.  lane (g, r), accumulator v holds key 16*(v/8) + 8g + v%8 (+32 for s1) of query r.
  auto valu_phase = [&](int nvalid, int tk) {
    if (tk > tq_wave && tk > tq) {            // own frame tk is after this row's frame
#pragma unroll
      for (int v = 0; v < 16; ++v) s0[v] = s1[v] = -INFINITY;
    }
    if (nvalid < kTileKeys) {                 // ragged last tile of a frame
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 16 * (v >> 3) + 8 * g + (v & 7);
        if (key >= nvalid) s0[v] = -INFINITY;
        if (key + 32 >= nvalid) s1[v] = -INFINITY;
      }
    }
    // Exponentials at the running max m_run.  The row max is only taken (and m_run moved,
    // with O and l rescaled) when a lane's sum of exponentials leaves [0, 2^kLazy]: on the
    // first tile (m_run = -inf gives inf or NaN) or once scores pass m_run by a margin.  So
    // exponentials stay <= 2^kLazy and O/l is unchanged (both use m_run).  Row sums are taken
    // from the rounded bf16 P that the PV product uses.
    uint32_t pw0[8], pw1[8];
    float ps;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#define SDV2_EXPS(M_)                                                                          \
    do {                                                                                       \
      _Pragma("unroll") for (int v = 0; v < 16; v += 2) {                                      \
        pw0[v / 2] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s0[v], sl, -(M_))),               \
                                 __builtin_amdgcn_exp2f(fmaf(s0[v + 1], sl, -(M_))));          \
        pw1[v / 2] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s1[v], sl, -(M_))),               \
                                 __builtin_amdgcn_exp2f(fmaf(s1[v + 1], sl, -(M_))));          \
      }                                                                                        \
      float sa = 0.f, sb = 0.f;                                                                \
      _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                          \
        sa = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw0[j]), ones, sa, false); \
        sb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw1[j]), ones, sb, false); \
      }                                                                                        \
      ps = sa + sb;                                                                            \
    } while (0)
    SDV2_EXPS(m_run);
    if (__builtin_amdgcn_ballot_w64(!(ps <= kLazyMass))) {   // wave-uniform, rare
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // a row that has seen only masked keys keeps m_run = -inf and gets P = 0
      const float m_new = fmaxf(m_run, mx * sl);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
      SDV2_EXPS(m_run == -INFINITY ? 0.f : m_run);
    }
#undef SDV2_EXPS
    l_run += ps;
    pb00 = __builtin_bit_cast(bf16x8, make_uint4(pw0[0], pw0[1], pw0[2], pw0[3]));
    pb01 = __builtin_bit_cast(bf16x8, make_uint4(pw0[4], pw0[5], pw0[6], pw0[7]));
    pb10 = __builtin_bit_cast(bf16x8, make_uint4(pw1[0], pw1[1], pw1[2], pw1[3]));
    pb11 = __builtin_bit_cast(bf16x8, make_uint4(pw1[4], pw1[5], pw1[6], pw1[7]));
  };

  // Loads of "phase pair" m: K(m+1) and V(m) into their ring slots (every wave its share).
  TileCursor kc = cursor_at(t_begin);         // K tile of the next loads
  TileCursor vc = kc;                         // V tile of the next loads
  TileCursor sc = kc;                         // tile of this wave's next VALU phase
  auto loads = [&](int m) {
    if (m + 1 <= last) {
      advance(kc);
      fill_k(kc, (m + 1) & 1);
    }
    if (m <= last) {
      fill_v(vc, m & 1);
      if (m + 1 <= last) advance(vc);
    }
  };
  // wait for this wave's loads (before the barrier that publishes them)
  auto loads_in = [&]() { __builtin_amdgcn_s_waitcnt(kWaitVm0); };

  // prologue: K(0) resident before phase 0; group B idles through phase 0 (it issues its
  // share of the phase-0 loads there)
  fill_k(kc, 0);
  // V^T slot 1 is read by M(0) (with P = 0) before V(1) arrives: make it finite
#pragma unroll
  for (int i = 0; i < V_BYTES / (512 * 16); ++i)
    reinterpret_cast<uint4*>(ldsV + V_BYTES)[tid + 512 * i] = make_uint4(0u, 0u, 0u, 0u);
  loads_in();
  __syncthreads();
  if (grp == 1) {
    loads(0);
    __syncthreads();
  }
  // Each wave runs M(0), V(0), M(1), ..., V(n-1), M(n).  Loads of pair m are issued at the
  // start of even phase 2m (A: M(m); B: V(m-1)) and awaited at the end of odd phase 2m+1
  // (A: V(m); B: M(m)), so every wave passes the same barriers with its loads complete.
  for (int k = 0; k <= ntiles; ++k) {
    if (grp == 0) loads(k);
    __builtin_amdgcn_s_setprio(2);            // MFMA phase first in issue arbitration
    SDV2_MFMA_PHASE(k);
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) loads_in();
    __syncthreads();
    if (k == ntiles && grp == 1) break;       // B's last phase was M(n)
    if (grp == 1) loads(k + 1);
    if (k <= last) {
      valu_phase(a.N - sc.k * kTileKeys, sc.f - a.nshared);
      if (k < last) advance(sc);
    }
    if (grp == 0) loads_in();
    __syncthreads();
  }
#undef SDV2_FRAG
#undef SDV2_FRAG_MFMA
#undef SDV2_MFMA_RUN
#undef SDV2_MFMA_PHASE

  // lane (g, r), accumulator v of o[i] holds O^T[d = 32i + 8(v/4) + 4g + v%4][query r]
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // 0: no visible key in this split
  if (nsplit == 1) {
    uint16_t* op = (uint16_t*)a.out + ((int64_t)(elem * R + qrow) * a.H + head) * D + 4 * g;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        uint2 w2;
        w2.x = pack_bf16x2(o[i][4 * a4 + 0] * inv, o[i][4 * a4 + 1] * inv);
        w2.y = pack_bf16x2(o[i][4 * a4 + 2] * inv, o[i][4 * a4 + 3] * inv);
        *(uint2*)(op + 32 * i + 8 * a4) = w2;
      }
  } else {
    const int64_t prow = ((int64_t)split * a.plan.tail_first[kNumXcd] + wi.tail) * kQTile + qrow - qtile * kQTile;
    uint16_t* po = a.part_o + prow * D + 4 * g;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        uint2 w2;
        w2.x = pack_bf16x2(o[i][4 * a4] * inv, o[i][4 * a4 + 1] * inv);
        w2.y = pack_bf16x2(o[i][4 * a4 + 2] * inv, o[i][4 * a4 + 3] * inv);
        *(uint2*)(po + 32 * i + 8 * a4) = w2;
      }
    if (g == 0) a.part_ml[prow] = make_float2(m_run, l_tot);
  }
}

// Merge split-KV partials: O = sum_s w_s O_s / sum_s w_s, w_s = l_s 2^(m_s - max m).  The
// partial O_s (already divided by l_s) are bf16: the merged row is rounded to bf16 anyway, and
// half the bytes halve the partial traffic of the attention epilogue and of this kernel.  Rows
// are those of the plan's tail items (row r of tail item t: query tile row r).
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  constexpr int TPR = D / 8;                        // threads per output row, 8 values each
  const int ntail = a.plan.tail_first[kNumXcd], nsplit = a.plan.nsplit;
  const int64_t rows = (int64_t)ntail * kQTile;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int t = (int)(row / kQTile), rq = (int)(row % kQTile);
  int head, elem, qtile;
  plan_tail(a.plan, a.qtiles, a.nbatch, t, head, elem, qtile);
  const int n = qtile * kQTile + rq;                // query row of the element
  if (n >= a.N) return;
  const int d0 = (threadIdx.x % TPR) * 8;
  // Splits in groups of eight: every load of a group is issued before any arithmetic, so the
  // kernel pays one memory round trip per group (one in all for up to eight splits); a later
  // group with a larger maximum rescales what the earlier ones summed.
  constexpr int G = 8;
  float M = -INFINITY, W = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += G) {
    float2 ml[G];
    uint4 p[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (s0 + j < nsplit) {
        ml[j] = a.part_ml[(s0 + j) * rows + row];
        p[j] = *(const uint4*)(a.part_o + ((s0 + j) * rows + row) * D + d0);
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (s0 + j < nsplit) Mn = fmaxf(Mn, ml[j].x);
    if (M != Mn && M != -INFINITY) {
      const float r = __builtin_amdgcn_exp2f(M - Mn);
      W *= r;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= r;
    }
    M = Mn;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (s0 + j < nsplit) {
        const float wgt = ml[j].y * __builtin_amdgcn_exp2f(ml[j].x - M);
        const uint32_t pw[4] = {p[j].x, p[j].y, p[j].z, p[j].w};
        W += wgt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wgt, __uint_as_float(pw[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wgt, __uint_as_float(pw[i] & 0xffff0000u), acc[2 * i + 1]);
        }
      }
    }
  }
  const float inv = 1.f / W;
  uint16_t* op = (uint16_t*)a.out + ((int64_t)(elem * a.N + n) * a.H + head) * D + d0;
  uint4 w4;
  w4.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w4.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  w4.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  w4.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *(uint4*)op = w4;
}

// fp32: one query row per lane, 32-key tiles through LDS, online softmax per row.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnArgs a) {
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const int R = a.T * a.N;                    // query rows per element
  const int qtiles = (R + 63) / 64;
  const int qtile = blockIdx.x % qtiles;
  const int head = (blockIdx.x / qtiles) % a.H;
  const int elem = blockIdx.x / (qtiles * a.H);
  const int lane = threadIdx.x;
  const int n = qtile * 64 + lane;
  const bool valid = n < R;
  const int tq = n / a.N;                     // the row's frame within the chunk
  const int tq_hi = min(a.T - 1, (qtile * 64 + 63) / a.N);

  float q[D], o[D];
  const float* qp = (const float*)a.q + ((int64_t)(elem * R + (valid ? n : 0)) * a.H + head) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* kvb = (const float*)a.kv;
  for (int f = 0; f <= a.nshared + tq_hi; ++f) {   // block-causal inside the chunk
    const int slot = f < a.nshared ? a.slots[f] : a.own_slot[elem * a.T + f - a.nshared];
    const bool seen = f - a.nshared <= tq;
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
        s[j] = (j < nv && seen) ? acc * a.scale : -INFINITY;
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
  float* op = (float*)a.out + ((int64_t)(elem * R + n) * a.H + head) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
}

// bf16 or e4m3 cache with head_dim 128: the 64-row kernel (k_attention_w64.hip); bf16 with
// head_dim 64: the 32-row ping-pong kernel above; fp32: the per-row kernel.
hipError_t launch_attention(const AttnArgs& a, int head_dim, int kv, hipStream_t s) {
  if (kv != kKvF32 && head_dim == 128) return launch_attention_w64(a, kv, s);
  if (kv == kKvBF16 && head_dim == 64) {
    const int grid = kNumXcd * a.plan.wg_per_xcd;
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(512), 0, s, a);
  } else if (kv == kKvF32) {
    const int grid = a.nbatch * a.H * ((a.T * a.N + 63) / 64);
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;             // e4m3 needs head_dim 128 (refused at validation)
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)a.plan.tail_first[kNumXcd] * kQTile;
  const int rows_per_block = 256 / (head_dim / 8);
  const int grid = (int)((rows + rows_per_block - 1) / rows_per_block);
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdv2
