// Chunk attention, bf16 and e4m3 caches, head_dim 128: one wave per SIMD, 64 query rows per wave.
//
// Same operation and split-KV interface as attn_bf16_kernel ([NEWS] method, algorithm item 1;
// [REPO] core components; [WT] SLO-aware batching scheduler names FlashAttention as the exact
// tiled evaluation): O = softmax(scale * Q_rot K^T) V over [sinks | window | own chunk], the
// own chunk block-causal, one 256-row query tile of one (element, head) per workgroup.
//
// Why 64 rows per wave: with 32 rows every 1 KB K or V^T fragment read from LDS feeds one
// MFMA, and one wave cannot read LDS fast enough to keep the matrix core busy.  With 64 rows
// (two 32-row blocks qb) every fragment feeds two MFMAs.  The state then needs
//   O^T 128 + Q^T 64 (AGPRs) and S^T 64 + P^T 2 x 32 + fragments 48 (VGPRs),
// which fits one wave per SIMD only.  The softmax of tile t is interleaved with the MFMAs of
// the same wave (QK of its key block 1, P V of tile t-1), so the wave overlaps its own VALU and
// matrix work; scalar set-up and tile loads sit in the remaining issue slots.  That
// needs an instruction order and a register assignment the compiler does not produce, so the
// whole tile loop (tile walk, global->LDS loads, waits, barriers, the 64 MFMAs and 32 fragment
// reads of a tile, the softmax, masks and the rare rescale) is one generated asm program
// (attn_w64_asm.h, written by gen_attn_w64.py, which documents the register plan and the
// gfx950 hazard rules it keeps) over registers named by the asm operands.  The C++ around it
// loads Q^T, computes lane constants and the first loads, and writes the outputs.
//
// Per tile t (iteration t = 0..n-1, n tiles in the split):
//   QK(t): S^T = K(t) Q^T;  PV(t-1): O^T += V^T(t-1) P^T(t-1);  softmax(t): P^T(t) from S^T
// with P(-1) = 0 over a zeroed V^T slot, then a last P V-only step.  LDS rings of four K and
// four V^T tiles (tile t in slot t mod 4, so the generated loop has one copy per slot and
// every LDS address is a register plus an immediate): iteration t loads K(t+2) and V(t+1)
// into the slots of K(t-2) and V(t-3), which every wave has finished reading; a wave waits for
// its own loads (vmcnt) two iterations after issue, before that iteration's barrier.
//
// Softmax: base 2 with a lazy running maximum m per row.  Q is staged as stored (bf16) and the
// first QK MFMA of each chain accumulates onto a block holding -(m + 8) / c, c = scale *
// log2(e), so one fp32 product by c turns the MFMA result into the exponent: P = 2^(s c - m -
// 8), the factor 2^-8 cancelling between O and l.  A cache whose keys carry c (SK, e4m3) runs
// with c = 1 and a program without the product.  Only when some P word of a tile reaches 2 (a score
// 9 above m, a NaN or an infinity), or a row has no maximum yet, is the row maximum taken and
// O, l rescaled.  The row sums l are MFMAs over P with a selector operand.  Masks (ragged last
// tile of a frame, block-causal own frames) are applied to the packed P words by AND.
#include "common.h"
#include "attn_tiles.h"
#include "attn_w64_asm.h"

namespace sdv2 {

typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef int i32x32 __attribute__((ext_vector_type(32)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x12 __attribute__((ext_vector_type(12)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// s_waitcnt immediate: vmcnt(n), lgkmcnt and expcnt at their maxima
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// F8: e4m3 cache.  Each wave loads its 2 KB share of a K and of a V^T tile (e4m3) into a
// staging slot (two slots of 16 KB, by iteration parity), and the next iteration widens exactly
// those bytes to bf16 into the ring slots (exact conversion) in the gaps of its stream before the
// softmax; the rest of the loop is the bf16 one.  Its keys are stored times key_scale * log2(e) * 2^k
// and the queries are staged times 2^-k, so its program has no product per score either.
// SK: bf16 cache whose keys are stored times scale * log2(e): the scores already are the
// exponent (the host passes scale_log2 = 1) and the program has no product per score.
template <bool F8, bool SK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_w64_kernel(const AttnArgs a) {
  constexpr int D = 128, KRB = 256, VRB = 128, EB = F8 ? 1 : 2;   // EB: cache bytes per element
  constexpr int K_BYTES = kTileKeys * KRB, V_BYTES = D * VRB, NBUF = 4;
  constexpr int STAGE = F8 ? 2 * kTileKeys * D : 0;              // e4m3 K + V^T tile bytes
  constexpr int LD = K_BYTES * EB / 2 / 1024 / 4;                 // 1 KB loads per wave per tile (K; the same for V^T)
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * (K_BYTES + V_BYTES) + 2 * STAGE];
  char* const ldsS = lds + NBUF * (K_BYTES + V_BYTES);            // e4m3 staging slots
  char* const ldsK = lds;
  char* const ldsV = lds + NBUF * K_BYTES;
  typedef __attribute__((address_space(3))) void lds_void;

  WorkItem wi;
  if (!plan_item(a.plan, a.qtiles, a.nbatch, blockIdx.x, wi)) return;   // past its XCD's share
  const int qtile = wi.qtile, elem = wi.elem, head = wi.head, split = wi.split, nsplit = wi.nsplit;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r = lane & 31;
  const int R = a.T * a.N;                    // query rows per element
  const int wrow = qtile * kQTile + wave * 64;   // first row of the wave
  int row[2], tq[2];
  bool valid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    row[qb] = wrow + 32 * qb + r;
    valid[qb] = row[qb] < R;
    tq[qb] = row[qb] / a.N;
  }
  const int tq_wave = wrow / a.N;             // lowest frame of the wave's rows

  // Q^T operands: lane (g, r) holds Q[row][16 kd + 8g .. +7] as dwords 4kd..4kd+3 of q[qb],
  // the stored bf16 values unchanged (the softmax scale is applied to each score in fp32, or
  // carried by the keys; the e4m3 program scales them by a power of two below).
  i32x32 q0, q1;
  {
    const uint16_t* qb0 = (const uint16_t*)a.q + ((int64_t)(elem * R + (valid[0] ? row[0] : 0)) * a.H + head) * D + 8 * g;
    const uint16_t* qb1 = (const uint16_t*)a.q + ((int64_t)(elem * R + (valid[1] ? row[1] : 0)) * a.H + head) * D + 8 * g;
#pragma unroll
    for (int kd = 0; kd < 8; ++kd) {
      // unconditional (an invalid row reads row 0 of the element and is zeroed below): a
      // conditional load compiles to a branch that waits for it
      const uint4 x = *(const uint4*)(qb0 + 16 * kd);
      const uint4 y = *(const uint4*)(qb1 + 16 * kd);
      q0[4 * kd] = x.x; q0[4 * kd + 1] = x.y; q0[4 * kd + 2] = x.z; q0[4 * kd + 3] = x.w;
      q1[4 * kd] = y.x; q1[4 * kd + 1] = y.y; q1[4 * kd + 2] = y.z; q1[4 * kd + 3] = y.w;
    }
  }

  // Tile range of this split (as in attn_bf16_kernel: the walk ends with the last own frame a
  // row of the query tile sees).
  const int tq_hi = min(a.T - 1, (qtile * kQTile + kQTile - 1) / a.N);
  const int tiles_q = (a.nshared + tq_hi + 1) * a.tiles_per_frame;
  const int t_begin = (int)((int64_t)split * tiles_q / nsplit);
  const int t_end = (int)((int64_t)(split + 1) * tiles_q / nsplit);
  const int n = t_end - t_begin;              // >= 1
  const char* kvb = (const char*)a.kv;
  const int64_t head_off = (int64_t)head * a.head_stride;
  const int own_i = min(max(lane - a.nshared, 0), a.T - 1);
  const int slot_lane = lane < a.nshared ? a.slots[lane] : a.own_slot[elem * a.T + own_i];
  const char* const kblk = kvb + (a.k_layer_off + head_off) * EB;
  const char* const vblk = kvb + (a.v_layer_off + head_off) * EB;
  const int64_t slot_bytes = a.slot_stride * EB;
  // frame f's ring slot, f uniform: a scalar load, so the first tiles' loads do not wait for
  // slot_lane (a vector load)
  auto slot_of = [&](int f) -> int {
    return f < a.nshared ? a.slots[f] : a.own_slot[elem * a.T + min(max(f - a.nshared, 0), a.T - 1)];
  };
  auto frame_at = [&](TileCursor& c) {
    const int slot = slot_of(c.f);
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

  // Global->LDS loads.  bf16: wave w fills 1 KB pieces w*LD .. w*LD+LD-1 of each ring tile.
  // e4m3: wave w loads 16-byte chunks of K rows 16w + 8i + [0, 8) and V^T rows 32w + 16i +
  // [0, 16), i = 0, 1, lane l taking chunk kc8 of K row kr (vc8 of V^T row vr) below, into its
  // 2 KB of the staging slot in lane order.  The widened write of a lane's chunk lands at the
  // row's swizzled bf16 chunks; the LDS serves a 16-byte write 8 lanes (128 bytes) at a time, so
  // each group of 8 lanes pairs 4 chunks of a row with 4 of a row whose swizzle differs in bit 1
  // (K rows r and r + 2, V^T rows r and r + 4): their positions mod 128 bytes are disjoint and
  // every write is free of bank conflicts (in row order two rows of a group collide).
  const int g8 = lane >> 3, sub = (lane >> 2) & 1;
  const int kr = (0x5410 >> (4 * (g8 >> 1)) & 15) + 2 * sub;     // row pairs {0,2} {1,3} {4,6} {5,7}
  const int kc8 = (lane & 3) + 4 * (sub ^ (g8 & 1));
  const int vr = ((g8 & 3) | ((g8 & 4) << 1)) + 4 * sub, vc8 = lane & 3;
  uint32_t koff[LD], voff[LD];
  int kr8[LD], vr8[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    int Rr, c;
    if constexpr (F8) {
      kr8[i] = 16 * wave + 8 * i + kr;
      koff[i] = (uint32_t)(perm_key(kr8[i]) * D + kc8 * 16);
      vr8[i] = 32 * wave + 16 * i + vr;
      voff[i] = (uint32_t)(vr8[i] * a.Npad + vc8 * 16);
    } else {
      lds_chunk_inv<KRB>((wave * LD + i) * 64 + lane, Rr, c);
      koff[i] = (uint32_t)(perm_key(Rr) * KRB + c * 16);
      lds_chunk_inv<VRB>((wave * LD + i) * 64 + lane, Rr, c);
      voff[i] = (uint32_t)(Rr * a.Npad * 2 + c * 16);
    }
  }
  auto fill_k = [&](const TileCursor& c, int slot) {
#pragma unroll
    for (int i = 0; i < LD; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(c.kp + koff[i]),
          (lds_void*)(F8 ? ldsS + slot * STAGE + wave * 2048 + i * 1024 : ldsK + slot * K_BYTES + (wave * LD + i) * 1024),
          16, 0, 0);
  };
  auto fill_v = [&](const TileCursor& c, int slot) {
#pragma unroll
    for (int i = 0; i < LD; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(c.vp + voff[i]),
          (lds_void*)(F8 ? ldsS + slot * STAGE + STAGE / 2 + wave * 2048 + i * 1024
                         : ldsV + slot * V_BYTES + (wave * LD + i) * 1024),
          16, 0, 0);
  };

  // Prologue: V^T slot 3 (read as V(-1) with P(-1) = 0) zeroed; K(0) into slot 0, K(1) into
  // slot 1 (K(0) again when n = 1: the loop counts the loads in flight at its start), V(0)
  // into slot 0.  e4m3: the V^T half of staging slot 0 is zeroed instead (the program widens
  // it into V^T slot 3 with K(0) before its loop); K(0) goes to staging slot 0, K(1) and V(0)
  // to slot 1, as if loaded by iterations -2 and -1, in the order the program's load waits count.
  if constexpr (F8) {
#pragma unroll
    for (int i = 0; i < STAGE / 2 / (256 * 16); ++i)
      reinterpret_cast<uint4*>(ldsS + STAGE / 2)[tid + 256 * i] = make_uint4(0u, 0u, 0u, 0u);
  } else {
#pragma unroll
    for (int i = 0; i < V_BYTES / (256 * 16); ++i)
      reinterpret_cast<uint4*>(ldsV + 3 * V_BYTES)[tid + 256 * i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  const TileCursor c0 = cursor_at(t_begin);
  TileCursor kc = c0;
  fill_k(kc, 0);
  if (n > 1) advance(kc);
  fill_k(kc, 1);
  fill_v(c0, F8 ? 1 : 0);

  // Rows past the end read row 0 of the element (unconditional loads, issued before the first
  // tiles' loads and not waited for until here) and are zeroed.
  __builtin_amdgcn_sched_barrier(0);
  {
    const int keep0 = valid[0] ? -1 : 0, keep1 = valid[1] ? -1 : 0;   // masks, not branches
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      q0[i] &= keep0;
      q1[i] &= keep1;
    }
  }
  if constexpr (F8) {
    // the e4m3 cache stores its keys times key_scale * log2(e) * 2^k: queries times 2^-k (a power
    // of two: exact in fp32, and the product is a bf16 value, so its top half is exact)
    const float qm = a.qmul;
    auto scale2 = [qm](int w) {
      const float lo = __uint_as_float((uint32_t)w << 16) * qm;
      const float hi = __uint_as_float((uint32_t)w & 0xffff0000u) * qm;
      return (int)((__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u));
    };
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      q0[i] = scale2(q0[i]);
      q1[i] = scale2(q1[i]);
    }
  }

  // The tile loop (generated asm, see gen_attn_w64.py).  Its state lives in the registers
  // named by the operands below; the compiler sees one statement.
  i32x8 kaddr;                                // LDS addresses of K fragments per k step (slot 0)
  i32x4 vaddr;                                // LDS addresses of V^T fragments per key step (slot 0)
  i32x4 lanec;                                // 8g, frame of the row per qb, (lane ^ 32) * 4
  i32x4 koffv, voffv;
  {
    const uint32_t kb = (uint32_t)(uintptr_t)ldsK, vb = (uint32_t)(uintptr_t)ldsV;
#pragma unroll
    for (int kd = 0; kd < 8; ++kd) kaddr[kd] = (int)(kb + lds_chunk<KRB>(r, 2 * kd + g));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) vaddr[ks] = (int)(vb + lds_chunk<VRB>(r, 2 * ks + g));
    lanec[0] = 8 * g;
    lanec[1] = tq[0];
    lanec[2] = tq[1];
    lanec[3] = (lane ^ 32) * 4;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      koffv[i] = (int)koff[i];
      voffv[i] = (int)voff[i];
    }
  }
  f32x32 o0, o1, o2, o3, s0, s1;
  i32x32 p0, p1, frg;
  i32x16 frg2;
  i32x12 tmp;
  f32x2 mrun, lrun;
  i32x8 tsum;
  // scalar state: cursors (frame, tile in frame): kf, kk of the last K tile set up, vf, vk the
  // same one iteration earlier, sf, sk of the walk's tile t; iteration t
  int kf = kc.f, kk = kc.k, vf = c0.f, vk = c0.k, sf = c0.f, sk = c0.k, t = 0;
  const uint64_t kblk64 = (uint64_t)(uintptr_t)kblk, vblk64 = (uint64_t)(uintptr_t)vblk;
  const uint32_t kblo = (uint32_t)kblk64, kbhi = (uint32_t)(kblk64 >> 32);
  const uint32_t vblo = (uint32_t)vblk64, vbhi = (uint32_t)(vblk64 >> 32);
  const int slotb = (int)slot_bytes, tpf = a.tiles_per_frame, nshared = a.nshared, Ntok = a.N;
  const int mk = (int)((uint32_t)(uintptr_t)ldsK + wave * LD * 1024);
  const int mv = (int)((uint32_t)(uintptr_t)ldsV + wave * LD * 1024);
  // softmax scale in log2 units, its inverse, and the bias blocks' start -8 / scale_log2: kernel
  // arguments made wave-uniform, so the "s" operands below are scalar registers (a value the
  // compiler computes in a VGPR can be handed to an "s" operand as that VGPR)
  auto uniform = [](float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); };
  const float sl = uniform(a.scale_log2), slinv = uniform(a.scale_log2_inv), nbias = uniform(a.neg_bias);
  unsigned long long trig;
  int x, y, nvalid, tk, mflag0, mflag1, m0save, stmp, ov;
  // Register plan: O^T a[0:127], Q^T a[128:191], mask words a[192:223], lane constants
  // a[224:227], row-sum selector a[228:231]; S^T v[0:63], P^T v[64:127], fragment ring
  // v[128:175], LDS addresses v[176:187], temporaries v[188:199], m v[200:201], -m blocks
  // v[202:233], load offsets and frame slots v[236:244], a mask temporary v245, the OR of a
  // tile's P words v246, l accumulators (row sums on the matrix core) v[248:255].  e4m3 only:
  // staging read addresses v[234:235], widened-chunk write addresses a[232:239].
#define SDV2_W64_OUTPUTS                                                                      \
  "={a[0:31]}"(o0), "={a[32:63]}"(o1), "={a[64:95]}"(o2), "={a[96:127]}"(o3),                  \
      "={v[0:31]}"(s0), "={v[32:63]}"(s1), "={v[64:95]}"(p0), "={v[96:127]}"(p1),               \
      "={v[128:159]}"(frg), "={v[160:175]}"(frg2), "+{v[176:183]}"(kaddr),                      \
      "+{v[184:187]}"(vaddr), "={v[188:199]}"(tmp), "={v[200:201]}"(mrun),                      \
      "={v[248:255]}"(tsum), [kf] "+s"(kf), [kk] "+s"(kk), [vf] "+s"(vf), [vk] "+s"(vk),        \
      [sf] "+s"(sf), [sk] "+s"(sk), [t] "+s"(t), [trig] "=&s"(trig), [x] "=&s"(x),              \
      [y] "=&s"(y), [nvalid] "=&s"(nvalid), [tk] "=&s"(tk), [mflag1] "=&s"(mflag1),             \
      [mflag0] "=&s"(mflag0), [m0save] "=&s"(m0save), [stmp] "=&s"(stmp), [ov] "=&s"(ov)
#define SDV2_W64_INPUTS                                                                       \
  "{a[128:159]}"(q0), "{a[160:191]}"(q1), [n] "s"(n), [tpf] "s"(tpf),                           \
      [nshared] "s"(nshared), [N] "s"(Ntok), [tqw] "s"(tq_wave), [kblo] "s"(kblo),              \
      [kbhi] "s"(kbhi), [vblo] "s"(vblo), [vbhi] "s"(vbhi), [slotb] "s"(slotb), [sl] "s"(sl),   \
      [slinv] "s"(slinv), [nbias] "s"(nbias)
#define SDV2_W64_CLOBBERS "vcc", "scc", "memory", "s84", "s85", "s86", "s87", "s88", "s89", "s90", "s91"
  i32x32 negm, amask;
  unsigned long long ninf;
  // row-sum selector: bf16 ones at lanes 0 and 32 (output row 0) and 17 and 49 (row 1)
  i32x4 sel;
  {
    const int one2 = (lane == 0 || lane == 17 || lane == 32 || lane == 49) ? 0x3F803F80 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) sel[i] = one2;
  }
#define SDV2_W64_NEGM_OUTPUTS "={v[202:233]}"(negm), "={a[192:223]}"(amask), [ninf] "=&s"(ninf)
#define SDV2_W64_PLAN_INPUTS                                                                  \
  "{a[224:227]}"(lanec), "{a[228:231]}"(sel), "{v[236:239]}"(koffv), "{v[240:243]}"(voffv),    \
      "{v244}"(slot_lane)
  if constexpr (F8) {
    // e4m3 widening addresses: this lane's staged 16 bytes of each load (K, V^T) and the two
    // bf16 chunks each widens into (ring slot 0; the program adds the slot)
    const int ms = (int)((uint32_t)(uintptr_t)ldsS + wave * 2048);
    const int sk_addr = ms + lane * 16, sv_addr = ms + STAGE / 2 + lane * 16;
    i32x4 wk, wv;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      wk[2 * i] = (int)((uint32_t)(uintptr_t)ldsK + lds_chunk<KRB>(kr8[i], 4 * (kc8 >> 1) + (kc8 & 1)));
      wk[2 * i + 1] = (int)((uint32_t)(uintptr_t)ldsK + lds_chunk<KRB>(kr8[i], 4 * (kc8 >> 1) + 2 + (kc8 & 1)));
      wv[2 * i] = (int)((uint32_t)(uintptr_t)ldsV + lds_chunk<VRB>(vr8[i], 4 * (vc8 >> 1) + (vc8 & 1)));
      wv[2 * i + 1] = (int)((uint32_t)(uintptr_t)ldsV + lds_chunk<VRB>(vr8[i], 4 * (vc8 >> 1) + 2 + (vc8 & 1)));
    }
    asm volatile(SDV2_W64_LOOP_FP8
                 : SDV2_W64_OUTPUTS, SDV2_W64_NEGM_OUTPUTS
                 : SDV2_W64_INPUTS, SDV2_W64_PLAN_INPUTS, [ms] "s"(ms), "{v234}"(sk_addr), "{v235}"(sv_addr),
                   "{a[232:235]}"(wk), "{a[236:239]}"(wv)
                 : SDV2_W64_CLOBBERS, "v245", "v246");   // mask word temporary, OR of the P words
  } else if constexpr (SK) {
    asm volatile(SDV2_W64_LOOP_SK
                 : SDV2_W64_OUTPUTS, SDV2_W64_NEGM_OUTPUTS
                 : SDV2_W64_INPUTS, SDV2_W64_PLAN_INPUTS, [mk] "s"(mk), [mv] "s"(mv)
                 : SDV2_W64_CLOBBERS, "v245", "v246");   // mask word temporary, OR of the P words
  } else {
    asm volatile(SDV2_W64_LOOP
                 : SDV2_W64_OUTPUTS, SDV2_W64_NEGM_OUTPUTS
                 : SDV2_W64_INPUTS, SDV2_W64_PLAN_INPUTS, [mk] "s"(mk), [mv] "s"(mv)
                 : SDV2_W64_CLOBBERS, "v245", "v246");   // mask word temporary, OR of the P words
  }
  (void)negm;
  (void)amask;
  (void)ninf;
  // l of row j < 16 sits in lane j, register 4 qb; of row j + 16 in lane j, register 4 qb + 1
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float x0 = __shfl(__int_as_float(tsum[4 * qb]), r & 15);
    const float x1 = __shfl(__int_as_float(tsum[4 * qb + 1]), r & 15);
    lrun[qb] = r < 16 ? x0 : x1;
  }
#undef SDV2_W64_NEGM_OUTPUTS
#undef SDV2_W64_PLAN_INPUTS
#undef SDV2_W64_OUTPUTS
#undef SDV2_W64_INPUTS
#undef SDV2_W64_CLOBBERS
  (void)frg;
  (void)frg2;
  (void)tmp;
  (void)s0;
  (void)s1;
  (void)p0;
  (void)p1;
  (void)trig;

  // Epilogue.  Lane (g, r), element v of o[db][qb] (o_db[16 qb + v]) holds
  // O^T[d = 32 db + 8 (v / 4) + 4 g + v % 4][row r of block qb].  The wave writes its 64 rows of
  // O / l (bf16) into LDS row by row, then stores them four whole rows per instruction: stored
  // straight from the accumulator layout, each instruction would write 8 bytes into each of
  // 32 rows, and the L2's write transactions took about 5 us per workgroup.
  constexpr int EP_STRIDE = D * 2 + 16;                         // bytes per LDS row (padded)
  __syncthreads();                                              // every wave is done with the rings
  char* const ep = lds + wave * 64 * EP_STRIDE;
  auto oval = [&](int db, int i) { return db == 0 ? o0[i] : db == 1 ? o1[i] : db == 2 ? o2[i] : o3[i]; };
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = lrun[qb];
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* const erow = ep + (32 * qb + r) * EP_STRIDE + 8 * g;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int i0 = 16 * qb + 4 * a4;
        uint2 w2;
        w2.x = pack_bf16x2(oval(db, i0) * inv, oval(db, i0 + 1) * inv);
        w2.y = pack_bf16x2(oval(db, i0 + 2) * inv, oval(db, i0 + 3) * inv);
        *(uint2*)(erow + 2 * (32 * db + 8 * a4)) = w2;
      }
    if (nsplit > 1 && g == 0 && valid[qb]) {
      const int64_t prow = ((int64_t)split * a.plan.tail_first[kNumXcd] + wi.tail) * kQTile + wave * 64 + 32 * qb + r;
      a.part_ml[prow] = make_float2(mrun[qb], l_tot);
    }
  }
  // lane L stores 16 bytes (8 values of d) of row 4 i + L / 16 of the wave
  const int chunk = lane & 15;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int rl = 4 * i + (lane >> 4), grow = wrow + rl;
    const uint4 w4 = *(const uint4*)(ep + rl * EP_STRIDE + 16 * chunk);
    if (grow < R) {
      uint16_t* dst = nsplit == 1
          ? (uint16_t*)a.out + ((int64_t)(elem * R + grow) * a.H + head) * D
          : a.part_o + (((int64_t)split * a.plan.tail_first[kNumXcd] + wi.tail) * kQTile + grow - qtile * kQTile) * D;
      *(uint4*)(dst + 8 * chunk) = w4;
    }
  }
}

hipError_t launch_attention_w64(const AttnArgs& a, int kv, hipStream_t s) {
  const int grid = kNumXcd * a.plan.wg_per_xcd;
  if (kv == kKvFP8)
    hipLaunchKernelGGL((attn_w64_kernel<true, true>), dim3(grid), dim3(256), 0, s, a);
  else if (a.scaled_keys)
    hipLaunchKernelGGL((attn_w64_kernel<false, true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_w64_kernel<false, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdv2
