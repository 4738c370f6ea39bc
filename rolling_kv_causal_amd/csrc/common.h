// Internal definitions shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdv2 {

constexpr int kMaxShared = 64;   // S + W + T'
constexpr int kMaxBatch = 8;     // B
constexpr int kMaxSinks = 16;    // S
constexpr int kMaxTPairs = 32;   // temporal RoPE pairs
constexpr int kTileKeys = 64;    // key tile; tokens are padded to a multiple of it
constexpr int kQTile = 256;      // query rows per attention workgroup (4 waves x 64, or 8 x 32 at d = 64)
constexpr int kNumXcd = 8;       // MI355X: 8 XCDs, workgroups dispatched round-robin over them

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 <-> fp32 (bit patterns in uint16_t) -------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round two fp32 values to bf16 (nearest even, hardware v_cvt_pk_bf16_f32); low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Cache element types: fp32, bf16, or OCP e4m3 (with bf16 activations).
constexpr int kKvF32 = 0, kKvBF16 = 1, kKvFP8 = 2;

// e4m3 cache layout: inside each group of 32 elements (32 dims of a K row; 32 tokens of a V^T
// row within a 64-token tile) element 32p + 16h + 8g + e is stored at 32p + 16g + 8h + e (bits
// 3 and 4 swapped; its own inverse).  A 16-byte read at 32p + 16g then holds the 8 elements
// lane half g needs for the two 16-wide MFMA k steps 2p and 2p + 1.
__host__ __device__ __forceinline__ int fp8_pos(int i) {
  return (i & ~24) | ((i & 8) << 1) | ((i & 16) >> 1);
}

// Four fp32 values -> four OCP e4m3 bytes (low byte first): round to nearest even, saturated
// at +-448 (the conversion instruction itself turns values past the last rounding interval
// into NaN).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// 16-byte store with the non-temporal hint: data written once and read by a later launch (from
// HBM, usually on another XCD) does not displace the L2 lines of the data still being read.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void* p, const uint4& w) {
  const u32x4_t v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// Workgroup id -> work item such that consecutive work items run on the same XCD (each XCD
// has its own L2): hardware sends workgroup i to XCD i % 8.  A bijection on [0, G).
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid % kNumXcd, per = G / kNumXcd, rem = G % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + bid / kNumXcd;
}

// ---- split-KV work plan ---------------------------------------------------------------------
// Work items are query tiles of kQTile rows of one (element, head), numbered
// item = (head * nbatch + elem) * qtiles + qtile.  XCD x owns items [first[x], first[x + 1]),
// so the items sharing one head's K/V use one L2.  On XCD x the first whole[x] items run whole,
// one workgroup each (output written directly); the rest, its tail items, are split into
// nsplit key ranges, one workgroup each, whose partial results combine_kernel merges.  Tail
// items are numbered across XCDs from tail_first[x].  Hardware sends workgroup b to XCD
// b % kNumXcd as that XCD's (b / kNumXcd)-th workgroup, so each XCD starts its whole items
// first; the grid holds wg_per_xcd workgroups per XCD, and those past an XCD's share exit.
struct WorkPlan {
  int first[kNumXcd + 1];
  int whole[kNumXcd];
  int tail_first[kNumXcd + 1];   // tail_first[kNumXcd] = tail items in all
  int nsplit;                    // key ranges of a tail item (>= 2 when there are tail items)
  int wg_per_xcd;
};

struct WorkItem {
  int head, elem, qtile;
  int split, nsplit;             // key range split of nsplit (0 of 1 for a whole item)
  int tail;                      // tail item index, or -1 for a whole item
};

// Workgroup b of the plan; false for a workgroup past its XCD's share.
__host__ __device__ __forceinline__ bool plan_item(const WorkPlan& p, int qtiles, int nbatch, int b,
                                                   WorkItem& w) {
  const int x = b % kNumXcd, j = b / kNumXcd;
  int item;
  if (j < p.whole[x]) {
    item = p.first[x] + j;
    w.split = 0;
    w.nsplit = 1;
    w.tail = -1;
  } else {
    const int jj = j - p.whole[x];
    const int t = jj / p.nsplit;
    item = p.first[x] + p.whole[x] + t;
    if (item >= p.first[x + 1]) return false;
    w.split = jj - t * p.nsplit;
    w.nsplit = p.nsplit;
    w.tail = p.tail_first[x] + t;
  }
  w.qtile = item % qtiles;
  const int r = item / qtiles;
  w.elem = r % nbatch;
  w.head = r / nbatch;
  return true;
}

// Tail item t -> (head, elem, qtile).
__host__ __device__ __forceinline__ void plan_tail(const WorkPlan& p, int qtiles, int nbatch, int t,
                                                   int& head, int& elem, int& qtile) {
  int x = 0;
  while (x + 1 < kNumXcd && t >= p.tail_first[x + 1]) ++x;
  const int item = p.first[x] + p.whole[x] + (t - p.tail_first[x]);
  qtile = item % qtiles;
  const int r = item / qtiles;
  elem = r % nbatch;
  head = r / nbatch;
}

// ---- kernel argument blocks (passed by value) ----------------------------------------------
struct AppendArgs {
  void* q;                 // [nbatch][T*N][H][D], rotated in place
  const void* k;
  const void* v;
  void* kv;                // cache base
  int64_t k_layer_off;     // element offsets of this layer's K and V blocks
  int64_t v_layer_off;
  int64_t slot_stride;
  int64_t head_stride;
  const float2* tab_h;     // [grid_h][ph] (cos, sin)
  const float2* tab_w;     // [grid_w][pw]
  int N, Npad, H, grid_w, nbatch;
  int T;                   // frames per chunk; nbatch * T <= kMaxBatch
  int dst_slot[kMaxBatch]; // slot of frame t of element b, index b * T + t
  int pt, ph, pw;          // RoPE pairs per axis
  float2 tcs[kMaxBatch][kMaxTPairs];   // temporal (cos, sin) per frame (b * T + t) and pair
  float kmul;              // factor on rotated k before its rounding (1, or key_scale * log2 e)
};

struct AttnArgs {
  const void* q;           // [nbatch][T*N][H][D] rotated queries
  void* out;               // [nbatch][T*N][H][D]
  const void* kv;
  int64_t k_layer_off, v_layer_off, slot_stride, head_stride;
  uint16_t* part_o;        // [nsplit][tail items][kQTile][D] bf16 O/l of the split
  float2* part_ml;         // [nsplit][tail items][kQTile] (m in log2 units, l)
  int N, Npad, H, nbatch;  // N: tokens per frame
  int T;                   // frames per chunk (block-causal inside the chunk)
  int nshared;             // cached frames attended (sinks + window)
  int own_slot[kMaxBatch]; // slot of own-chunk frame t of element b, index b * T + t
  int tiles_per_frame;     // Npad / kTileKeys
  int total_tiles;         // (nshared + T) * tiles_per_frame
  int qtiles;
  WorkPlan plan;
  float scale_log2;        // softmax scale * log2(e); 1 when the keys are cached times it
  float scale;
  int scaled_keys;         // keys cached times scale * log2(e): the 64-row kernel's program without products
  float qmul;              // e4m3 cache: queries times this power of two (2^-k of the key factor)
  float scale_log2_inv;    // 1 / scale_log2
  float neg_bias;          // -8 / scale_log2: start of the 64-row kernel's -(m + 8) / scale_log2 blocks
  int slots[kMaxShared];   // cache slots of the shared frames, in attention order
};

struct CombineArgs {
  const uint16_t* part_o;
  const float2* part_ml;
  void* out;
  int N, H, nbatch, qtiles;  // N: query rows per (element, head)
  WorkPlan plan;
};

struct RebaseArgs {
  void* kv;
  int64_t layer_stride, slot_stride, head_stride;   // elements
  int L, H, N, pt, nslots;
  int cpr;                 // 16-byte chunks at the start of a key row that hold every temporal pair
  int slots[kMaxShared];
  float2 cs[kMaxTPairs];   // (cos, sin) of the rebase angle per temporal pair
};

struct CopyArgs {
  char* kv;
  int64_t layer_stride_bytes;
  int64_t v_block_bytes;   // byte offset of the V block inside a layer
  int64_t slot_bytes;      // bytes of one slot of K (= of V)
  int src_slot;
  int dst_slot;            // used when dst_from == nullptr
  const int32_t* dst_from; // device decision: copy into slot *dst_from, skip if < 0
  int L;
};

// Fused chunk statistics ([NEWS] algorithm item 2 and [WT] motion-aware noise scheduler: the
// distance between consecutive latent frames; [WT] adaptive sink and RoPE refresh: cosine
// similarity of the chunk embedding against the sinks).  Pass 1, many blocks: per block the
// fp64 partial sums of sum (cur - prev)^2 over a range of latent elements and of h.h, e_j.e_j,
// h.e_j over a range of embedding elements.  Pass 2, one block: the partials summed in block
// order, the statistics, the replacement decision and the embedding stores.
constexpr int kStatsQ = 2 + 2 * kMaxSinks;   // per block: motion, h.h, e_j.e_j, h.e_j
constexpr int kStatsMaxBlocks = 256;
constexpr int kStatsLatPerBlock = 8192;      // latent elements per block (at least)
constexpr int kStatsEmbPerBlock = 1024;      // embedding elements per block (at least)

struct StatsArgs {
  const float* prev;       // [n_lat] previous latent frame (n_lat = 0: no motion term)
  const float* cur;        // [n_lat] newest latent frame
  int64_t n_lat;
  int64_t lat_per_block;   // multiple of 4
  const float* h;          // [D] chunk embedding (D = 0: no similarity terms)
  const float* embeds;     // [S][D] sink embeddings
  int S, D, emb_per_block;
  double* part;            // [gridDim.x][kStatsQ] partial sums
};

struct SinkArgs {
  const double* part;      // [blocks][kStatsQ] from the stats pass
  int blocks;
  int64_t n_lat;
  const float* h;          // [D] chunk embedding
  float* embeds;           // [S][D] sink embeddings
  int S, D;
  int store_lo, store_hi;  // sinks [store_lo, store_hi) take h as their embedding (chunk frames below S)
  int decide;              // 1: take the replacement decision (frame >= S, tau on)
  double tau;
  int32_t* decision;       // [0] = replaced slot or -1
  double* alpha;           // [0] = alpha of the least similar sink
  double* stats;           // [4 + 2S] caller's statistics, or nullptr
};

// ---- launchers (defined in the .hip files) --------------------------------------------------
hipError_t launch_rope_append(const AppendArgs& a, int head_dim, int kv, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int head_dim, int kv, hipStream_t s);
hipError_t launch_attention_w64(const AttnArgs& a, int kv, hipStream_t s);   // bf16 or e4m3 cache, head_dim 128
hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s);
hipError_t launch_rebase(const RebaseArgs& a, int head_dim, int kv, hipStream_t s);
hipError_t launch_copy_slots(const CopyArgs& a, hipStream_t s);
hipError_t launch_chunk_stats(const StatsArgs& a, int blocks, hipStream_t s);
hipError_t launch_sink_decide(const SinkArgs& a, hipStream_t s);
hipError_t launch_motion(const float* frames, int nframes, int64_t elems, double* dist,
                         double* partials, int parts, hipStream_t s);
int motion_parts(int64_t elems);

}  // namespace sdv2
