// Internal definitions shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdv2 {

constexpr int kMaxShared = 64;   // S + W
constexpr int kMaxBatch = 8;     // B
constexpr int kMaxSinks = 16;    // S
constexpr int kMaxTPairs = 32;   // temporal RoPE pairs
constexpr int kTileKeys = 64;    // key tile; tokens are padded to a multiple of it
constexpr int kQTile = 256;      // query rows per attention workgroup (8 waves x 32)
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

// Workgroup id -> work item such that consecutive work items run on the same XCD (each XCD
// has its own L2): hardware sends workgroup i to XCD i % 8.  A bijection on [0, G).
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid % kNumXcd, per = G / kNumXcd, rem = G % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + bid / kNumXcd;
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
};

struct AttnArgs {
  const void* q;           // [nbatch][T*N][H][D] rotated queries
  void* out;               // [nbatch][T*N][H][D]
  const void* kv;
  int64_t k_layer_off, v_layer_off, slot_stride, head_stride;
  uint16_t* part_o;        // [nsplit][nbatch][H][T*N][D] bf16 O/l of the split (split-KV only)
  float2* part_ml;         // [nsplit][nbatch][H][T*N] (m in log2 units, l)
  int N, Npad, H, nbatch;  // N: tokens per frame
  int T;                   // frames per chunk (block-causal inside the chunk)
  int nshared;             // cached frames attended (sinks + window)
  int own_slot[kMaxBatch]; // slot of own-chunk frame t of element b, index b * T + t
  int tiles_per_frame;     // Npad / kTileKeys
  int total_tiles;         // (nshared + T) * tiles_per_frame
  int nsplit, qtiles;
  float scale_log2;        // softmax scale * log2(e)
  float scale;
  int slots[kMaxShared];   // cache slots of the shared frames, in attention order
};

struct CombineArgs {
  const uint16_t* part_o;
  const float2* part_ml;
  void* out;
  int N, H, nbatch, nsplit;  // N: query rows per (element, head)
};

struct RebaseArgs {
  void* kv;
  int64_t layer_stride, slot_stride, head_stride;
  int L, H, N, pt, nslots;
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

struct SinkArgs {
  const float* h;          // [D] new chunk embedding
  float* embeds;           // [S][D] sink embeddings
  int32_t* decision;       // [0] = replaced slot or -1
  double* alpha;           // [0] = alpha of the least similar sink
  int S, D;
  int store_slot;          // >= 0: store h as that sink's embedding, no decision
  double tau;
};

// ---- launchers (defined in the .hip files) --------------------------------------------------
hipError_t launch_rope_append(const AppendArgs& a, int head_dim, int kv, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int head_dim, int kv, hipStream_t s);
hipError_t launch_attention_w64(const AttnArgs& a, int kv, hipStream_t s);   // bf16 or e4m3 cache, head_dim 128
hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s);
hipError_t launch_rebase(const RebaseArgs& a, int head_dim, int kv, hipStream_t s);
hipError_t launch_copy_slots(const CopyArgs& a, hipStream_t s);
hipError_t launch_sink_decide(const SinkArgs& a, hipStream_t s);
hipError_t launch_motion(const float* frames, int nframes, int64_t elems, double* dist,
                         double* partials, int parts, hipStream_t s);
int motion_parts(int64_t elems);

}  // namespace sdv2
