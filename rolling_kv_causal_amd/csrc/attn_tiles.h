// LDS tile layout and tile walk shared by the bf16 attention kernels.
#pragma once

#include "common.h"

namespace sdv2 {

constexpr float kLazyMass = 256.0f;   // 2^8: bound on a lane's sum of exponentials
// s_waitcnt immediate for gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);

// LDS row of key `key` within a 64-key tile: swap bits 2 and 3 of the key index.
__device__ __forceinline__ int perm_key(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Byte offset of 16-byte chunk c of row R in an LDS tile whose rows are RB bytes (256 or 128).
// The LDS has 64 four-byte banks (a 256-byte period): 256-byte rows XOR the chunk index with
// (R & 15); 128-byte rows are paired into 256-byte double rows J = R >> 1 whose 16 chunk
// positions are XORed with (J & 15).  Either way the 16 lanes that read one chunk column of 16
// consecutive rows hit 16 different bank groups.
template <int RB>
__device__ __forceinline__ int lds_chunk(int R, int c) {
  if constexpr (RB == 256) return R * 256 + ((c ^ (R & 15)) << 4);
  else if constexpr (RB == 128) return (R >> 1) * 256 + (((((R & 1) << 3) | c) ^ ((R >> 1) & 15)) << 4);
  else return R * 64 + ((c ^ ((R >> 2) & 3)) << 4);   // 64-byte rows: 16 rows x 1 chunk column
}
// Inverse: LDS chunk position pos -> (row, logical chunk).
template <int RB>
__device__ __forceinline__ void lds_chunk_inv(int pos, int& R, int& c) {
  if constexpr (RB == 256) {
    R = pos >> 4;
    c = (pos & 15) ^ (R & 15);
  } else if constexpr (RB == 128) {
    const int J = pos >> 4, p = (pos & 15) ^ (J & 15);
    R = 2 * J + (p >> 3);
    c = p & 7;
  } else {
    R = pos >> 2;
    c = (pos & 3) ^ ((R >> 2) & 3);
  }
}

// Tile walk of one split: frame f, tile k within the frame, and the addresses of the tile's
// K rows and V^T columns.  Frames are [shared frames..., own chunk].
struct TileCursor {
  int f, k;
  const char* kp;
  const char* vp;
};

}  // namespace sdv2
