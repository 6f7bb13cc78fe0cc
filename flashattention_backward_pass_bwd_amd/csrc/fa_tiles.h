// bf16 LDS tiles for the gfx950 MFMA kernels.
//
// A tile holds ROWS rows of D bf16 values, row-major, 2*D bytes per row with no
// padding; the 16-byte chunk c of row r is stored at chunk position
// c ^ swz(r).  Two read patterns hit the tile:
//   * row reads (ds_read_b128): lane l reads chunk c of row r0 + l%32 -- the
//     MFMA operand whose k index runs along the row;
//   * transposed reads (ds_read_b64_tr_b16): each 16-lane group reads a
//     4-row x 16-column block and every lane receives one column of 4 rows --
//     the MFMA operand whose k index runs down the rows.
// swz(r) = 2*(r%4) + (r/4)%2 makes both conflict-free: eight consecutive rows
// see eight distinct 16-byte bank groups, and four consecutive rows see four
// distinct 32-byte bank groups.
#pragma once

#include "fa_common.h"

namespace fa {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Element offset of chunk c of row r in a swizzled tile with D columns.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * D + ((c ^ swz(r)) << 3);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 concat(const bf16x4& a, const bf16x4& b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Per-lane element offset (excluding the 16-row block base qb*D) of the
// transposed read that gives lane l column 32*db + l%32 and rows
// qb + 4*(l/32) + 0..3 (the second half of the operand is 8 rows further on).
template <int D>
__device__ __forceinline__ int tr_lane_off(int lane, int db) {
  const int g = lane >> 4;        // 16-lane group
  const int s = lane & 15;        // source slot within the group
  const int r = 4 * (g >> 1) + (s >> 2);            // row within the 16-row block
  const int col = 32 * db + 16 * (g & 1) + 4 * (s & 3);
  return r * D + (((col >> 3) ^ swz(r)) << 3) + (col & 7);
}

}  // namespace fa
