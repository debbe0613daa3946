// Transposing LDS reads (gfx950 ds_read_b64_tr_b16) for matrix-core operands whose
// contraction index runs down the rows of a row-major 16-bit tile in LDS.
//
// Within each group of 16 lanes, the four 16-bit values that source lane i loads from its own
// address, M[i][0..3], reach lane j as M[4k + j / 4][j % 4], k = 0..3 (pinned on the GPU with
// an in-bounds probe).  So with lane i of a group addressing X[r0 + i / 4][c0 + 4 (i % 4)],
// lane j receives X[r0 + k][c0 + j], k = 0..3: four consecutive rows of column c0 + j, which is
// half of the eight-element k-run a 16x16x32 bf16 operand lane holds.
#pragma once
#include "sla2_device.hpp"

namespace sla2 {

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_tr16(const void* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Unswizzled tile, row stride `ld` elements (8-byte aligned rows): rows r0..r0+3, column c0 + j.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* x, int ld, int r0, int c0, int i) {
  return lds_tr16(x + (r0 + (i >> 2)) * ld + c0 + 4 * (i & 3));
}

// The same on a tile of 256-byte rows (128 elements) whose 16-byte chunk k of row r sits at
// chunk k ^ (r % 16).
__device__ __forceinline__ u32x2 lds_read_tr16_sw256(const uint8_t* tile, int r0, int c0, int i) {
  const int row = r0 + (i >> 2), col = c0 + 4 * (i & 3);
  return lds_tr16(tile + row * 256 + 16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7));
}

// Tiles of 256-byte rows (128 bf16) whose 16-byte chunk k of row r sits at chunk k ^ rswz(r),
// rswz(r) = (n(r mod 4) << 2) | n((r / 4) mod 4) with n(x) = (4 - x) mod 4.  Measured on gfx950:
// the transposing reads of a 16 x 16 operand (16-lane groups over four rows, eight groups of
// rows 8 apart) run at about 218 bytes per clock and CU in this layout, against 118 with rows
// padded to 272 bytes or with chunk k ^ (r mod 16); 16 lanes writing or reading one whole row
// with 16-byte accesses stay conflict-free as well.
__device__ __forceinline__ int rswz(int r) {
  return (((4 - (r & 3)) & 3) << 2) | ((4 - ((r >> 2) & 3)) & 3);
}
__device__ __forceinline__ uint8_t* rswz_chunk(uint8_t* tile, int r, int k) { return tile + r * 256 + 16 * (k ^ rswz(r)); }
__device__ __forceinline__ const uint8_t* rswz_chunk(const uint8_t* tile, int r, int k) {
  return tile + r * 256 + 16 * (k ^ rswz(r));
}
// rows r0..r0+3, column c0 + j of such a tile (the transposing read; c0 a multiple of 4)
__device__ __forceinline__ u32x2 lds_read_tr16_rswz(const uint8_t* tile, int r0, int c0, int i) {
  const int row = r0 + (i >> 2), col = c0 + 4 * (i & 3);
  return lds_tr16(rswz_chunk(tile, row, col >> 3) + 2 * (col & 7));
}

}  // namespace sla2
