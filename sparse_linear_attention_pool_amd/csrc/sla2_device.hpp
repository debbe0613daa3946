// Device helpers shared by the SLA2 kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace sla2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
// native 16-byte vector (HIP's uint4 is a struct; copying it goes through memcpy, which keeps
// register arrays of it in stack memory)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;           // b_q = b_kv (SLA page, section 2 Q2)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFp8Max = 448.0f;    // largest finite OCP e4m3 magnitude
// phi values lie in (0, 1]: their e4m3 codes use the fixed scale 1/448, so a product of two
// codes carries the factor 448^2.
constexpr float kPhiCodeScale = 448.0f;

// E8M0 exponent passed to the scaled fp8 matrix-core instruction for "no extra scaling".
#ifndef SLA2_FP8_MFMA_SCALE
#define SLA2_FP8_MFMA_SCALE 0
#endif

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Round to nearest even into a packed pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// The four e4m3 codes of w (byte k = code k) as floats, by the hardware conversion (OCP e4m3 on
// gfx950, exact).  A GPU test pins it against the e4m3 definition on all 256 codes.
__device__ __forceinline__ f32x4 e4m3_decode4(uint32_t w) {
  return f32x4{__builtin_amdgcn_cvt_f32_fp8((int)w, 0), __builtin_amdgcn_cvt_f32_fp8((int)w, 1),
               __builtin_amdgcn_cvt_f32_fp8((int)w, 2), __builtin_amdgcn_cvt_f32_fp8((int)w, 3)};
}

// Four floats -> four e4m3 codes (round to nearest even) in one dword, byte k = value k.
// Callers clamp to +-448 first.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ float clamp_fp8(float y) { return fminf(fmaxf(y, -kFp8Max), kFp8Max); }

// fl32(x / s) for the block quantisers, given inv_s = fl64(1 / s): fl32(fl64(x * inv_s)).  The
// fp64 product is within 2^-52 (relative) of x / s, while a quotient of two fp32 values is
// never an fp32 rounding midpoint and lies more than 2^-49 (relative) from every one, so
// rounding the product to fp32 gives the correctly rounded quotient.
__device__ __forceinline__ float div_by_scale(float x, double inv_s) { return (float)((double)x * inv_s); }

// ---------------------------------------------------------------- matrix cores
// D(16x16) += A(16x32) * B(32x16), bf16 in, fp32 accumulate.  Lane l holds A[l%16][8(l/16)+e]
// and B[8(l/16)+e][l%16] (e = 0..7); D[4(l/16)+r][l%16] in accumulator r.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x128) * B(128x16), e4m3 in (32 bytes per lane), fp32 accumulate; the same
// lane/row/column mapping as above with 32 k-values per lane.
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, SLA2_FP8_MFMA_SCALE, 0,
                                                          SLA2_FP8_MFMA_SCALE);
}

// D(16x16) += A(16x4) * B(4x16), fp64.  Lane l holds A[l%16][l/16] and B[l/16][l%16];
// D[4r+l/16][l%16] in accumulator r (rows interleaved, unlike the fp32-output forms above).
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- cross-lane
// All-reduce over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).  The max takes
// v with both values of the swapped pair as one three-input max: fmaxf of the pair alone made the
// compiler quiet both inputs first (two more instructions per stage).
__device__ __forceinline__ float rows4_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(fmaxf(v, __uint_as_float(r[0])), __uint_as_float(r[1]));
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(fmaxf(v, __uint_as_float(s[0])), __uint_as_float(s[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// All-reduce within each 16-lane row: rotate by 8 and 4, then swap pairs and neighbours.  Each
// stage is a three-input max with -inf as the third input: the two-input form made the compiler
// quiet the moved value first, one more instruction per stage.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(fmaxf(v, -INFINITY), dpp<0x128>(v));   // row_ror:8
  v = fmaxf(fmaxf(v, -INFINITY), dpp<0x124>(v));   // row_ror:4
  v = fmaxf(fmaxf(v, -INFINITY), dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(fmaxf(v, -INFINITY), dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp<0x128>(v);
  v = v + dpp<0x124>(v);
  v = v + dpp<0x4E>(v);
  v = v + dpp<0xB1>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  return rows4_max(row16_max(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  return rows4_sum(row16_sum(v));
}

// ---------------------------------------------------------------- LDS staging
// Barrier for LDS hand-offs inside a loop over staged tiles: this wave's LDS writes are retired,
// then all waves meet.  Unlike __syncthreads() it does not drain the vector-memory loads in
// flight (the prefetched tile), which the compiler waits for where they are used.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 0xF | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Tiles move from memory straight into LDS (buffer loads with the LDS destination): lane l
// of a wave writes the 16 bytes at its wave's LDS pointer + 16 l, so each thread loads the
// chunk that belongs at its LDS slot.  A swizzle of the LDS rows (chunk c of row r at
// position c ^ (r & 7), fp8_chunk(r, c) for e4m3 rows read by lds_fp8_row, or c ^ (r & 15) for
// 256-byte rows) is applied to the memory address instead.  Callers keep every read inside the buffer.
__device__ __forceinline__ void lds_dma(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// All of this wave's tile copies have landed in LDS (they count as vector-memory loads).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0) only

// Physical slot of 16-byte chunk c in row r of a tile of 128-byte e4m3 rows: c XOR the 3-bit
// left rotation of r mod 8 (an involution, so the copy into LDS fetches chunk fp8_chunk(r, p)
// for slot p).  Measured on gfx950, the two reads of lds_fp8_row (16 consecutive rows, chunks
// 2g and 2g+1 for lane group g) then run at the full LDS read rate of 256 bytes per clock and
// CU; with c XOR (r mod 8) every such read costs two passes.
__device__ __forceinline__ int fp8_chunk(int row, int c) { return c ^ (((row << 1) | ((row >> 2) & 1)) & 7); }

// 32 e4m3 codes of one 128-byte LDS row (logical chunks 2g and 2g+1, stored at fp8_chunk): the
// A operand of a 16x16x128 matrix-core product for row `row`.
__device__ __forceinline__ i32x8 lds_fp8_row(const uint8_t* base, int row, int g) {
  const uint8_t* r = base + row * 128;
  const u32x4 a = *reinterpret_cast<const u32x4*>(r + 16 * fp8_chunk(row, 2 * g));
  const u32x4 b = *reinterpret_cast<const u32x4*>(r + 16 * fp8_chunk(row, 2 * g + 1));
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// ---------------------------------------------------------------- launch order
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup id w runs on XCD w % 8).
// Returns a logical id such that consecutive logical ids run on the same XCD, so that
// neighbouring query blocks of a head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int X = 8;
  const int per = nblocks / X, rem = nblocks % X;
  const int xcd = bid % X, idx = bid / X;
  const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return start + idx;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0..N-1, so that array indices
// inside f are constants from the start (register arrays then never become stack memory).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

}  // namespace sla2
