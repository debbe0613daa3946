// SLA2 linear-branch precompute: per key block j, with the smoothed keys K~ = K - mu,
//   phi(K~_t) = softmax over the d features of token t,
//   h_j = sum_t phi(K~_t)^T V_t (d x d, stored transposed: h[j][c][a]),
//   z_j = sum_t phi(K~_t),
// plus h_sum = sum_j h_j and z_sum = sum_j z_j (chunk partials, then a fixed-order sum).
// In FP8 mode the same pass quantises K~ per 64-token block (absmax/448 scale, e4m3 codes).
// The bf16 pass also writes, for the fused forward kernel, each block's V transposed (with
// the key order of its matrix-core operands) and the e4m3 codes of 448 phi(K~) (phi <= 1, so
// one fixed scale serves every block; features permuted to the forward kernel's operand
// order); h_j and z_j themselves are stored only if asked for.
//
// Pages: "SLA: Beyond Sparsity in Diffusion Transformers...", section 2 Q2 step 3 and the
// section 3 figure (h_j = phi(K_j)^T V_j, z_j = rowsum(phi(K_j)^T), phi = softmax), section 4
// (linear re-association); "SLA2: Sparse-Linear Attention with Learnable Routing and QAT",
// section 3 (the linear branch first forms K^T V statistics, then multiplies by Q), section 5
// (K quantised with scales), section 6 (key smoothing before block processing).
#include <math.h>

#include "sla2_device.hpp"
#include "sla2_internal.hpp"
#include "sla2_lds.hpp"

namespace sla2 {

// ---------------------------------------------------------------------------------------
// bf16, d = 128: one workgroup per (chunk of kChunk key blocks, head), 256 threads.
// Thread (c = tid % 16, r0 = tid / 16) holds columns 8c..8c+7 of rows r0 + 16p, p = 0..3
// (a 16-lane row of a wave holds one token).  Block j's V is copied straight into LDS (tile
// j % 2) while block j - 1 is processed, and its K into registers (set j % 2) while block j - 2
// is: both copies have a whole block's work to land.  The block loop is unrolled by two so that
// the tile and register set are fixed at compile time.
// phi and V go to LDS token-major (256-byte rows, rswz layout); the operands whose contraction index
// runs down those rows (tokens) are read with the transposing LDS reads.  Wave w computes the
// 4 x 4 tiles (a-tiles 4*(w/2).., c-tiles 4*(w%2)..) of D[a][c] = sum_t phi[t][a] V[t][c] with
// v_mfma_f32_16x16x32_bf16 over 64 tokens.  phi is
// split into bf16 hi + lo parts (phi - hi rounded again), so the product carries phi to about
// 2^-16 relative although the matrix cores take bf16; V is bf16 already.
// ---------------------------------------------------------------------------------------
// the 8-element operand of rows r0 .. r0 + 7 at column c0 + j (two transposing reads)
__device__ __forceinline__ bf16x8 lds_op_tr16(const uint8_t* x, int r0, int c0, int i) {
  const u32x2 a = lds_read_tr16_rswz(x, r0, c0, i), b = lds_read_tr16_rswz(x, r0 + 4, c0, i);
  return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// Exponent e of the power-of-two scale of one V channel of a key block (SLA2 page, section 5,
// low-bit P.V): the smallest integer e >= -127 with amax <= 448 * 2^e; -127 for amax = 0.
// The comparisons are exact (448 * 2^e is a float), so the choice has one answer.
__device__ __forceinline__ int v_scale_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  int e = __builtin_amdgcn_frexp_expf(amax) - 10;    // amax = f 2^x, 0.5 <= f < 1: 448 2^(x-10) < amax
  while (__builtin_amdgcn_ldexpf(kFp8Max, e) < amax) ++e;   // at most three steps
  return e > -127 ? e : -127;
}

template <bool FP8, bool STORE, bool PV8>
__global__ __launch_bounds__(256, STORE ? 1 : 2) void precompute_bf16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ k_mean,
    int N, int T, int P, uint8_t* __restrict__ k8, float* __restrict__ k_scale,
    uint16_t* __restrict__ h, float* __restrict__ z, float* __restrict__ hpart,
    float* __restrict__ zpart, uint16_t* __restrict__ vt, uint8_t* __restrict__ phik8, float* __restrict__ zblk,
    uint8_t* __restrict__ vexp) {
  constexpr int D = 128;
  // token-major tiles of 256-byte rows in the rswz layout (sla2_lds.hpp): phi hi, phi lo, V
  __shared__ __attribute__((aligned(16))) uint8_t phiS[64 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t phiLoS[64 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t vS0[64 * 256];   // V of even blocks
  __shared__ __attribute__((aligned(16))) uint8_t vS1[64 * 256];   // V of odd blocks
  __shared__ float zred[16 * D];
  __shared__ float wred[4];

  const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int c = tid & 15, r0 = tid >> 4;

  float mu[8];
  {
    const f32x4 m0 = *reinterpret_cast<const f32x4*>(k_mean + (size_t)bh * D + 8 * c);
    const f32x4 m1 = *reinterpret_cast<const f32x4*>(k_mean + (size_t)bh * D + 8 * c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mu[e] = m0[e];
      mu[4 + e] = m1[e];
    }
  }
  const int mbase = 4 * (w >> 1), nbase = 4 * (w & 1);
  f32x4 hs[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) hs[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zs = 0.f;

  const int j_lo = chunk * kChunk, j_hi = min(T, j_lo + kChunk);
  // Memory goes through buffer descriptors of this head's tensors, with 32-bit offsets.  K rows
  // past N read as zeros (phase 1 zeroes their K~), so no select waits for the data here; the
  // range check covers the per-lane offset, so the row offset goes there.  The code and V^T
  // stores, always in range, keep the block offset in a scalar register.
  const __amdgpu_buffer_rsrc_t ksrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + (size_t)bh * N * D), 0, N * D * 2, 0x00020000);
  const int koff = (r0 * D + 8 * c) * 2;   // row r0 + 16 p of block j: + (64 j + 16 p) * 2D bytes
  auto load_k = [&](int j, u32x4 (&kd)[4]) {
    static_for<4>([&](auto p) {
      kd[p] = __builtin_amdgcn_raw_buffer_load_b128(ksrc, koff + (kBlock * j + 16 * p) * (2 * D), 0, 0);
    });
  };
  const int tile8 = T * kBlock * D;   // bytes of one head's e4m3 codes (K8, phi)
  const __amdgpu_buffer_rsrc_t phsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(phik8 + (size_t)bh * tile8), 0, tile8, 0x00020000);
  const int phoff = r0 * D + 32 * (c & 3) + 8 * (c >> 2);
  const __amdgpu_buffer_rsrc_t k8src = __builtin_amdgcn_make_buffer_rsrc(
      FP8 ? (void*)(k8 + (size_t)bh * tile8) : (void*)phik8, 0, FP8 ? tile8 : 0, 0x00020000);
  const int k8off = r0 * D + 8 * c;
  // V rows of this head; copies past its N rows read as zeros (the buffer's range check)
  const __amdgpu_buffer_rsrc_t vsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + (size_t)bh * N * D), 0, N * D * 2, 0x00020000);
  const int wofs = 1024 * __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's 1 KB of each 4 KB
  auto dma_v = [&](int j, uint8_t* dst) {
    static_for<4>([&](auto P) {
      // LDS chunk qd = 16 row + pc holds column chunk pc ^ rswz(row) of token 64 j + row
      const int qd = tid + 256 * P, row = qd >> 4, pc = qd & 15;
      lds_dma(vsrc, dst + 4096 * P + wofs, (kBlock * j + row) * (2 * D) + 16 * (pc ^ rswz(row)), 0);
    });
  };
  u32x4 kw[2][4];
  dma_v(j_lo, vS0);
  load_k(j_lo, kw[0]);
  if (j_lo + 1 < j_hi) load_k(j_lo + 1, kw[1]);
  // the first block needs these anyway; waiting here keeps the compiler's wait counts inside the
  // loop those of its steady state (merged with this entry, they would drain the copies in flight)
  wait_dma();

  auto block = [&](auto B, int j) {
    uint8_t* const vS = B ? vS1 : vS0;
    // ---- phase 1: K~, exp, row sums; phi (hi/lo) to LDS; z partials; block maxima
    float kt[4][8];
    bool valid[4];
    float amax = 0.f;
    float zp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zp[e] = 0.f;
    static_for<4>([&](auto p) {
      // rows past N (read as zeros) get K~ = -mu here; they are left out where it matters: the
      // block absmax and the K8 codes below take valid rows only, and their phi is zeroed by inv
      valid[p] = kBlock * j + r0 + 16 * p < N;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kt[p][2 * e] = bf16_lo(kw[B][p][e]) - mu[2 * e];
        kt[p][2 * e + 1] = bf16_hi(kw[B][p][e]) - mu[2 * e + 1];
      }
      float mx = kt[p][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, kt[p][e]);
      mx = row16_max(mx);
      const float mxl = mx * kLog2e;
      float sm = 0.f, ex[8], am = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ex[e] = __builtin_amdgcn_exp2f(fmaf(kt[p][e], kLog2e, -mxl));   // 2^((k - max) log2 e)
        sm += ex[e];
        am = fmaxf(am, fabsf(kt[p][e]));
      }
      if (valid[p]) amax = fmaxf(amax, am);
      sm = row16_sum(sm);
      const float inv = valid[p] ? 1.f / sm : 0.f;
      uint32_t pw[4], pl[4];
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = ex[2 * e] * inv, a1 = ex[2 * e + 1] * inv;
        zp[2 * e] += a0;
        zp[2 * e + 1] += a1;
        pw[e] = pack_bf16x2(a0, a1);
        pl[e] = pack_bf16x2(a0 - bf16_lo(pw[e]), a1 - bf16_hi(pw[e]));
        y[2 * e] = a0 * kPhiCodeScale;   // phi <= 1: |y| <= 448, no saturation needed
        y[2 * e + 1] = a1 * kPhiCodeScale;
      }
      const int r = r0 + 16 * p;
      *reinterpret_cast<u32x4*>(rswz_chunk(phiS, r, c)) = u32x4{pw[0], pw[1], pw[2], pw[3]};
      *reinterpret_cast<u32x4*>(rswz_chunk(phiLoS, r, c)) = u32x4{pl[0], pl[1], pl[2], pl[3]};
      // e4m3 codes of 448 phi from the fp32 values: features 8c..8c+7 = 32s + 8g' + e with
      // s = c / 4, g' = c % 4 go to bytes 32g' + 8s + e of the row
      u32x2 codes;
      codes[0] = pack_fp8x4(y[0], y[1], y[2], y[3]);
      codes[1] = pack_fp8x4(y[4], y[5], y[6], y[7]);
      __builtin_amdgcn_raw_buffer_store_b64(codes, phsrc, phoff, (kBlock * j + 16 * p) * D, 0);   // row r
    });
#pragma unroll
    for (int e = 0; e < 8; ++e) zred[r0 * D + 8 * c + e] = zp[e];
    amax = wave_max(amax);
    if (lane == 0) wred[w] = amax;
    wait_dma();   // this wave's part of block j's V (and every older load) has landed
    // barriers that only hand over LDS: a __syncthreads() here would also drain the copies
    // started below before the next block
    lds_barrier();
    // block j + 1's V into the other tile (last read before the previous barrier) and block
    // j + 2's K into the registers phase 1 just consumed.  Past the chunk's last block they copy
    // that block again (from L2; nothing reads it): every path then issues the same copies, so
    // the compiler's wait counts are those of the steady state.
    dma_v(min(j + 1, j_hi - 1), B ? vS0 : vS1);
    load_k(min(j + 2, j_hi - 1), kw[B]);

    // ---- phase 2: codes of K~ and phi, z, h tiles, V^T
    if constexpr (FP8) {
      const float bm = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
      float s = __fdiv_rn(bm, kFp8Max);
      if (s == 0.f) s = 1.f;
      if (tid == 0) k_scale[(size_t)bh * T + j] = s;
      const double inv_s = 1.0 / (double)s;
      static_for<4>([&](auto p) {
        float y[8];
#pragma unroll
        // |K~| <= bm and s = RN(bm / 448), so |y| <= 448 (1 + 2^-23), which e4m3 rounds to 448:
        // no saturation needed
        for (int e = 0; e < 8; ++e) y[e] = div_by_scale(kt[p][e], inv_s);
        u32x2 codes;
        codes[0] = valid[p] ? pack_fp8x4(y[0], y[1], y[2], y[3]) : 0u;   // pad rows: code 0
        codes[1] = valid[p] ? pack_fp8x4(y[4], y[5], y[6], y[7]) : 0u;
        __builtin_amdgcn_raw_buffer_store_b64(codes, k8src, k8off, (kBlock * j + 16 * p) * D, 0);   // row r0 + 16p
      });
    }
    if (tid < D) {
      float sz = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sz += zred[r * D + tid];
      if constexpr (STORE) z[((size_t)bh * T + j) * D + tid] = sz;
      zblk[((size_t)bh * T + j) * D + tid] = sz;
      zs += sz;
    }

    // h^T tiles on the matrix cores: D[a][c] = sum_t phi[t][a] V[t][c]
    f32x4 acc[4][4];
    if constexpr (STORE) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // operands of tokens t0 .. t0 + 7 (the contraction index, down the LDS rows)
      const int t0 = 32 * ks + 8 * g;
      bf16x8 Bv[4];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) Bv[ni] = lds_op_tr16(vS, t0, 16 * (nbase + ni), l16);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const bf16x8 Ah = lds_op_tr16(phiS, t0, 16 * (mbase + mi), l16);
        const bf16x8 Al = lds_op_tr16(phiLoS, t0, 16 * (mbase + mi), l16);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          f32x4& dst = STORE ? acc[mi][ni] : hs[mi][ni];
          dst = mfma_bf16(Al, Bv[ni], dst);
          dst = mfma_bf16(Ah, Bv[ni], dst);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (STORE) {
      // D[a = 16m + 4g + r][c = 16n + l16] -> h[j][c][a .. a+3]
      uint16_t* hj = h + ((size_t)bh * T + j) * D * D;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int a0 = 16 * (mbase + mi) + 4 * g;
          const int cc = 16 * (nbase + ni) + l16;
          u32x2 st;
          st[0] = pack_bf16x2(acc[mi][ni][0], acc[mi][ni][1]);
          st[1] = pack_bf16x2(acc[mi][ni][2], acc[mi][ni][3]);
          *reinterpret_cast<u32x2*>(hj + (size_t)cc * D + a0) = st;
          hs[mi][ni] += acc[mi][ni];
        }
    }

    if constexpr (PV8) {
      // e4m3 V of this block, transposed, one power-of-two scale per channel: row c of the tile
      // holds key 16mt + 4g + rr at byte 16g + 4mt + rr (the keys lane group g of the forward
      // holds).  Wave w, pass pp takes channels c = 16ct + l16 with ct = 4pp + w; lane group g
      // reads keys 16mt + 4g .. + 3 of its channel with the transposing reads, so the 64 keys
      // of a channel lie in the four lane groups of one wave and its absmax is a 4-row max.
      uint8_t* v8j = reinterpret_cast<uint8_t*>(vt) + ((size_t)bh * T + j) * D * kBlock;
      static_for<2>([&](auto pp) {
        const int ct = 4 * pp + w, ch = 16 * ct + l16;
        float x[16];
        static_for<4>([&](auto mt) {
          const u32x2 r4 = lds_read_tr16_rswz(vS, 16 * mt + 4 * g, 16 * ct, l16);
          x[4 * mt + 0] = bf16_lo(r4.x);
          x[4 * mt + 1] = bf16_hi(r4.x);
          x[4 * mt + 2] = bf16_lo(r4.y);
          x[4 * mt + 3] = bf16_hi(r4.y);
        });
        float am = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(x[e]));
        const int ex = v_scale_exponent(rows4_max(am));
        uint32_t wd[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)   // |x| 2^-ex <= 448: exact scaling, then round to e4m3
          wd[mt] = pack_fp8x4(__builtin_amdgcn_ldexpf(x[4 * mt], -ex), __builtin_amdgcn_ldexpf(x[4 * mt + 1], -ex),
                              __builtin_amdgcn_ldexpf(x[4 * mt + 2], -ex), __builtin_amdgcn_ldexpf(x[4 * mt + 3], -ex));
        *reinterpret_cast<u32x4*>(v8j + (size_t)ch * kBlock + 16 * g) = u32x4{wd[0], wd[1], wd[2], wd[3]};
        if (g == 0) vexp[((size_t)bh * T + j) * D + 8 * l16 + ct] = (uint8_t)(ex + 127);
      });
    } else {
      // V of this block, transposed: vt[j][c][32s + 8gg + e] = V[key][c] with
      // key = 32s + 4gg + e (e < 4) or 32s + 16 + 4gg + (e - 4) (e >= 4).  Each 16-lane group
      // takes 16 columns of one (s, gg); the four groups of a wave take gg = 0..3 of the same
      // columns, so each column receives 64 contiguous bytes per store.
      const __amdgpu_buffer_rsrc_t vtsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vt + (size_t)bh * T * D * kBlock), 0, T * D * kBlock * 2, 0x00020000);
      const int vtoff = ((16 * (w >> 1) + l16) * kBlock + 32 * (w & 1) + 8 * g) * 2;
      static_for<4>([&](auto pp) {
        const int ct = 2 * pp + (w >> 1), s = w & 1, gg = g;
        const u32x2 lo4 = lds_read_tr16_rswz(vS, 32 * s + 4 * gg, 16 * ct, l16);
        const u32x2 hi4 = lds_read_tr16_rswz(vS, 32 * s + 16 + 4 * gg, 16 * ct, l16);
        // vt[j][16 ct + l16][32 s + 8 gg ..]: the lane part in vtoff, block and pass in the scalar
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{lo4.x, lo4.y, hi4.x, hi4.y}, vtsrc, vtoff,
                                               (j * D + 32 * pp) * (kBlock * 2), 0);
      });
    }
    lds_barrier();
  };
  // pairs of blocks with no exit between them, so that the only way back to an even block is
  // through an odd one (the compiler's wait counts then assume that order); an odd count ends
  // with one more even block
  const int npair = (j_hi - j_lo) >> 1;
  for (int q = 0; q < npair; ++q) {
    block(std::integral_constant<int, 0>{}, j_lo + 2 * q);
    block(std::integral_constant<int, 1>{}, j_lo + 2 * q + 1);
  }
  if ((j_hi - j_lo) & 1) block(std::integral_constant<int, 0>{}, j_hi - 1);
  wait_dma();   // no copy into this workgroup's LDS outlives it

  float* hp = hpart + ((size_t)bh * P + chunk) * D * D;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int a0 = 16 * (mbase + mi) + 4 * g;
      const int cc = 16 * (nbase + ni) + l16;
      *reinterpret_cast<f32x4*>(hp + (size_t)cc * D + a0) = hs[mi][ni];
    }
  if (tid < D) zpart[((size_t)bh * P + chunk) * D + tid] = zs;
}

// ---------------------------------------------------------------------------------------
// fp32, d in {64, 128}: the same statistics with plain fp32 arithmetic.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void precompute_f32_kernel(
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ k_mean, int N,
    int T, int P, float* __restrict__ h, float* __restrict__ z, float* __restrict__ hpart,
    float* __restrict__ zpart) {
  constexpr int NA = D * D / 256;  // h entries per thread
  __shared__ float phiS[64 * D];
  __shared__ float vS[64 * D];
  const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int cb = tid % D, a0 = (tid / D) * NA;
  float hs[NA];
#pragma unroll
  for (int x = 0; x < NA; ++x) hs[x] = 0.f;
  float zs = 0.f;

  const int j_lo = chunk * kChunk, j_hi = min(T, j_lo + kChunk);
  for (int j = j_lo; j < j_hi; ++j) {
    for (int x = tid; x < 64 * D; x += 256) {
      const int t = x / D, col = x % D, row = kBlock * j + t;
      const bool ok = row < N;
      const size_t off = ((size_t)bh * N + row) * D + col;
      phiS[x] = ok ? k[off] - k_mean[(size_t)bh * D + col] : 0.f;
      vS[x] = ok ? v[off] : 0.f;
    }
    __syncthreads();
    // phi per token: 4 threads (one quad) per row
    {
      const int t = tid >> 2, part = tid & 3;
      const int row = kBlock * j + t;
      float* pr = phiS + t * D;
      float mx = -INFINITY;
      for (int col = part; col < D; col += 4) mx = fmaxf(mx, pr[col]);
      mx = fmaxf(mx, dpp<0xB1>(mx));
      mx = fmaxf(mx, dpp<0x4E>(mx));
      float sm = 0.f;
      for (int col = part; col < D; col += 4) sm += expf(pr[col] - mx);
      sm += dpp<0xB1>(sm);
      sm += dpp<0x4E>(sm);
      const float inv = row < N ? 1.f / sm : 0.f;
      for (int col = part; col < D; col += 4) pr[col] = expf(pr[col] - mx) * inv;
    }
    __syncthreads();
    float acc[NA];
#pragma unroll
    for (int x = 0; x < NA; ++x) acc[x] = 0.f;
    for (int t = 0; t < 64; ++t) {
      const float vv = vS[t * D + cb];
#pragma unroll
      for (int x = 0; x < NA; ++x) acc[x] = fmaf(phiS[t * D + a0 + x], vv, acc[x]);
    }
    float* hj = h + ((size_t)bh * T + j) * D * D + (size_t)cb * D + a0;
#pragma unroll
    for (int x = 0; x < NA; ++x) {
      hj[x] = acc[x];
      hs[x] += acc[x];
    }
    if (tid < D) {
      float s = 0.f;
      for (int t = 0; t < 64; ++t) s += phiS[t * D + tid];
      z[((size_t)bh * T + j) * D + tid] = s;
      zs += s;
    }
    __syncthreads();
  }
  float* hp = hpart + ((size_t)bh * P + chunk) * D * D + (size_t)cb * D + a0;
#pragma unroll
  for (int x = 0; x < NA; ++x) hp[x] = hs[x];
  if (tid < D) zpart[((size_t)bh * P + chunk) * D + tid] = zs;
}

// h_sum / z_sum: sum of the chunk partials.  A workgroup owns 256 consecutive entries (64
// quads) of one head; thread (quad q, part u) adds the partials p = u, u + 4, ... of its quad
// with 16-byte loads, then the 4 parts are combined in fixed order.
__device__ __forceinline__ void reduce_sums_block(int blk, int bh, const float* __restrict__ hpart,
                                                  const float* __restrict__ zpart, int P, int D,
                                                  float* __restrict__ h_sum, float* __restrict__ z_sum,
                                                  uint16_t* __restrict__ hbf) {
  __shared__ f32x4 red[4][64];
  const int tid = threadIdx.x;
  const int q = tid & 63, u = tid >> 6;
  const int DD = D * D;
  const int e0 = blk * 256 + 4 * q;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (e0 < DD) {
#pragma unroll 16
    for (int p = u; p < P; p += 4) acc += *reinterpret_cast<const f32x4*>(hpart + ((size_t)bh * P + p) * DD + e0);
  }
  red[u][q] = acc;
  __syncthreads();
  if (u == 0 && e0 < DD) {
    const f32x4 sm = (red[0][q] + red[1][q]) + (red[2][q] + red[3][q]);
    *reinterpret_cast<f32x4*>(h_sum + (size_t)bh * DD + e0) = sm;
    if (hbf != nullptr) {   // D = 128: 8 bf16 per 16-byte chunk, chunk k of row c at k ^ (c % 16)
      const int c = e0 / D, a = e0 % D;
      u32x2 w2;
      w2.x = pack_bf16x2(sm.x, sm.y);
      w2.y = pack_bf16x2(sm.z, sm.w);
      *reinterpret_cast<u32x2*>(hbf + (size_t)bh * DD + c * D + 8 * ((a >> 3) ^ (c & 15)) + (a & 7)) = w2;
    }
  }
  if (blk == 0) {
    // z_sum: thread (c, part v) adds partials p = v, v + 256/D, ...; parts combined in order
    __shared__ float zred[256];
    const int parts = 256 / D, c = tid % D, v = tid / D;
    float sz = 0.f;
#pragma unroll 8
    for (int p = v; p < P; p += parts) sz += zpart[((size_t)bh * P + p) * D + c];
    zred[tid] = sz;
    __syncthreads();
    if (v == 0) {
      for (int k = 1; k < parts; ++k) sz += zred[k * D + c];
      z_sum[(size_t)bh * D + c] = sz;
    }
  }
}

// The tail of the precompute: workgroup x reduces entries 256 x .. 256 x + 255 of head y's chunk
// partials (and writes the bf16 H^T image when hbf is given).  The per-row sums of z_j over the
// routed blocks are formed by the forward pass as it walks each LUT row, so this pass never reads
// the LUT.
__global__ __launch_bounds__(256) void precompute_tail_kernel(const float* __restrict__ hpart,
                                                              const float* __restrict__ zpart, int P, int D,
                                                              float* __restrict__ h_sum,
                                                              float* __restrict__ z_sum, uint16_t* __restrict__ hbf) {
  reduce_sums_block(blockIdx.x, blockIdx.y, hpart, zpart, P, D, h_sum, z_sum, hbf);
}

template <bool FP8, bool STORE, bool PV8 = false>
static void launch_precompute_bf16(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s) {
  hipLaunchKernelGGL((precompute_bf16_kernel<FP8, STORE, PV8>), dim3(g.P, g.BH), dim3(256), 0, s,
                     (const uint16_t*)t.k, (const uint16_t*)t.v, t.k_mean, g.N, g.T, g.P, t.k8, t.k_scale,
                     (uint16_t*)t.h, t.z, ws.hpart, ws.zpart, ws.vt, ws.phik8, ws.zblk, ws.vexp);
}

hipError_t launch_precompute(const Geometry& g, const sla2_tensors& t, const Workspace& ws,
                             hipStream_t s) {
  dim3 grid(g.P, g.BH);
  if (g.bf16) {
    // h_j and z_j are stored only when both buffers are given
    const bool store = t.h != nullptr && t.z != nullptr;
    if (g.pv8) {
      if (store) launch_precompute_bf16<true, true, true>(g, t, ws, s);
      else launch_precompute_bf16<true, false, true>(g, t, ws, s);
    } else if (g.fp8) {
      if (store) launch_precompute_bf16<true, true>(g, t, ws, s);
      else launch_precompute_bf16<true, false>(g, t, ws, s);
    } else {
      if (store) launch_precompute_bf16<false, true>(g, t, ws, s);
      else launch_precompute_bf16<false, false>(g, t, ws, s);
    }
  } else if (g.D == 128) {
    hipLaunchKernelGGL(precompute_f32_kernel<128>, grid, dim3(256), 0, s, (const float*)t.k,
                       (const float*)t.v, t.k_mean, g.N, g.T, g.P, (float*)t.h, t.z, ws.hpart,
                       ws.zpart);
  } else {
    hipLaunchKernelGGL(precompute_f32_kernel<64>, grid, dim3(256), 0, s, (const float*)t.k,
                       (const float*)t.v, t.k_mean, g.N, g.T, g.P, (float*)t.h, t.z, ws.hpart,
                       ws.zpart);
  }
  const int nred = (g.D * g.D + 255) / 256;
  hipLaunchKernelGGL(precompute_tail_kernel, dim3(nred, g.BH), dim3(256), 0, s, ws.hpart, ws.zpart, g.P, g.D,
                     t.h_sum, t.z_sum, g.bf16 ? ws.hbf : (uint16_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* parts, const float* zparts, int P, int D, int BH, float* out,
                            float* zout, hipStream_t s) {
  const int nred = (D * D + 255) / 256;
  hipLaunchKernelGGL(precompute_tail_kernel, dim3(nred, BH), dim3(256), 0, s, parts, zparts, P, D, out, zout,
                     (uint16_t*)nullptr);
  return hipGetLastError();
}

}  // namespace sla2
