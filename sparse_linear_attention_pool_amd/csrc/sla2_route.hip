// SLA2 router: block mean pooling of Q and K, the token mean of K (key smoothing), the
// learnable d x d projections, block scores and the row-wise hard Top-k with block-index
// compaction into an ascending LUT.  Also quantises Q to FP8 e4m3 per 64-token block.
//
// Pages: "SLA2: Sparse-Linear Attention with Learnable Routing and QAT", section 4 (mean
// pooling of consecutive Q/K blocks, proj_q and proj_k, Top-k over each row of the compressed
// scores), section 5 (Q and K quantised with scales before the scores), section 6 (key
// smoothing); "SLA: Beyond Sparsity in Diffusion Transformers...", section 2 Q2 step 1
// (compressed scores pool(Q) pool(K)^T / sqrt(d) over 64-token blocks) and section 7 (the
// token mean subtracted from K before routing).
#include <math.h>

#include "sla2_device.hpp"
#include "sla2_internal.hpp"

namespace sla2 {

// ---------------------------------------------------------------------------------------
// Pool: one workgroup per (block i, head).  Column sums of the block's Q and K rows in fp64
// (exact for bf16 inputs, so their order does not matter); in FP8 mode also the block's absmax
// scale and the e4m3 codes of Q.  Rows past N count as zero and receive code 0.
// Thread (c = tid % CPR, r0 = tid / CPR) loads the 16-byte chunk c of rows r0 + RPP p.  Its
// fp64 column partials go to LDS, where thread j then sums column j % D of Q (j < D) or K over
// the row groups.  The FP8 codes re-read the block's Q rows (from L2) once the scale is known,
// rather than holding them in registers.
// ---------------------------------------------------------------------------------------
template <typename Tin, int D, bool FP8>
__global__ __launch_bounds__(256) void pool_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   int N, int T, double* __restrict__ qsum,
                                                   double* __restrict__ ksum, uint8_t* __restrict__ q8,
                                                   float* __restrict__ q_scale) {
  constexpr int VEC = 16 / sizeof(Tin);  // elements per 16-byte chunk
  constexpr int CPR = D / VEC;           // chunks per row
  constexpr int RPP = 256 / CPR;         // rows per pass (= row groups)
  constexpr int PASSES = kBlock / RPP;
  static_assert(!FP8 || VEC == 8, "FP8 quantisation needs bf16 input");
  static_assert(2 * D <= 256, "one thread per column of Q and of K");
  __shared__ double part[2][RPP][D];   // column partials of each row group (32 KB at D = 128, bf16)
  __shared__ float wmax[4];

  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = tid % CPR, r0 = tid / CPR;
  const size_t head = (size_t)bh * N;

  double qs[VEC], ks[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) qs[e] = ks[e] = 0.0;
  float amax = 0.f;

  u32x4 qw[PASSES], kw[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = kBlock * i + r0 + p * RPP;
    const bool ok = row < N;
    const size_t off = (head + (ok ? row : 0)) * D + c * VEC;
    const u32x4 a = *reinterpret_cast<const u32x4*>(q + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(k + off);
    qw[p] = ok ? a : u32x4{0, 0, 0, 0};
    kw[p] = ok ? b : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float qv[VEC], kv[VEC];
    if constexpr (sizeof(Tin) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[2 * e] = bf16_lo(qw[p][e]);
        qv[2 * e + 1] = bf16_hi(qw[p][e]);
        kv[2 * e] = bf16_lo(kw[p][e]);
        kv[2 * e + 1] = bf16_hi(kw[p][e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[e] = __uint_as_float(qw[p][e]);
        kv[e] = __uint_as_float(kw[p][e]);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      qs[e] += (double)qv[e];
      ks[e] += (double)kv[e];
      amax = fmaxf(amax, fabsf(qv[e]));
    }
  }

  // column sums: each row group's partials to LDS, then one thread per (tensor, column).
  // Column x of a row group sits at slot pslot(x): its 16-byte pair index XORed with bits 4-5
  // of itself, so that the 16 lanes of a row group writing their 64-byte runs, and 32 lanes
  // reading consecutive columns, each hit distinct banks.
  auto pslot = [](int x) { const int pr = x >> 1; return 2 * (pr ^ ((pr >> 4) & 3)) + (x & 1); };
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    part[0][r0][pslot(c * VEC + e)] = qs[e];
    part[1][r0][pslot(c * VEC + e)] = ks[e];
  }
  __syncthreads();
  {
    const int which = tid / D, col = tid % D;
    if (which < 2) {
      double sm = 0.0;
#pragma unroll
      for (int rg = 0; rg < RPP; ++rg) sm += part[which][rg][pslot(col)];
      (which ? ksum : qsum)[((size_t)bh * T + i) * D + col] = sm;
    }
  }

  if constexpr (FP8) {
    const float wm = wave_max(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = wm;
    __syncthreads();
    const float bm = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    float s = __fdiv_rn(bm, kFp8Max);
    if (s == 0.f) s = 1.f;
    if (tid == 0) q_scale[(size_t)bh * T + i] = s;
    const double inv_s = 1.0 / (double)s;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = kBlock * i + r0 + p * RPP;
      const bool ok = row < N;
      const u32x4 a = *reinterpret_cast<const u32x4*>(q + (head + (ok ? row : 0)) * D + c * VEC);
      const u32x4 w4 = ok ? a : u32x4{0, 0, 0, 0};   // rows past N: code 0
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[2 * e] = clamp_fp8(div_by_scale(bf16_lo(w4[e]), inv_s));
        y[2 * e + 1] = clamp_fp8(div_by_scale(bf16_hi(w4[e]), inv_s));
      }
      u32x2 codes;
      codes.x = pack_fp8x4(y[0], y[1], y[2], y[3]);
      codes.y = pack_fp8x4(y[4], y[5], y[6], y[7]);
      *reinterpret_cast<u32x2*>(q8 + ((size_t)bh * T * kBlock + row) * D + c * 8) = codes;
    }
  }
}

// Partial sums of the K block sums over 32 consecutive blocks: kpart [BH, ceil(T/32), D].
template <int D>
__global__ __launch_bounds__(D) void kpart_kernel(const double* __restrict__ ksum, int T,
                                                  double* __restrict__ kpart) {
  const int p = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const int P32 = (T + 31) / 32;
  double s = 0.0;
  const int lo = 32 * p, hi = min(T, lo + 32);
#pragma unroll 32
  for (int i = lo; i < hi; ++i) s += ksum[((size_t)bh * T + i) * D + c];
  kpart[((size_t)bh * P32 + p) * D + c] = s;
}

// ---------------------------------------------------------------------------------------
// Project: one workgroup per (16 blocks, head, Q or K), 256 threads.
// mu = (sum of all K) / N; q_bar = block mean of Q; k_bar = block mean of K - mu;
// q_hat = q_bar W_q, k_hat = k_bar W_k in fp64 (W NULL = identity) on the fp64 matrix cores.
// Wave w computes the 16 x 16 output tiles of columns 16 ct .. 16 ct + 15, ct = w, w + 4, ...
// For K the transposed tile k_hat^T = W_k^T k_bar^T is formed (the same two operands in
// swapped roles), so both outputs are stored in 128-byte rows.
// ---------------------------------------------------------------------------------------
constexpr int kProjRows = 16;

template <int D>
__global__ __launch_bounds__(256) void project_kernel(
    const double* __restrict__ qsum, const double* __restrict__ ksum, const double* __restrict__ kpart,
    int N, int T, int smooth_k, const float* __restrict__ wq, const float* __restrict__ wk,
    float* __restrict__ q_pool, float* __restrict__ k_pool, float* __restrict__ k_mean,
    double* __restrict__ mu_out, double* __restrict__ qhat, double* __restrict__ khatT) {
  constexpr int R = kProjRows;
  constexpr int KS = D / 4;   // matrix-core steps over the input channel
  __shared__ double mu_s[D];
  __shared__ double rows[R][D + 1];
  const int bh = blockIdx.y, i0 = blockIdx.x * R, which = blockIdx.z, tid = threadIdx.x;
  const int P32 = (T + 31) / 32;

  if (which == 1 && tid < D) {
    double sm = 0.0;
    for (int p = 0; p < P32; ++p) sm += kpart[((size_t)bh * P32 + p) * D + tid];
    const double m = smooth_k ? sm / (double)N : 0.0;
    mu_s[tid] = m;
    if (blockIdx.x == 0) {
      k_mean[(size_t)bh * D + tid] = (float)m;
      mu_out[(size_t)bh * D + tid] = m;
    }
  }
  __syncthreads();
  for (int x = tid; x < R * D; x += 256) {
    const int r = x / D, c = x % D, i = i0 + r;
    double v = 0.0;
    if (i < T) {
      const int n = min(kBlock, N - kBlock * i);
      const size_t idx = ((size_t)bh * T + i) * D + c;
      if (which == 0) {
        v = qsum[idx] / (double)n;
        q_pool[idx] = (float)v;
      } else {
        v = ksum[idx] / (double)n - mu_s[c];
        k_pool[idx] = (float)v;
      }
    }
    rows[r][c] = v;
  }
  __syncthreads();

  const float* W = which ? wk : wq;
  const int w = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;
  if (W == nullptr) {
    for (int x = tid; x < R * D; x += 256) {
      if (which == 0) {
        const int r = x / D, c = x % D;
        if (i0 + r < T) qhat[((size_t)bh * T + i0 + r) * D + c] = rows[r][c];
      } else {
        const int c = x / R, r = x % R;
        if (i0 + r < T) khatT[((size_t)bh * D + c) * T + i0 + r] = rows[r][c];
      }
    }
    return;
  }
  double xa[KS];   // pooled row li, input channels 4s + lk
  static_for<KS>([&](auto s) { xa[s] = rows[li][4 * s + lk]; });
  for (int ct = w; ct < D / 16; ct += 4) {
    double wb[KS];   // W[4s + lk][16 ct + li]
    static_for<KS>([&](auto s) { wb[s] = (double)W[(4 * s + lk) * D + 16 * ct + li]; });
    f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
    if (which == 0) {
      static_for<KS>([&](auto s) { acc = mfma_f64(xa[s], wb[s], acc); });
      // acc[r] = q_hat[i0 + 4 r + lk][16 ct + li]
      static_for<4>([&](auto r) {
        const int i = i0 + 4 * r + lk;
        if (i < T) qhat[((size_t)bh * T + i) * D + 16 * ct + li] = acc[int(r)];
      });
    } else {
      static_for<KS>([&](auto s) { acc = mfma_f64(wb[s], xa[s], acc); });
      // acc[r] = k_hat[i0 + li][16 ct + 4 r + lk]
      if (i0 + li < T) {
        static_for<4>([&](auto r) { khatT[((size_t)bh * D + 16 * ct + 4 * r + lk) * T + i0 + li] = acc[int(r)]; });
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// SoftTop-k router mask (SLA2 page, section 4: for training the row's hard Top-k is replaced
// by SoftTop-k, which keeps its row sum; section 6: a sigmoid with temperature tau and a
// per-row offset lambda_i found by binary search so that each row sums to the Top-k count).
// Input: P_c = softmax over the row of the router scores s_ij (SLA page, section 2 Q2 step 1),
// the scores the hard Top-k ranks.  M_ij = sigmoid((P_ij - lambda_i) / tau).  lambda_i is the
// root of sum_j sigmoid((P_ij - lambda) / tau) = k_sel in [min P - tau (ln T + 2), max P +
// tau (ln T + 2)] (row sum above T - 1 at the lower end, below 1 at the upper end).  The
// bracket is kept as in a binary search, halved on the side where the row sum crosses
// k_sel; each step tries the Newton point of the (strictly decreasing) row sum and takes it
// when it falls inside the bracket, else the midpoint.  It stops after a Newton step below
// 2^-30 of lambda (the point it lands on is then within about 2^-60), when the bracket is at
// the rounding level, or after kSoftSteps steps: the root that kSoftSteps plain halvings reach
// (to 2^-kSoftSteps of the bracket), in a few steps.  The fp64 search starts from the point
// the same search finds in fp32, which is cheap and close.
// k_sel = T gives M = 1 and lambda = -inf.  Lane l holds the columns j = l + 64 m of a row;
// fp64 throughout, like the hard router.
// ---------------------------------------------------------------------------------------
constexpr int kSoftSteps = 60;

// Sum over the wave, then lane 0's value on every lane: a branch on the result is then
// uniform even though the butterfly adds in a different order on each lane.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return __shfl(v, 0);
}
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;   // exact, so every lane holds the same value
}
__device__ __forceinline__ double wave_min_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmin(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double sigmoid_f64(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

// One row of the soft mask from its scores p[] (fp64, lane l holds columns l + 64 m).
template <int MAXS>
__device__ __forceinline__ void soft_row(double (&p)[MAXS], int T, int topk, double inv_sqrt_d, double tau,
                                         float* __restrict__ mrow, float* __restrict__ lam_out, int lane) {
  // P_c: softmax over the row's T columns
  double mx = -INFINITY;
  static_for<MAXS>([&](auto m) {
    p[m] *= inv_sqrt_d;
    if (64 * m + lane < T) mx = fmax(mx, p[m]);
  });
  mx = wave_max_f64(mx);
  double z = 0.0;
  static_for<MAXS>([&](auto m) {
    p[m] = 64 * m + lane < T ? exp(p[m] - mx) : 0.0;
    z += p[m];
  });
  z = wave_sum_f64(z);
  double pmin = INFINITY, pmax = -INFINITY;
  static_for<MAXS>([&](auto m) {
    p[m] /= z;
    if (64 * m + lane < T) {
      pmin = fmin(pmin, p[m]);
      pmax = fmax(pmax, p[m]);
    }
  });
  pmin = wave_min_f64(pmin);
  pmax = wave_max_f64(pmax);

  double lam = -INFINITY;
  if (topk < T) {
    const double pad = tau * (log((double)T) + 2.0), itau = 1.0 / tau, k = (double)topk;
    double lo = pmin - pad, hi = pmax + pad, x = 0.5 * (lo + hi);
    {
      // a start near the root from the same search in fp32 (about 1e-7 relative)
      const float itf = (float)itau, kf = (float)topk;
      float lof = (float)lo, hif = (float)hi, xf = (float)x;
      float pf[MAXS];
      static_for<MAXS>([&](auto m) { pf[m] = (float)p[m]; });
      for (int it = 0; it < kSoftSteps; ++it) {
        float f = 0.f, df = 0.f;
        static_for<MAXS>([&](auto m) {
          if (64 * m + lane < T) {
            const float sg = 1.f / (1.f + __expf((xf - pf[m]) * itf));
            f += sg;
            df += sg - sg * sg;
          }
        });
        f = __shfl(wave_sum(f), 0);   // lane 0's value everywhere: the steps below are uniform
        df = __shfl(wave_sum(df), 0) * itf;
        if (f > kf) lof = xf;
        else hif = xf;
        if (f == kf) break;
        float xn = xf + (f - kf) / df;
        if (!(df > 0.f) || !(xn > lof && xn < hif)) xn = 0.5f * (lof + hif);
        const bool done = fabsf(xn - xf) <= 0x1p-18f * fabsf(xn) || hif - lof <= 0x1p-21f * fmaxf(fabsf(lof), fabsf(hif));
        xf = xn;
        if (done) break;
      }
      if ((double)xf > lo && (double)xf < hi) x = (double)xf;
    }
    for (int it = 0; it < kSoftSteps; ++it) {
      // row sum f(x) and its slope -f'(x) = sum sigma (1 - sigma) / tau
      double f = 0.0, df = 0.0;
      static_for<MAXS>([&](auto m) {
        if (64 * m + lane < T) {
          const double sg = sigmoid_f64((p[m] - x) * itau);
          f += sg;
          df += sg - sg * sg;
        }
      });
      f = wave_sum_f64(f);   // identical on every lane: the steps below are uniform
      df = wave_sum_f64(df) * itau;
      if (f > k) lo = x;     // row sum too large: the offset must grow
      else hi = x;
      if (f == k) break;
      double xn = x + (f - k) / df;
      if (!(df > 0.0) || !(xn > lo && xn < hi)) xn = 0.5 * (lo + hi);
      // a Newton step this small leaves an error about its square (the row sum's own rounding
      // keeps later steps near 1e-16 relative, so a test at the rounding level would not stop)
      const bool done = fabs(xn - x) <= 0x1p-30 * fabs(xn) || hi - lo <= 0x1p-52 * fmax(fabs(lo), fabs(hi));
      x = xn;
      if (done) break;
    }
    lam = x;
  }
  static_for<MAXS>([&](auto m) {
    const int j = 64 * m + lane;
    if (j < T) mrow[j] = topk < T ? (float)sigmoid_f64((p[m] - lam) / tau) : 1.f;
  });
  if (lane == 0) *lam_out = (float)lam;
}

// ---------------------------------------------------------------------------------------
// Scores + Top-k: one workgroup per (R query blocks, head), 256 threads.
//
// Phase 1: scores q_hat k_hat^T / sqrt(d) in fp64 on the matrix cores.  The A operand is the
// 16 x D tile of q_hat rows (rows past R repeat earlier rows and are discarded); wave w takes
// the 16-key tiles tt = w, w + 4, ..., loading the k_hat operand one half tile (D/2 channels)
// ahead of the multiplies.  The scores are stored in LDS as order-preserving 64-bit keys.
//
// Phase 2: one wave per row.  The topk-th largest key is found by a bitwise binary search:
// bit by bit from the top, a candidate threshold is kept when at least topk keys reach it
// (counted with ballots); the search stops as soon as exactly topk keys reach the threshold.
// The high 32 bits are searched first; the low 32 bits only when the high halves tie.
// Keys equal to the final threshold are taken in increasing j until topk are chosen, which
// gives the lower block index on ties.  The mask row and the ascending LUT row follow by
// ballot compaction.
//
// Phase 3 (SOFT, for sla2_route_soft): one wave per row, the SoftTop-k mask and lambda of the
// row (soft_row above) from the same fp64 scores, read back from LDS.
// ---------------------------------------------------------------------------------------

// Order-preserving map of a double to an unsigned key (-0.0 is taken as +0.0).
__device__ __forceinline__ uint64_t score_key(double v) {
  uint64_t u = __double_as_longlong(v);
  if (u == 0x8000000000000000ull) u = 0;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ int ballot_count(bool p) {
  return __popcll(__builtin_amdgcn_ballot_w64(p));
}

// The score a key was made from (score_key is a bijection onto its range).
__device__ __forceinline__ double key_score(uint64_t key) {
  const uint64_t u = (key >> 63) ? (key & 0x7fffffffffffffffull) : ~key;
  return __longlong_as_double((long long)u);
}

// NW waves per workgroup: 4, or 8 where the keys of one workgroup fill most of the LDS (so
// that the CU still runs two waves per SIMD).
template <int R, int MAXS, int D, bool SOFT, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void topk_kernel(const double* __restrict__ qhat,
                                                      const double* __restrict__ khatT, int T, int topk,
                                                      double inv_sqrt_d, int32_t* __restrict__ lut,
                                                      uint8_t* __restrict__ mask, double tau,
                                                      float* __restrict__ soft_mask, float* __restrict__ lambda) {
  constexpr int KS = D / 4;    // matrix-core steps over the channels
  constexpr int HS = KS / 2;   // steps per half tile
  extern __shared__ uint64_t keys_s[];   // [R][T]
  // consecutive row blocks of a head run on one XCD, which then holds that head's k_hat in L2
  const int nrb = gridDim.x;
  const int lid = xcd_remap(blockIdx.x + nrb * blockIdx.y, nrb * gridDim.y);
  const int bh = lid / nrb, i0 = (lid % nrb) * R, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  {
    const int li = lane & 15, lk = lane >> 4;
    const int arow = min(i0 + li % R, T - 1);
    const double* qrow = qhat + ((size_t)bh * T + arow) * D + lk;
    double qa[KS];
    static_for<KS>([&](auto s) { qa[s] = qrow[4 * s]; });
    const double* kb = khatT + ((size_t)bh * D + lk) * T;
    const int ntiles = (T + 15) >> 4;
    // half tiles: the k_hat operand of steps half*HS .. half*HS + HS - 1 of key tile tt
    double kv[2][HS];
    auto load_half = [&](double(&dst)[HS], int tt, int half) {
      const int j = min(16 * tt + li, T - 1);
      static_for<HS>([&](auto s) { dst[s] = kb[(size_t)(4 * (half * HS + s)) * T + j]; });
    };
    if (w < ntiles) load_half(kv[0], w, 0);
    for (int tt = w; tt < ntiles; tt += NW) {
      load_half(kv[1], tt, 1);
      // two accumulators (even / odd steps) keep two independent chains in flight
      f64x4 acc0 = f64x4{0.0, 0.0, 0.0, 0.0}, acc1 = acc0;
      static_for<HS / 2>([&](auto s) {
        acc0 = mfma_f64(qa[2 * s], kv[0][2 * s], acc0);
        acc1 = mfma_f64(qa[2 * s + 1], kv[0][2 * s + 1], acc1);
      });
      if (tt + NW < ntiles) load_half(kv[0], tt + NW, 0);
      static_for<HS / 2>([&](auto s) {
        acc0 = mfma_f64(qa[HS + 2 * s], kv[1][2 * s], acc0);
        acc1 = mfma_f64(qa[HS + 2 * s + 1], kv[1][2 * s + 1], acc1);
      });
      const f64x4 acc = acc0 + acc1;
      const int j = 16 * tt + li;
      static_for<4>([&](auto r) {
        const int row = 4 * r + lk;   // accumulator r holds tile row 4r + lane/16
        if (row < R && j < T) keys_s[row * T + j] = score_key(acc[int(r)] * inv_sqrt_d);
      });
    }
  }
  __syncthreads();

  const uint64_t lt_mask = (1ull << lane) - 1ull;

  // Finish row r from the threshold found on the high halves: search the low halves when the
  // high halves tie at the boundary, then emit the LUT and mask rows.
  auto finish_row = [&](int r, uint32_t thr_hi, bool exact) {
    uint64_t key[MAXS];
    static_for<MAXS>([&](auto s) {
      const int j = 64 * s + lane;
      key[s] = j < T ? keys_s[r * T + j] : 0ull;   // 0 is below every score key
    });
    uint64_t thr = (uint64_t)thr_hi << 32;
    if (!exact) {
      // low 32 bits among the keys whose high half equals thr_hi; keys above it count as base
      int base_cnt = 0;
      uint32_t lo[MAXS];
      static_for<MAXS>([&](auto s) {
        const uint32_t hs = (uint32_t)(key[s] >> 32);
        base_cnt += ballot_count(hs > thr_hi);
        lo[s] = hs == thr_hi ? (uint32_t)key[s] : 0u;   // 0 never reaches a candidate
      });
      uint32_t thr_lo = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr_lo | (1u << bit);
        uint64_t bl[MAXS];
        static_for<MAXS>([&](auto s) { bl[s] = __builtin_amdgcn_ballot_w64(lo[s] >= cand); });
        int cnt = base_cnt;
        static_for<MAXS>([&](auto s) { cnt += __popcll(bl[s]); });
        if (cnt >= topk) {
          thr_lo = cand;
          if (cnt == topk) break;
        }
      }
      thr |= thr_lo;
    }
    // keys above thr are all taken; keys equal to thr fill the rest in increasing j
    int need = topk;
    static_for<MAXS>([&](auto s) { need -= ballot_count(key[s] > thr); });
    const size_t row = (size_t)bh * T + i0 + r;
    int base = 0;
    static_for<MAXS>([&](auto s) {
      const int j = 64 * s + lane;
      const uint64_t eq = __builtin_amdgcn_ballot_w64(key[s] == thr);
      const int n_eq = __popcll(eq);
      const int take = n_eq < need ? n_eq : need;
      const bool on = key[s] > thr || (key[s] == thr && __popcll(eq & lt_mask) < take);
      need -= take;
      const uint64_t bmask = __builtin_amdgcn_ballot_w64(on);
      if (on) lut[row * topk + base + __popcll(bmask & lt_mask)] = j;
      base += __popcll(bmask);
      if (j < T) mask[row * T + j] = on ? 1 : 0;
    });
  };

  // J rows of a wave are searched together, so that their independent steps overlap.
  constexpr int J = (MAXS <= 8) ? R / NW : 1;
  static_assert(J >= 1, "at least one row per wave");
  for (int r0 = w * J; r0 < R; r0 += NW * J) {
    uint32_t hi[J][MAXS];
    uint32_t thr[J];
    bool done[J];
    static_for<J>([&](auto jj) {
      const int r = r0 + jj;
      static_for<MAXS>([&](auto s) {
        const int j = 64 * s + lane;
        hi[jj][s] = (j < T && i0 + r < T) ? (uint32_t)(keys_s[r * T + j] >> 32) : 0u;
      });
      thr[jj] = 0;
      done[jj] = i0 + r >= T;   // rows past T are skipped
    });
    // Largest high-half threshold reached by at least topk keys; a row is done once exactly
    // topk keys reach its threshold (all ballots of a step are formed before they are counted).
    for (int bit = 31; bit >= 0; --bit) {
      bool all = true;
      static_for<J>([&](auto jj) {
        const uint32_t cand = thr[jj] | (1u << bit);
        uint64_t bl[MAXS];
        static_for<MAXS>([&](auto s) { bl[s] = __builtin_amdgcn_ballot_w64(hi[jj][s] >= cand); });
        int cnt = 0;
        static_for<MAXS>([&](auto s) { cnt += __popcll(bl[s]); });
        const bool take = !done[jj] && cnt >= topk;
        thr[jj] = take ? cand : thr[jj];
        done[jj] = done[jj] || (take && cnt == topk);
        all = all && done[jj];
      });
      if (all) break;
    }
    static_for<J>([&](auto jj) {
      const int r = r0 + jj;
      if (i0 + r < T) {
        // a row left undone after bit 0 ties in its high halves at the boundary
        finish_row(r, thr[jj], done[jj]);
      }
    });
  }

  if constexpr (SOFT) {
    for (int r = w; r < R; r += NW) {
      if (i0 + r >= T) break;
      double p[MAXS];
      static_for<MAXS>([&](auto s) {
        const int j = 64 * s + lane;
        p[s] = j < T ? key_score(keys_s[r * T + j]) : 0.0;   // already divided by sqrt(d)
      });
      const size_t row = (size_t)bh * T + i0 + r;
      soft_row<MAXS>(p, T, topk, 1.0, tau, soft_mask + row * T, lambda + row, lane);
    }
  }
}

// LDS for the score keys of one workgroup: R rows of T keys.
constexpr size_t kTopkLdsBudget = 160 * 1024;

// Soft-mask arguments of the fused SoftTop-k phase (unused by the plain router).
struct SoftOut {
  double tau;
  float* mask;
  float* lambda;
};

template <int R, int MAXS, int D, bool SOFT, int NW = 4>
static void launch_topk_s(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const SoftOut& so,
                          hipStream_t s) {
  const size_t lds = (size_t)R * g.T * sizeof(uint64_t);
  static bool attr_set = false;   // dynamic LDS above the 64 KB default
  if (!attr_set) {
    hipFuncSetAttribute((const void*)topk_kernel<R, MAXS, D, SOFT, NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)kTopkLdsBudget);
    attr_set = true;
  }
  dim3 grid((g.T + R - 1) / R, g.BH);
  hipLaunchKernelGGL((topk_kernel<R, MAXS, D, SOFT, NW>), grid, dim3(64 * NW), lds, s, ws.qhat, ws.khatT, g.T, g.topk,
                     1.0 / sqrt((double)g.D), t.lut, t.mask, so.tau, so.mask, so.lambda);
}

// Rows per workgroup R: 16 (one matrix-core tile) when the keys fit in the LDS budget, else
// 8 or 4.  Candidate slots per lane MAXS: the smallest of 4, 8, 16, 24, 32, 64 that is at
// least ceil(T / 64).  T <= 4096 leaves the pairs below.  The hard tiers whose keys allow one
// workgroup per CU (16 rows above 8 slots, and 8 rows) run 8 waves per workgroup; the soft
// phase keeps 4 waves and 8 rows, which ran faster.
template <int D, bool SOFT>
static void launch_topk(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const SoftOut& so,
                        hipStream_t s) {
  int R = 16;
  while (R > 4 && (size_t)R * g.T * sizeof(uint64_t) > kTopkLdsBudget) R >>= 1;
  const int S = (g.T + 63) / 64;
  // the soft phase runs long fp64 chains per row: above 8 slots per lane, 8 rows per workgroup
  // leave room for two workgroups per CU
  if (SOFT && S > 8 && R > 8) R = 8;
  if (R == 16 && S <= 4) launch_topk_s<16, 4, D, SOFT>(g, t, ws, so, s);
  else if (R == 16 && S <= 8) launch_topk_s<16, 8, D, SOFT>(g, t, ws, so, s);
  else if (R == 16 && S <= 16) launch_topk_s<16, 16, D, SOFT, 8>(g, t, ws, so, s);
  else if (R == 16) launch_topk_s<16, 24, D, SOFT, 8>(g, t, ws, so, s);   // 16 rows fit only T <= 1280: S <= 20
  else if (R == 8 && S <= 16) launch_topk_s<8, 16, D, SOFT>(g, t, ws, so, s);
  else if (R == 8 && S <= 24) launch_topk_s<8, 24, D, SOFT, SOFT ? 4 : 8>(g, t, ws, so, s);
  else if (R == 8 && S <= 32) launch_topk_s<8, 32, D, SOFT, SOFT ? 4 : 8>(g, t, ws, so, s);
  else if constexpr (SOFT) launch_topk_s<4, 64, D, SOFT>(g, t, ws, so, s);   // 8 rows would spill
  else if (R == 8) launch_topk_s<8, 64, D, SOFT, 8>(g, t, ws, so, s);
  else launch_topk_s<4, 64, D, SOFT>(g, t, ws, so, s);
}

template <typename Tin, int D>
static void launch_route_typed(const Geometry& g, const sla2_tensors& t, const Workspace& ws,
                               hipStream_t s) {
  dim3 grid(g.T, g.BH);
  if (g.fp8) {
    if constexpr (sizeof(Tin) == 2)
      hipLaunchKernelGGL((pool_kernel<Tin, D, true>), grid, dim3(256), 0, s, (const Tin*)t.q,
                         (const Tin*)t.k, g.N, g.T, ws.qsum, ws.ksum, t.q8, t.q_scale);
  } else {
    hipLaunchKernelGGL((pool_kernel<Tin, D, false>), grid, dim3(256), 0, s, (const Tin*)t.q,
                       (const Tin*)t.k, g.N, g.T, ws.qsum, ws.ksum, (uint8_t*)nullptr, (float*)nullptr);
  }
  const int P32 = (g.T + 31) / 32;
  hipLaunchKernelGGL(kpart_kernel<D>, dim3(P32, g.BH), dim3(D), 0, s, ws.ksum, g.T, ws.mu);
  // ws.mu first holds the 32-block partials; the projection kernel reads them and writes
  // the final mean into the tail of the same region.
  double* mu_final = ws.mu + (size_t)g.BH * P32 * D;
  hipLaunchKernelGGL(project_kernel<D>, dim3((g.T + kProjRows - 1) / kProjRows, g.BH, 2), dim3(256), 0, s, ws.qsum,
                     ws.ksum, ws.mu, g.N, g.T, (int)g.smooth_k, t.wq, t.wk, t.q_pool, t.k_pool,
                     t.k_mean, mu_final, ws.qhat, ws.khatT);
}

// Pooling, projections, then the Top-k kernel (with the SoftTop-k phase when SOFT).
template <bool SOFT>
static hipError_t route(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const SoftOut& so,
                        hipStream_t s) {
  if (g.bf16) {
    launch_route_typed<uint16_t, 128>(g, t, ws, s);   // bf16 inputs have d = 128
  } else {
    if (g.D == 128) launch_route_typed<float, 128>(g, t, ws, s);
    else launch_route_typed<float, 64>(g, t, ws, s);
  }
  if (g.D == 128) launch_topk<128, SOFT>(g, t, ws, so, s);
  else launch_topk<64, SOFT>(g, t, ws, so, s);
  return hipGetLastError();
}

hipError_t launch_route_soft(const Geometry& g, const sla2_tensors& t, const Workspace& ws, double tau,
                             float* soft_mask, float* lambda, hipStream_t s) {
  return route<true>(g, t, ws, SoftOut{tau, soft_mask, lambda}, s);
}

hipError_t launch_route(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s) {
  return route<false>(g, t, ws, SoftOut{0.0, nullptr, nullptr}, s);
}

}  // namespace sla2
