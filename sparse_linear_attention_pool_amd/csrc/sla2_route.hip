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
// the row groups.  The FP8 codes come from the block's Q rows still held in registers as packed
// bf16 (16 VGPRs): re-reading them once the scale was known missed L2 for a third of the rows
// while the rest of the inputs streamed through.
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
      const u32x4 w4 = qw[p];   // rows past N hold 0: code 0
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
// Wave w computes the 16 x 16 output tiles of columns 16 ct .. 16 ct + 15, ct = w + 4 t; at
// d = 128 its two tiles run as two interleaved multiply chains.  Step s of lane group lk
// takes input channel (d/4) lk + s, so a lane's W operand is a run of consecutive rows of W.
// For K the transposed tile k_hat^T = W_k^T k_bar^T is formed (the same two operands in
// swapped roles), so both outputs are stored in 128-byte rows.
// Every load is issued before the arithmetic that waits on it: the block sums, the W operand
// and (for K) the 32-block partials of the token sum, which are then added in increasing
// order.  Three workgroups fit on a CU, so the whole grid of a 12-head layer is resident.
// ---------------------------------------------------------------------------------------
constexpr int kProjRows = 16;

// A W element widened to fp64 where it is used: the empty asm keeps the compiler from
// widening all of them as soon as they load (twice the registers, which then spill).
__device__ __forceinline__ double w_at_use(float x) {
  asm volatile("" : "+v"(x));
  return (double)x;
}

template <int D>
__global__ __launch_bounds__(256, 3) void project_kernel(
    const double* __restrict__ qsum, const double* __restrict__ ksum, const double* __restrict__ kpart,
    int N, int T, int smooth_k, const float* __restrict__ wq, const float* __restrict__ wk,
    float* __restrict__ q_pool, float* __restrict__ k_pool, float* __restrict__ k_mean,
    double* __restrict__ mu_out, double* __restrict__ qhat, double* __restrict__ khatT) {
  constexpr int R = kProjRows;
  constexpr int KS = D / 4;          // matrix-core steps over the input channel
  constexpr int CT = D / 64;         // output tiles per wave
  constexpr int EPT = R * D / 256;   // pooled elements per thread
  constexpr int PB = 16;             // token-sum partials loaded per batch
  // pooled rows in LDS: channel c of row r at r * RP + (c / KS) * (KS + 1) + c % KS, so that the
  // 16 rows and the lane groups' runs of KS channels read in one step fall in distinct banks
  constexpr int RP = D == 128 ? 134 : 70;
  static_assert(4 * (KS + 1) <= RP, "row pitch holds the padded runs");
  auto rix = [](int r, int c) { return r * RP + (c / KS) * (KS + 1) + c % KS; };
  __shared__ double mu_s[D];
  __shared__ double rows[R * RP];
  const int bh = blockIdx.y, i0 = blockIdx.x * R, which = blockIdx.z, tid = threadIdx.x;
  const int P32 = (T + 31) / 32;
  const double* __restrict__ sums = which ? ksum : qsum;
  const float* W = which ? wk : wq;
  const int w = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;

  // block sums of this workgroup's rows: element x = tid + 256 e is row x / D, channel x % D
  double bs[EPT];
  static_for<EPT>([&](auto e) {
    const int x = tid + 256 * e, i = min(i0 + x / D, T - 1);
    bs[e] = sums[((size_t)bh * T + i) * D + x % D];
  });
  // W operand of both tiles: W[KS lk + s][16 ct + li]
  float wf[CT][KS];
  if (W != nullptr) {
    static_for<CT>([&](auto t) {
      static_for<KS>([&](auto s) { wf[t][s] = W[(KS * lk + s) * D + 16 * (w + 4 * t) + li]; });
    });
  }
  if (which == 1 && tid < D) {
    double sm = 0.0;
    for (int p0 = 0; p0 < P32; p0 += PB) {
      double v[PB];
      static_for<PB>([&](auto u) { v[u] = kpart[((size_t)bh * P32 + min(p0 + (int)u, P32 - 1)) * D + tid]; });
      static_for<PB>([&](auto u) {
        if (p0 + (int)u < P32) sm += v[u];
      });
    }
    const double m = smooth_k ? sm / (double)N : 0.0;
    mu_s[tid] = m;
    if (blockIdx.x == 0) {
      k_mean[(size_t)bh * D + tid] = (float)m;
      mu_out[(size_t)bh * D + tid] = m;
    }
  }
  __syncthreads();
  static_assert(256 % D == 0, "every element of a thread is in channel tid % D");
  const int c = tid % D;
  const double muc = which ? mu_s[c] : 0.0;
  static_for<EPT>([&](auto e) {
    const int r = (tid + 256 * e) / D, i = i0 + r;
    double v = 0.0;
    if (i < T) {
      const int n = min(kBlock, N - kBlock * i);
      const size_t idx = ((size_t)bh * T + i) * D + c;
      if (which == 0) {
        v = bs[e] / (double)n;
        q_pool[idx] = (float)v;
      } else {
        v = bs[e] / (double)n - muc;
        k_pool[idx] = (float)v;
      }
    }
    rows[rix(r, c)] = v;
  });
  __syncthreads();

  if (W == nullptr) {
    for (int x = tid; x < R * D; x += 256) {
      if (which == 0) {
        const int r = x / D, c = x % D;
        if (i0 + r < T) qhat[((size_t)bh * T + i0 + r) * D + c] = rows[rix(r, c)];
      } else {
        const int c = x / R, r = x % R;
        if (i0 + r < T) khatT[((size_t)bh * D + c) * T + i0 + r] = rows[rix(r, c)];
      }
    }
    return;
  }
  // the pooled-row operand (row li, input channel KS lk + s) is read from LDS at each step
  f64x4 acc[CT];
  static_for<CT>([&](auto t) { acc[t] = f64x4{0.0, 0.0, 0.0, 0.0}; });
  if (which == 0) {
    static_for<KS>([&](auto s) {
      const double xa = rows[li * RP + lk * (KS + 1) + s];
      static_for<CT>([&](auto t) { acc[t] = mfma_f64(xa, w_at_use(wf[t][s]), acc[t]); });
    });
    // acc[t][r] = q_hat[i0 + 4 r + lk][16 ct + li]
    static_for<CT>([&](auto t) {
      static_for<4>([&](auto r) {
        const int i = i0 + 4 * r + lk;
        if (i < T) qhat[((size_t)bh * T + i) * D + 16 * (w + 4 * t) + li] = acc[t][int(r)];
      });
    });
  } else {
    static_for<KS>([&](auto s) {
      const double xa = rows[li * RP + lk * (KS + 1) + s];
      static_for<CT>([&](auto t) { acc[t] = mfma_f64(w_at_use(wf[t][s]), xa, acc[t]); });
    });
    // acc[t][r] = k_hat[i0 + li][16 ct + 4 r + lk]
    if (i0 + li < T) {
      static_for<CT>([&](auto t) {
        static_for<4>([&](auto r) {
          khatT[((size_t)bh * D + 16 * (w + 4 * t) + 4 * r + lk) * T + i0 + li] = acc[t][int(r)];
        });
      });
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
// Scores, then Top-k, in two kernels.
//
// Scores: one workgroup per (32 query blocks, 128 key blocks, head), 256 threads; a 12-head
// layer of 512 blocks gives 768 workgroups, three per CU.  The scores q_hat k_hat^T / sqrt(d)
// are formed in fp64 on the matrix cores: the A operands are the two 16 x D tiles of q_hat
// rows, staged in LDS (rows past T repeat row T - 1 and are not stored); wave w takes key
// tiles w and w + 4 of the workgroup's 8, and each quarter tile of the k_hat operand, loaded two
// quarters ahead, serves both row tiles, which halves the k_hat reads of 16-row workgroups.
// Each score goes to the workspace as an order-preserving 64-bit key.
//
// Top-k: one wave per row (four rows per workgroup), holding the row's keys in registers (key j
// in slot j / 64 of lane j % 64).  The topk-th largest key is found by a bitwise binary search:
// bit by bit from the top, a candidate threshold is kept when at least topk keys reach it
// (counted with ballots); the search stops as soon as exactly topk keys reach the threshold.
// The high 32 bits are searched first; the low 32 bits only when the high halves tie.
// Keys equal to the final threshold are taken in increasing j until topk are chosen, which
// gives the lower block index on ties.  The mask row and the ascending LUT row follow by
// ballot compaction.
// For topk <= 64 the search over all keys is narrowed first (prune_rows below): the maxima
// of topk lanes are topk distinct keys, so the largest t (in steps of 2^16) that topk lane
// maxima reach is a lower bound lb of the threshold.  The keys reaching lb are the only
// candidates; when there are at most 64 they are compacted to one per lane (through LDS) and
// the threshold is searched among them, one comparison per step instead of one per slot.
// Every search starts below the common leading bits of its lower and upper bound, which the
// threshold shares.  The result is the same threshold, so the same selection.
// With SOFT (sla2_route_soft) the wave then forms the row's SoftTop-k mask and lambda
// (soft_row above) from the same fp64 scores.
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

// Max / min of a 32-bit unsigned value over the wave, in a scalar register.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, dpp_u32<0x128>(v));   // row_ror:8
  v = op(v, dpp_u32<0x124>(v));   // row_ror:4
  v = op(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = op(r[0], r[1]);
  auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __builtin_amdgcn_readfirstlane(op(q[0], q[1]));
}

// Highest set bit of x (-1 for 0), and x with its bits p .. 0 cleared (none for p < 0).
__device__ __forceinline__ int high_bit(uint32_t x) { return 31 - __clz((int)x); }
__device__ __forceinline__ uint32_t keep_above(uint32_t x, int p) {
  return p < 0 ? x : (p >= 31 ? 0u : x & (~0u << (p + 1)));
}

// Narrows the search of J rows (high halves hi of the keys, MAXS slots per lane), using 64
// words of LDS per row at cscr.  On return a row is either resolved (done: thr is its
// threshold, exact when exactly topk keys reach it) or left to the search over all keys from
// bit top with thr holding the bits above.
template <int J, int MAXS>
__device__ __forceinline__ void prune_rows(const uint32_t (&hi)[J][MAXS], uint32_t (&thr)[J], int (&top)[J],
                                           bool (&done)[J], bool (&exact)[J], int topk, uint32_t* cscr,
                                           int lane, uint64_t lt_mask) {
  // lower bound: the largest t (high 16 bits) reached by the maxima of at least topk lanes,
  // searched from below the leading bits shared by the smallest and largest lane maximum
  uint32_t m16[J], mx[J], t1[J];
  int p1[J];
  bool stop[J];
  int pmax = -1;
  static_for<J>([&](auto jj) {
    uint32_t m = hi[jj][0];
    static_for<MAXS - 1>([&](auto s) { m = m > hi[jj][s + 1] ? m : hi[jj][s + 1]; });
    m16[jj] = m >> 16;
    mx[jj] = wave_ext_u32<true>(m);
    const uint32_t mn16 = wave_ext_u32<false>(m16[jj]);
    p1[jj] = high_bit(mn16 ^ (mx[jj] >> 16));
    t1[jj] = keep_above(mn16, p1[jj]);   // every lane maximum reaches it
    stop[jj] = done[jj];
    pmax = max(pmax, p1[jj]);
  });
  for (int bit = pmax; bit >= 0; --bit) {
    bool all = true;
    static_for<J>([&](auto jj) {
      const uint32_t cand = t1[jj] | (1u << bit);
      const int cnt = ballot_count(m16[jj] >= cand);
      const bool take = !stop[jj] && bit <= p1[jj] && cnt >= topk;
      t1[jj] = take ? cand : t1[jj];
      stop[jj] = stop[jj] || (take && cnt == topk);
      all = all && stop[jj];
    });
    if (all) break;
  }
  // the keys reaching lb, compacted in order of slot and lane (the first 64 of them)
  uint32_t lb[J], cv[J];
  int cnum[J];
  static_for<J>([&](auto jj) {
    lb[jj] = t1[jj] << 16;
    int base = 0;
    static_for<MAXS>([&](auto s) {
      const bool on = hi[jj][s] >= lb[jj];
      const uint64_t b = __builtin_amdgcn_ballot_w64(on);
      const int pos = base + __popcll(b & lt_mask);
      if (on && pos < 64) cscr[jj * 64 + pos] = hi[jj][s];
      base += __popcll(b);
    });
    cnum[jj] = base;
  });
  static_for<J>([&](auto jj) { cv[jj] = lane < cnum[jj] ? cscr[jj * 64 + lane] : 0u; });
  // threshold among the candidates, searched from below the leading bits of lb and the row max
  uint32_t th[J];
  int p2[J];
  bool ex[J], fin[J];
  pmax = -1;
  static_for<J>([&](auto jj) {
    p2[jj] = high_bit(lb[jj] ^ mx[jj]);
    th[jj] = keep_above(lb[jj], p2[jj]);
    ex[jj] = cnum[jj] == topk;
    fin[jj] = done[jj] || ex[jj] || cnum[jj] > 64;
    if (!fin[jj]) pmax = max(pmax, p2[jj]);
  });
  for (int bit = pmax; bit >= 0; --bit) {
    bool all = true;
    static_for<J>([&](auto jj) {
      const uint32_t cand = th[jj] | (1u << bit);
      const int cnt = ballot_count(cv[jj] >= cand);
      const bool take = !fin[jj] && bit <= p2[jj] && cnt >= topk;
      th[jj] = take ? cand : th[jj];
      const bool hit = take && cnt == topk;
      ex[jj] = ex[jj] || hit;
      fin[jj] = fin[jj] || hit;
      all = all && fin[jj];
    });
    if (all) break;
  }
  static_for<J>([&](auto jj) {
    if (done[jj]) return;   // rows past T
    if (cnum[jj] == topk) {
      thr[jj] = lb[jj];
      done[jj] = exact[jj] = true;
    } else if (cnum[jj] <= 64) {
      thr[jj] = th[jj];
      exact[jj] = ex[jj];
      done[jj] = true;
    } else {
      thr[jj] = keep_above(lb[jj], p2[jj]);
      top[jj] = p2[jj];
    }
  });
}

constexpr int kScoreRows = 32;    // query blocks per scores workgroup (two matrix-core tiles)
constexpr int kScoreKeys = 128;   // key blocks per scores workgroup

template <int D>
__global__ __launch_bounds__(256, 3) void scores_kernel(const double* __restrict__ qhat,
                                                        const double* __restrict__ khatT, int T, int nrb, int ncb,
                                                        double inv_sqrt_d, uint64_t* __restrict__ keys) {
  constexpr int KS = D / 4;    // matrix-core steps over the channels
  constexpr int QS = KS / 4;   // steps per quarter tile
  constexpr int QP = D + 2;    // LDS row pitch of q_hat (doubles): 16 rows x 4 lane groups hit 64 banks
  __shared__ double qs[kScoreRows * QP];
  // consecutive workgroups (row blocks of one key range of one head) run on one XCD, whose L2
  // then holds that part of k_hat
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / (nrb * ncb), cb = (lid / nrb) % ncb, i0 = (lid % nrb) * kScoreRows;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;
  // the workgroup's q_hat rows (rows past T repeat row T - 1; their scores are not stored)
  for (int x = tid; x < kScoreRows * D / 2; x += 256) {
    const int r = x / (D / 2), c = 2 * (x % (D / 2));
    const double* src = qhat + ((size_t)bh * T + min(i0 + r, T - 1)) * D + c;
    qs[r * QP + c] = src[0];
    qs[r * QP + c + 1] = src[1];
  }
  const double* kb = khatT + (size_t)bh * D * T;   // the head's k_hat^T (a scalar base)
  const int t_end = min((T + 15) >> 4, (cb + 1) * (kScoreKeys / 16));
  // quarter tiles: the k_hat operand of steps q*QS .. q*QS + QS - 1 of key tile tt goes to
  // buffer q, loaded two quarters ahead of its multiplies and used by both row tiles; step s
  // adds a uniform 4 s T to the lane's offset lk T + j, so the loads share one offset register
  double kv[4][QS];
  auto load_quarter = [&](double(&dst)[QS], int tt, int q) {
    const int voff = lk * T + min(16 * tt + li, T - 1);
    static_for<QS>([&](auto s) { dst[s] = kb[(size_t)(4 * (q * QS + s)) * T + voff]; });
  };
  const int t0 = cb * (kScoreKeys / 16) + w;
  if (t0 < t_end) {
    load_quarter(kv[0], t0, 0);
    load_quarter(kv[1], t0, 1);
  }
  __syncthreads();
  const double* qa = qs + li * QP + lk;   // row li of the first row tile, channel 4 s + lk
  for (int tt = t0; tt < t_end; tt += 4) {
    // per row tile two accumulators (even / odd steps): four independent chains in flight
    f64x4 a0 = f64x4{0.0, 0.0, 0.0, 0.0}, a1 = a0, b0 = a0, b1 = a0;
    static_for<4>([&](auto q) {
      // each quarter's LDS operand reads stay in that quarter (hoisting them all spills)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (q < 2) load_quarter(kv[q + 2], tt, q + 2);
      else if (tt + 4 < t_end) load_quarter(kv[q - 2], tt + 4, q - 2);
      static_for<QS / 2>([&](auto s) {
        constexpr int k0 = 4 * (q * QS + 2 * s), k1 = k0 + 4;
        a0 = mfma_f64(qa[k0], kv[q][2 * s], a0);
        b0 = mfma_f64(qa[16 * QP + k0], kv[q][2 * s], b0);
        a1 = mfma_f64(qa[k1], kv[q][2 * s + 1], a1);
        b1 = mfma_f64(qa[16 * QP + k1], kv[q][2 * s + 1], b1);
      });
    });
    const f64x4 sa = a0 + a1, sb = b0 + b1;
    const int j = 16 * tt + li;
    static_for<4>([&](auto r) {
      const int i = i0 + 4 * r + lk;   // accumulator r holds tile row 4r + lane/16
      if (j < T) {
        if (i < T) keys[((size_t)bh * T + i) * T + j] = score_key(sa[int(r)] * inv_sqrt_d);
        if (i + 16 < T) keys[((size_t)bh * T + i + 16) * T + j] = score_key(sb[int(r)] * inv_sqrt_d);
      }
    });
  }
}

// Emits one row of the LUT and the mask from the row's keys and the threshold found on their
// high halves: the low halves are searched when the high halves tie at the boundary (exact
// false); keys above the threshold are all taken, keys equal to it fill the rest in
// increasing j.
template <int MAXS>
__device__ __forceinline__ void emit_row(const uint64_t (&key)[MAXS], uint32_t thr_hi, bool exact, int T, int topk,
                                         int32_t* __restrict__ lut_row, uint8_t* __restrict__ mask_row, int lane,
                                         uint64_t lt_mask) {
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
  int need = topk;
  static_for<MAXS>([&](auto s) { need -= ballot_count(key[s] > thr); });
  int base = 0;
  static_for<MAXS>([&](auto s) {
    const int j = 64 * s + lane;
    const uint64_t eq = __builtin_amdgcn_ballot_w64(key[s] == thr);
    const int n_eq = __popcll(eq);
    const int take = n_eq < need ? n_eq : need;
    const bool on = key[s] > thr || (key[s] == thr && __popcll(eq & lt_mask) < take);
    need -= take;
    const uint64_t bmask = __builtin_amdgcn_ballot_w64(on);
    const int at = base + __popcll(bmask & lt_mask);
    if (on && at < topk) lut_row[at] = j;   // exactly topk are on; the test only bounds the store
    base += __popcll(bmask);
    if (j < T) mask_row[j] = on ? 1 : 0;
  });
}

// Waves per SIMD the select kernel is compiled for: six where a row's keys take few registers,
// one for the soft mask over 4096 keys (whose fp64 scores fill the registers).
template <int MAXS, bool SOFT>
constexpr int select_waves() { return MAXS <= 8 ? 6 : (MAXS <= 24 ? 4 : (MAXS <= 32 || !SOFT ? 2 : 1)); }

template <int MAXS, bool SOFT>
__global__ __launch_bounds__(256, (select_waves<MAXS, SOFT>())) void select_kernel(
    const uint64_t* __restrict__ keys, long long rows, int T, int topk, int32_t* __restrict__ lut,
    uint8_t* __restrict__ mask, double tau, float* __restrict__ soft_mask, float* __restrict__ lambda) {
  __shared__ uint32_t cscr[4][64];   // candidate compaction, one row per wave
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + w;   // bh * T + i
  if (row >= rows) return;                                // the whole wave
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const uint64_t* krow = keys + row * T;
  uint64_t key[MAXS];
  uint32_t hi[1][MAXS];
  static_for<MAXS>([&](auto s) {
    const int j = 64 * s + lane;
    key[s] = j < T ? krow[j] : 0ull;   // 0 is below every score key
    hi[0][s] = (uint32_t)(key[s] >> 32);
  });
  uint32_t thr[1] = {0u};   // bits of the high-half threshold decided so far
  int top[1] = {31};        // highest bit still to decide
  bool done[1] = {false}, exact[1] = {false};
  if (topk <= 64) prune_rows<1, MAXS>(hi, thr, top, done, exact, topk, cscr[w], lane, lt_mask);
  if (!done[0]) {
    // largest high-half threshold reached by at least topk keys (all ballots of a step are
    // formed before they are counted)
    for (int bit = top[0]; bit >= 0; --bit) {
      const uint32_t cand = thr[0] | (1u << bit);
      uint64_t bl[MAXS];
      static_for<MAXS>([&](auto s) { bl[s] = __builtin_amdgcn_ballot_w64(hi[0][s] >= cand); });
      int cnt = 0;
      static_for<MAXS>([&](auto s) { cnt += __popcll(bl[s]); });
      if (cnt >= topk) {
        thr[0] = cand;
        if (cnt == topk) {
          exact[0] = true;
          break;
        }
      }
    }
  }
  emit_row<MAXS>(key, thr[0], exact[0], T, topk, lut + row * topk, mask + row * T, lane, lt_mask);
  if constexpr (SOFT) {
    double p[MAXS];
    static_for<MAXS>([&](auto s) {
      const int j = 64 * s + lane;
      p[s] = j < T ? key_score(key[s]) : 0.0;   // already divided by sqrt(d)
    });
    soft_row<MAXS>(p, T, topk, 1.0, tau, soft_mask + row * T, lambda + row, lane);
  }
}

// Soft-mask arguments of the SoftTop-k step (unused by the plain router).
struct SoftOut {
  double tau;
  float* mask;
  float* lambda;
};

template <int MAXS, bool SOFT>
static void launch_select(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const SoftOut& so,
                          hipStream_t s) {
  const long long rows = (long long)g.BH * g.T;
  hipLaunchKernelGGL((select_kernel<MAXS, SOFT>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, ws.keys, rows,
                     g.T, g.topk, t.lut, t.mask, so.tau, so.mask, so.lambda);
}

// The scores, then the row selection with MAXS slots per lane: the smallest of 4, 8, 16, 24,
// 32, 64 that is at least ceil(T / 64) (T <= 4096).
template <int D, bool SOFT>
static void launch_topk(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const SoftOut& so,
                        hipStream_t s) {
  const int nrb = (g.T + kScoreRows - 1) / kScoreRows, ncb = (g.T + kScoreKeys - 1) / kScoreKeys;
  hipLaunchKernelGGL(scores_kernel<D>, dim3((unsigned)(nrb * ncb * g.BH)), dim3(256), 0, s, ws.qhat, ws.khatT, g.T,
                     nrb, ncb, 1.0 / sqrt((double)g.D), ws.keys);
  const int S = (g.T + 63) / 64;
  if (S <= 4) launch_select<4, SOFT>(g, t, ws, so, s);
  else if (S <= 8) launch_select<8, SOFT>(g, t, ws, so, s);
  else if (S <= 16) launch_select<16, SOFT>(g, t, ws, so, s);
  else if (S <= 24) launch_select<24, SOFT>(g, t, ws, so, s);
  else if (S <= 32) launch_select<32, SOFT>(g, t, ws, so, s);
  else launch_select<64, SOFT>(g, t, ws, so, s);
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
