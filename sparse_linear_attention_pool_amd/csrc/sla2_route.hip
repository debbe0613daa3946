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
// (exact for bf16 inputs); in FP8 mode also the block's absmax scale and the e4m3 codes of
// Q.  Rows past N count as zero and receive code 0.
// ---------------------------------------------------------------------------------------
template <typename Tin, int D, bool FP8>
__global__ __launch_bounds__(256) void pool_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   int N, int T, double* __restrict__ qsum,
                                                   double* __restrict__ ksum, uint8_t* __restrict__ q8,
                                                   float* __restrict__ q_scale) {
  constexpr int VEC = 16 / sizeof(Tin);  // elements per 16-byte chunk
  constexpr int CPR = D / VEC;           // chunks per row
  constexpr int RPP = 256 / CPR;         // rows per pass
  constexpr int PASSES = kBlock / RPP;
  static_assert(!FP8 || VEC == 8, "FP8 quantisation needs bf16 input");
  __shared__ double red[RPP * D];
  __shared__ float wmax[4];

  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = tid % CPR, r0 = tid / CPR;
  const size_t head = (size_t)bh * N;

  float qv[PASSES][VEC];
  double qs[VEC], ks[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) qs[e] = ks[e] = 0.0;
  float amax = 0.f;

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = kBlock * i + r0 + p * RPP;
    float kv[VEC];
    if (row < N) {
      const uint4 qw = *reinterpret_cast<const uint4*>(q + (head + row) * D + c * VEC);
      const uint4 kw = *reinterpret_cast<const uint4*>(k + (head + row) * D + c * VEC);
      if constexpr (sizeof(Tin) == 2) {
        const uint32_t qa[4] = {qw.x, qw.y, qw.z, qw.w}, ka[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[p][2 * e] = bf16_lo(qa[e]);
          qv[p][2 * e + 1] = bf16_hi(qa[e]);
          kv[2 * e] = bf16_lo(ka[e]);
          kv[2 * e + 1] = bf16_hi(ka[e]);
        }
      } else {
        const uint32_t qa[4] = {qw.x, qw.y, qw.z, qw.w}, ka[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[p][e] = __uint_as_float(qa[e]);
          kv[e] = __uint_as_float(ka[e]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) qv[p][e] = kv[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      qs[e] += (double)qv[p][e];
      ks[e] += (double)kv[e];
      amax = fmaxf(amax, fabsf(qv[p][e]));
    }
  }

  // column sums: per-thread partials -> LDS -> one thread per column
  const size_t out = ((size_t)bh * T + i) * D;
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[r0 * D + c * VEC + e] = qs[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    for (int r = 0; r < RPP; ++r) s += red[r * D + tid];
    qsum[out + tid] = s;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[r0 * D + c * VEC + e] = ks[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    for (int r = 0; r < RPP; ++r) s += red[r * D + tid];
    ksum[out + tid] = s;
  }

  if constexpr (FP8) {
    const float wm = wave_max(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = wm;
    __syncthreads();
    const float bm = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    float s = __fdiv_rn(bm, kFp8Max);
    if (s == 0.f) s = 1.f;
    if (tid == 0) q_scale[(size_t)bh * T + i] = s;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = kBlock * i + r0 + p * RPP;
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = clamp_fp8(__fdiv_rn(qv[p][e], s));
      uint2 codes;
      codes.x = pack_fp8x4(y[0], y[1], y[2], y[3]);
      codes.y = pack_fp8x4(y[4], y[5], y[6], y[7]);
      *reinterpret_cast<uint2*>(q8 + ((size_t)bh * T * kBlock + row) * D + c * 8) = codes;
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
// q_hat = q_bar W_q, k_hat = k_bar W_k in fp64 (W NULL = identity).  Thread (rg, cg) computes
// rows 2rg, 2rg+1 and output columns 4cg..4cg+3 (D = 128) or 2cg..2cg+1 (D = 64).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void project_kernel(
    const double* __restrict__ qsum, const double* __restrict__ ksum, const double* __restrict__ kpart,
    int N, int T, int smooth_k, const float* __restrict__ wq, const float* __restrict__ wk,
    float* __restrict__ q_pool, float* __restrict__ k_pool, float* __restrict__ k_mean,
    double* __restrict__ mu_out, double* __restrict__ qhat, double* __restrict__ khatT) {
  constexpr int R = 16;
  constexpr int CPT = D / 32;                 // output columns per thread
  __shared__ double mu_s[D];
  __shared__ __attribute__((aligned(16))) double rows[D][R];   // [a][r]: a row pair is 16 bytes
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
    rows[c][r] = v;
  }
  __syncthreads();

  const int rg = tid >> 5, cg = tid & 31;
  const int r0 = 2 * rg, c0 = CPT * cg;
  double acc[2][CPT];
  const float* W = which ? wk : wq;
  if (W != nullptr) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int x = 0; x < CPT; ++x) acc[u][x] = 0.0;
#pragma unroll 8
    for (int a = 0; a < D; ++a) {
      const double2 rv = *reinterpret_cast<const double2*>(&rows[a][r0]);
      float wv[CPT];
      if constexpr (CPT == 4) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(W + a * D + c0);
        wv[0] = w4[0]; wv[1] = w4[1]; wv[2] = w4[2]; wv[3] = w4[3];
      } else {
#pragma unroll
        for (int x = 0; x < CPT; ++x) wv[x] = W[a * D + c0 + x];
      }
#pragma unroll
      for (int x = 0; x < CPT; ++x) {
        acc[0][x] = fma(rv.x, (double)wv[x], acc[0][x]);
        acc[1][x] = fma(rv.y, (double)wv[x], acc[1][x]);
      }
    }
  } else {
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      acc[0][x] = rows[c0 + x][r0];
      acc[1][x] = rows[c0 + x][r0 + 1];
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = i0 + r0 + u;
    if (i >= T) continue;
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      if (which == 0)
        qhat[((size_t)bh * T + i) * D + c0 + x] = acc[u][x];
      else
        khatT[((size_t)bh * D + c0 + x) * T + i] = acc[u][x];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Scores + Top-k: one workgroup per (R query blocks, head).  Phase 1: every thread scores
// key blocks j = tid, tid+256, ... against the R query rows (fp64; k_hat read once per
// workgroup) into LDS.  Phase 2: one wave per row picks the topk largest scores by
// repeated wave arg-max (ties -> lower j), then writes the mask row and the ascending LUT
// row by ballot compaction.
// ---------------------------------------------------------------------------------------
constexpr int kMaxSlots = 64;   // T <= 64 * 64 = 4096

template <int R, int MAXS>
__global__ __launch_bounds__(256) void topk_kernel(const double* __restrict__ qhat,
                                                   const double* __restrict__ khatT, int T, int D,
                                                   int topk, double inv_sqrt_d,
                                                   int32_t* __restrict__ lut, uint8_t* __restrict__ mask) {
  extern __shared__ double smem_d[];
  double* qs = smem_d;            // [R][D]
  double* sc = smem_d + R * D;    // [R][T]
  const int bh = blockIdx.y, i0 = blockIdx.x * R, tid = threadIdx.x;

  for (int x = tid; x < R * D; x += 256) {
    const int r = x / D, c = x % D;
    const int i = i0 + r;
    qs[x] = (i < T) ? qhat[((size_t)bh * T + i) * D + c] : 0.0;
  }
  __syncthreads();
  for (int j = tid; j < T; j += 256) {
    double acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0;
    const double* kc = khatT + (size_t)bh * D * T + j;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      const double kv = kc[(size_t)c * T];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = fma(qs[r * D + c], kv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r * T + j] = acc[r] * inv_sqrt_d;
  }
  __syncthreads();

  const int w = tid >> 6, lane = tid & 63;
  const int S = (T + 63) >> 6;
  for (int r = w; r < R; r += 4) {
    const int i = i0 + r;
    if (i >= T) break;
    double v[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      const int j = 64 * s + lane;
      v[s] = (s < S && j < T) ? sc[r * T + j] : -INFINITY;
    }
    uint64_t sel = 0;
    for (int it = 0; it < topk; ++it) {
      double bv = -INFINITY;
      int bj = 0x7fffffff;
#pragma unroll
      for (int s = 0; s < MAXS; ++s) {
        if (s < S) {
          const int j = 64 * s + lane;
          if (!((sel >> s) & 1ull) && j < T && (v[s] > bv || bj == 0x7fffffff)) {
            bv = v[s];
            bj = j;
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off);
        const int oj = __shfl_xor(bj, off);
        if (oj != 0x7fffffff && (bj == 0x7fffffff || ov > bv || (ov == bv && oj < bj))) {
          bv = ov;
          bj = oj;
        }
      }
      if (bj == 0x7fffffff) break;
      if ((bj & 63) == lane) sel |= 1ull << (bj >> 6);
    }
    const size_t row = (size_t)bh * T + i;
    int base = 0;
    for (int s = 0; s < S; ++s) {
      const int j = 64 * s + lane;
      const bool on = (sel >> s) & 1ull;
      const uint64_t b = __ballot(on);
      if (on) lut[row * topk + base + __popcll(b & ((1ull << lane) - 1ull))] = j;
      base += __popcll(b);
      if (j < T) mask[row * T + j] = on ? 1 : 0;
    }
  }
}

constexpr size_t kTopkLdsMax = 160 * 1024;

template <int R, int MAXS>
static void launch_topk_s(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s) {
  const size_t lds = (size_t)R * (g.D + g.T) * sizeof(double);
  static bool attr_set = false;   // the kernel may use up to 160 KB of dynamic LDS
  if (!attr_set) {
    hipFuncSetAttribute((const void*)topk_kernel<R, MAXS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)kTopkLdsMax);
    attr_set = true;
  }
  dim3 grid((g.T + R - 1) / R, g.BH);
  hipLaunchKernelGGL((topk_kernel<R, MAXS>), grid, dim3(256), lds, s, ws.qhat, ws.khatT, g.T, g.D, g.topk,
                     1.0 / sqrt((double)g.D), t.lut, t.mask);
}

// candidate slots per lane: the smallest power of two >= ceil(T / 64)
template <int R>
static void launch_topk(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s) {
  const int S = (g.T + 63) / 64;
  if (S <= 4) launch_topk_s<R, 4>(g, t, ws, s);
  else if (S <= 8) launch_topk_s<R, 8>(g, t, ws, s);
  else if (S <= 16) launch_topk_s<R, 16>(g, t, ws, s);
  else if (S <= 32) launch_topk_s<R, 32>(g, t, ws, s);
  else launch_topk_s<R, 64>(g, t, ws, s);
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
  hipLaunchKernelGGL(project_kernel<D>, dim3((g.T + 15) / 16, g.BH, 2), dim3(256), 0, s, ws.qsum,
                     ws.ksum, ws.mu, g.N, g.T, (int)g.smooth_k, t.wq, t.wk, t.q_pool, t.k_pool,
                     t.k_mean, mu_final, ws.qhat, ws.khatT);
}

hipError_t launch_route(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s) {
  if (g.bf16) {
    if (g.D == 128) launch_route_typed<uint16_t, 128>(g, t, ws, s);
    else launch_route_typed<uint16_t, 64>(g, t, ws, s);
  } else {
    if (g.D == 128) launch_route_typed<float, 128>(g, t, ws, s);
    else launch_route_typed<float, 64>(g, t, ws, s);
  }
  // rows per workgroup: the largest power of two <= 16 whose scores fit in the LDS budget
  int R = 16;
  while (R > 1 && (size_t)R * (g.D + g.T) * sizeof(double) > kTopkLdsMax) R >>= 1;
  switch (R) {
    case 16: launch_topk<16>(g, t, ws, s); break;
    case 8: launch_topk<8>(g, t, ws, s); break;
    case 4: launch_topk<4>(g, t, ws, s); break;
    case 2: launch_topk<2>(g, t, ws, s); break;
    default: launch_topk<1>(g, t, ws, s); break;
  }
  return hipGetLastError();
}

}  // namespace sla2
