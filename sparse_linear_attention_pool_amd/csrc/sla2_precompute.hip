// SLA2 linear-branch precompute: per key block j, with the smoothed keys K~ = K - mu,
//   phi(K~_t) = softmax over the d features of token t,
//   h_j = sum_t phi(K~_t)^T V_t (d x d, stored transposed: h[j][c][a]),
//   z_j = sum_t phi(K~_t),
// plus h_sum = sum_j h_j and z_sum = sum_j z_j (chunk partials, then a fixed-order sum).
// In FP8 mode the same pass quantises K~ per 64-token block (absmax/448 scale, e4m3 codes).
// The bf16 pass also writes, for the fused forward kernel, each block's V transposed (with
// the key order of its matrix-core operands) and the e4m3 codes of phi(K~) with one
// max/448 scale per block; h_j and z_j themselves are stored only if asked for.
//
// Pages: "SLA: Beyond Sparsity in Diffusion Transformers...", section 2 Q2 step 3 and the
// section 3 figure (h_j = phi(K_j)^T V_j, z_j = rowsum(phi(K_j)^T), phi = softmax), section 4
// (linear re-association); "SLA2: Sparse-Linear Attention with Learnable Routing and QAT",
// section 3 (the linear branch first forms K^T V statistics, then multiplies by Q), section 5
// (K quantised with scales), section 6 (key smoothing before block processing).
#include <math.h>

#include "sla2_device.hpp"
#include "sla2_internal.hpp"

namespace sla2 {

// ---------------------------------------------------------------------------------------
// bf16, d = 128: one workgroup per (chunk of kChunk key blocks, head), 256 threads.
// Thread (c = tid % 16, r0 = tid / 16) holds columns 8c..8c+7 of rows r0 + 16p, p = 0..3.
// phi and V go to LDS row-major (row stride 65 words, conflict-free 16-bit column gathers);
// wave w computes the 4 x 4 tiles (a-tiles 4*(w/2).., c-tiles 4*(w%2)..) of
// D[a][c] = sum_t phi[t][a] V[t][c] with v_mfma_f32_16x16x32_bf16 over 64 tokens.  phi is
// split into bf16 hi + lo parts (phi - hi rounded again), so the product carries phi to about
// 2^-16 relative although the matrix cores take bf16; V is bf16 already.
// ---------------------------------------------------------------------------------------
template <bool FP8>
__global__ __launch_bounds__(256) void precompute_bf16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ k_mean,
    int N, int T, int P, uint8_t* __restrict__ k8, float* __restrict__ k_scale,
    uint16_t* __restrict__ h, float* __restrict__ z, float* __restrict__ hpart,
    float* __restrict__ zpart, uint16_t* __restrict__ vt, uint8_t* __restrict__ phik8,
    float* __restrict__ phik_scale) {
  constexpr int D = 128;
  constexpr int SW = 65;  // LDS row stride in 32-bit words
  __shared__ uint32_t phiS[64 * SW];
  __shared__ uint32_t phiLoS[64 * SW];
  __shared__ uint32_t vS[64 * SW];
  __shared__ float zred[16 * D];
  __shared__ float wmax[4];
  __shared__ float pmax[4];

  const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int c = tid & 15, r0 = tid >> 4;
  const uint16_t* phi16 = reinterpret_cast<const uint16_t*>(phiS);
  const uint16_t* philo16 = reinterpret_cast<const uint16_t*>(phiLoS);
  const uint16_t* v16 = reinterpret_cast<const uint16_t*>(vS);

  float mu[8];
  {
    const float4 m0 = *reinterpret_cast<const float4*>(k_mean + (size_t)bh * D + 8 * c);
    const float4 m1 = *reinterpret_cast<const float4*>(k_mean + (size_t)bh * D + 8 * c + 4);
    mu[0] = m0.x; mu[1] = m0.y; mu[2] = m0.z; mu[3] = m0.w;
    mu[4] = m1.x; mu[5] = m1.y; mu[6] = m1.z; mu[7] = m1.w;
  }
  const int mbase = 4 * (w >> 1), nbase = 4 * (w & 1);
  f32x4 hs[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) hs[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zs = 0.f;

  const int j_lo = chunk * kChunk, j_hi = min(T, j_lo + kChunk);
  for (int j = j_lo; j < j_hi; ++j) {
    float kt[4][8];
    uint4 vraw[4];
    bool valid[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = kBlock * j + r0 + 16 * p;
      valid[p] = row < N;
      uint4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
      if (valid[p]) {
        const size_t off = ((size_t)bh * N + row) * D + 8 * c;
        kw = *reinterpret_cast<const uint4*>(k + off);
        vw = *reinterpret_cast<const uint4*>(v + off);
      }
      vraw[p] = vw;
      const uint32_t ka[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kt[p][2 * e] = valid[p] ? bf16_lo(ka[e]) - mu[2 * e] : 0.f;
        kt[p][2 * e + 1] = valid[p] ? bf16_hi(ka[e]) - mu[2 * e + 1] : 0.f;
      }
    }

    if constexpr (FP8) {
      float amax = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(kt[p][e]));
      amax = wave_max(amax);
      if (lane == 0) wmax[w] = amax;
      __syncthreads();
      const float bm = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
      float s = __fdiv_rn(bm, kFp8Max);
      if (s == 0.f) s = 1.f;
      if (tid == 0) k_scale[(size_t)bh * T + j] = s;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = clamp_fp8(__fdiv_rn(kt[p][e], s));
        uint2 codes;
        codes.x = pack_fp8x4(y[0], y[1], y[2], y[3]);
        codes.y = pack_fp8x4(y[4], y[5], y[6], y[7]);
        const int row = kBlock * j + r0 + 16 * p;
        *reinterpret_cast<uint2*>(k8 + ((size_t)bh * T * kBlock + row) * D + 8 * c) = codes;
      }
    }

    // phi over the 128 features of each row (16 lanes of one 16-lane row hold a token)
    float zp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zp[e] = 0.f;
    float phv[4][8];
    float phmax = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float mx = kt[p][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, kt[p][e]);
      mx = row16_max(mx);
      float ex[8], sm = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ex[e] = exp2f((kt[p][e] - mx) * kLog2e);
        sm += ex[e];
      }
      sm = row16_sum(sm);
      const float inv = valid[p] ? 1.f / sm : 0.f;
      uint32_t pw[4], pl[4];
      float ph[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ph[e] = ex[e] * inv;
        zp[e] += ph[e];
        phv[p][e] = ph[e];
        phmax = fmaxf(phmax, ph[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[e] = pack_bf16x2(ph[2 * e], ph[2 * e + 1]);
        pl[e] = pack_bf16x2(ph[2 * e] - bf16_lo(pw[e]), ph[2 * e + 1] - bf16_hi(pw[e]));
      }
      const int r = r0 + 16 * p;
      uint32_t* pd = phiS + r * SW + 4 * c;
      pd[0] = pw[0]; pd[1] = pw[1]; pd[2] = pw[2]; pd[3] = pw[3];
      uint32_t* pld = phiLoS + r * SW + 4 * c;
      pld[0] = pl[0]; pld[1] = pl[1]; pld[2] = pl[2]; pld[3] = pl[3];
      uint32_t* vd = vS + r * SW + 4 * c;
      vd[0] = vraw[p].x; vd[1] = vraw[p].y; vd[2] = vraw[p].z; vd[3] = vraw[p].w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) zred[r0 * D + 8 * c + e] = zp[e];
    phmax = wave_max(phmax);
    if (lane == 0) pmax[w] = phmax;
    __syncthreads();

    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s += zred[r * D + tid];
      if (z != nullptr) z[((size_t)bh * T + j) * D + tid] = s;
      zs += s;
    }
    // e4m3 codes of phi(K~) for the fused forward kernel: one max/448 scale per block
    {
      const float bm = fmaxf(fmaxf(pmax[0], pmax[1]), fmaxf(pmax[2], pmax[3]));
      float sp = __fdiv_rn(bm, kFp8Max);
      if (sp == 0.f) sp = 1.f;
      if (tid == 0) phik_scale[(size_t)bh * T + j] = sp;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = clamp_fp8(__fdiv_rn(phv[p][e], sp));
        uint2 codes;
        codes.x = pack_fp8x4(y[0], y[1], y[2], y[3]);
        codes.y = pack_fp8x4(y[4], y[5], y[6], y[7]);
        const int row = kBlock * j + r0 + 16 * p;
        *reinterpret_cast<uint2*>(phik8 + ((size_t)bh * T * kBlock + row) * D + 8 * c) = codes;
      }
    }

    // h^T tiles on the matrix cores
    f32x4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int t0 = 32 * ks + 8 * g;
      bf16x8 A[4], Alo[4], Bv[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int a = 16 * (mbase + mi) + l16;
        uint16_t e16[8], l16v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          e16[e] = phi16[(t0 + e) * 2 * SW + a];
          l16v[e] = philo16[(t0 + e) * 2 * SW + a];
        }
        A[mi] = __builtin_bit_cast(bf16x8, e16);
        Alo[mi] = __builtin_bit_cast(bf16x8, l16v);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int cc = 16 * (nbase + ni) + l16;
        uint16_t e16[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e16[e] = v16[(t0 + e) * 2 * SW + cc];
        Bv[ni] = __builtin_bit_cast(bf16x8, e16);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          acc[mi][ni] = mfma_bf16(Alo[mi], Bv[ni], acc[mi][ni]);
          acc[mi][ni] = mfma_bf16(A[mi], Bv[ni], acc[mi][ni]);
        }
    }
    // D[a = 16m + 4g + r][c = 16n + l16] -> h[j][c][a .. a+3] (if stored)
    uint16_t* hj = h + ((size_t)bh * T + j) * D * D;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int a0 = 16 * (mbase + mi) + 4 * g;
        const int cc = 16 * (nbase + ni) + l16;
        if (h != nullptr) {
          uint2 st;
          st.x = pack_bf16x2(acc[mi][ni][0], acc[mi][ni][1]);
          st.y = pack_bf16x2(acc[mi][ni][2], acc[mi][ni][3]);
          *reinterpret_cast<uint2*>(hj + (size_t)cc * D + a0) = st;
        }
        hs[mi][ni] += acc[mi][ni];
      }

    // V of this block, transposed: vt[j][c][32s + 8gg + e] = V[key][c] with
    // key = 32s + 4gg + e (e < 4) or 32s + 16 + 4gg + (e - 4) (e >= 4)
    uint16_t* vtj = vt + ((size_t)bh * T + j) * D * kBlock;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int qd = tid + 256 * pp;
      const int cc = qd >> 3, s = (qd >> 2) & 1, gg = qd & 3;
      uint16_t e16[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 32 * s + (e < 4 ? 4 * gg + e : 16 + 4 * gg + (e - 4));
        e16[e] = v16[key * 2 * SW + cc];
      }
      *reinterpret_cast<uint4*>(vtj + (size_t)cc * kBlock + 32 * s + 8 * gg) =
          __builtin_bit_cast(uint4, e16);
    }
    __syncthreads();
  }

  float* hp = hpart + ((size_t)bh * P + chunk) * D * D;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int a0 = 16 * (mbase + mi) + 4 * g;
      const int cc = 16 * (nbase + ni) + l16;
      *reinterpret_cast<float4*>(hp + (size_t)cc * D + a0) =
          make_float4(hs[mi][ni][0], hs[mi][ni][1], hs[mi][ni][2], hs[mi][ni][3]);
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

// h_sum / z_sum: sum of the chunk partials in chunk order.
__global__ __launch_bounds__(256) void reduce_sums_kernel(const float* __restrict__ hpart,
                                                          const float* __restrict__ zpart, int P, int D,
                                                          float* __restrict__ h_sum,
                                                          float* __restrict__ z_sum) {
  const int bh = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  const int DD = D * D;
  if (e < DD) {
    float s = 0.f;
    for (int p = 0; p < P; ++p) s += hpart[((size_t)bh * P + p) * DD + e];
    h_sum[(size_t)bh * DD + e] = s;
  }
  if (blockIdx.x == 0 && threadIdx.x < D) {
    float s = 0.f;
    for (int p = 0; p < P; ++p) s += zpart[((size_t)bh * P + p) * D + threadIdx.x];
    z_sum[(size_t)bh * D + threadIdx.x] = s;
  }
}

hipError_t launch_precompute(const Geometry& g, const sla2_tensors& t, const Workspace& ws,
                             hipStream_t s) {
  dim3 grid(g.P, g.BH);
  if (g.bf16) {
    if (g.fp8)
      hipLaunchKernelGGL(precompute_bf16_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)t.k,
                         (const uint16_t*)t.v, t.k_mean, g.N, g.T, g.P, t.k8, t.k_scale,
                         (uint16_t*)t.h, t.z, ws.hpart, ws.zpart, ws.vt, ws.phik8, ws.phik_scale);
    else
      hipLaunchKernelGGL(precompute_bf16_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)t.k,
                         (const uint16_t*)t.v, t.k_mean, g.N, g.T, g.P, (uint8_t*)nullptr,
                         (float*)nullptr, (uint16_t*)t.h, t.z, ws.hpart, ws.zpart, ws.vt, ws.phik8,
                         ws.phik_scale);
  } else if (g.D == 128) {
    hipLaunchKernelGGL(precompute_f32_kernel<128>, grid, dim3(256), 0, s, (const float*)t.k,
                       (const float*)t.v, t.k_mean, g.N, g.T, g.P, (float*)t.h, t.z, ws.hpart,
                       ws.zpart);
  } else {
    hipLaunchKernelGGL(precompute_f32_kernel<64>, grid, dim3(256), 0, s, (const float*)t.k,
                       (const float*)t.v, t.k_mean, g.N, g.T, g.P, (float*)t.h, t.z, ws.hpart,
                       ws.zpart);
  }
  hipLaunchKernelGGL(reduce_sums_kernel, dim3((g.D * g.D + 255) / 256, g.BH), dim3(256), 0, s,
                     ws.hpart, ws.zpart, g.P, g.D, t.h_sum, t.z_sum);
  return hipGetLastError();
}

}  // namespace sla2
