// SLA2 fused forward: for each query block i, over the routed key blocks j in LUT order,
//   S = Q_i K_j^T / sqrt(d) (FP8 e4m3 codes times the two block scales, or bf16),
//   online softmax (running max and sum, exp2 with log2(e) folded into the scale),
//   acc += P V_j (bf16 matrix cores), and C += h_j, c += z_j for the linear complement;
// then O_s = acc / l, H_i = h_sum - C, Z_i = z_sum - c (the sum over the unrouted blocks),
// O_l = phi(Q_i) H_i / (phi(Q_i) Z_i + eps) and O = alpha * O_s + (1 - alpha) * O_l.
//
// Pages: "SLA2: Sparse-Linear Attention with Learnable Routing and QAT", section 3 (sparse
// attention only where M = 1 on FlashAttention-style computation; linear branch from the
// M = 0 statistics; O = alpha * O_s + (1 - alpha) * O_l), section 5 (low-bit Q.K^T with
// scales), section 6 (M = 1 blocks: sparse scores and values; M = 0 blocks: linear
// statistics); "SLA: Beyond Sparsity in Diffusion Transformers...", section 3 figure
// (O_s = diag(l)^-1 O_acc, O_l = phi(Q_i) H_i / (phi(Q_i) Z_i)), section 4 (online softmax
// with a running max, 1e-5 in the linear denominator), section 7 (the loop walks a LUT of
// routed block indices; exp2 with log2(e) folded into the score scale).
#include <math.h>

#include "sla2_device.hpp"
#include "sla2_internal.hpp"

namespace sla2 {

struct FwdArgs {
  const uint16_t* q;      // bf16 [BH, N, D]
  const uint16_t* k;      // bf16 [BH, N, D] (native Q.K^T only)
  const uint8_t* q8;      // [BH, T*64, D]
  const uint8_t* k8;
  const float* q_scale;   // [BH, T]
  const float* k_scale;
  const uint16_t* vt;     // [BH, T, D, 64]
  const int32_t* lut;     // [BH, T, topk]
  const uint16_t* h;      // [BH, T, D, D] transposed
  const float* z;         // [BH, T, D]
  const float* h_sum;     // [BH, D, D]
  const float* z_sum;     // [BH, D]
  const float* alpha;     // [H, D]
  const float* k_mean;    // [BH, D] (lse of the native mode is shifted to the smoothed keys)
  uint16_t* o;            // [BH, N, D]
  float* lse;             // [BH, N] or null
  int N, T, H, topk, nblocks;
  float eps;
};

// LDS geometry (bytes).  Rows are padded by 16 bytes so that the 16-byte operand reads of
// consecutive lanes (consecutive rows) fall on distinct banks.
template <bool FP8>
struct FwdLds {
  static constexpr int KSTR = FP8 ? 144 : 272;   // one key row: 128 codes or 128 bf16
  static constexpr int VSTR = 144;                // one V^T row: 64 bf16
  static constexpr int KTILE = 64 * KSTR;
  static constexpr int VTILE = 128 * VSTR;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int HSTR = 272;                // epilogue H^T row: 128 bf16
  static constexpr int BYTES = 2 * STAGE;
  static_assert(128 * HSTR + 512 <= BYTES, "epilogue tile must fit in the staging buffers");
};

// Global -> registers: this thread's part of one key block's K tile and V^T tile.
template <bool FP8>
struct TileRegs {
  uint4 kk[FP8 ? 2 : 4];
  uint4 vv[4];
};

template <bool FP8>
__device__ __forceinline__ void load_tile(const FwdArgs& A, int bh, int j, int tid, TileRegs<FP8>& r) {
  constexpr int D = 128;
  if constexpr (FP8) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int qd = tid + 256 * p, row = qd >> 3, cc = qd & 7;
      r.kk[p] = *reinterpret_cast<const uint4*>(A.k8 + (((size_t)bh * A.T + j) * kBlock + row) * D + 16 * cc);
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qd = tid + 256 * p, row = qd >> 4, cc = qd & 15;
      const int tok = kBlock * j + row;
      r.kk[p] = tok < A.N ? *reinterpret_cast<const uint4*>(A.k + ((size_t)bh * A.N + tok) * D + 8 * cc)
                          : uint4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int qd = tid + 256 * p, b = qd >> 3, cc = qd & 7;
    r.vv[p] = *reinterpret_cast<const uint4*>(A.vt + (((size_t)bh * A.T + j) * D + b) * kBlock + 8 * cc);
  }
}

template <bool FP8>
__device__ __forceinline__ void store_tile(uint8_t* stage, int tid, const TileRegs<FP8>& r) {
  using L = FwdLds<FP8>;
  if constexpr (FP8) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int qd = tid + 256 * p, row = qd >> 3, cc = qd & 7;
      *reinterpret_cast<uint4*>(stage + row * L::KSTR + 16 * cc) = r.kk[p];
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qd = tid + 256 * p, row = qd >> 4, cc = qd & 15;
      *reinterpret_cast<uint4*>(stage + row * L::KSTR + 16 * cc) = r.kk[p];
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int qd = tid + 256 * p, b = qd >> 3, cc = qd & 7;
    *reinterpret_cast<uint4*>(stage + L::KTILE + b * L::VSTR + 16 * cc) = r.vv[p];
  }
}

// One workgroup (4 waves) per (head, query block).  Wave w owns queries 16w..16w+15 and
// computes S^T = K_j Q_w^T so that each lane holds one query (l % 16) and 16 of the block's
// keys (16mt + 4(l/16) + r): the softmax state is per lane, and P feeds the P.V product as
// the B operand of O^T = V^T P^T without a transpose.  The same lane also accumulates
// 64 entries of C = sum h_j (rows c = 32w + 16mt + l%16, columns a = 32s + 8(l/16) + e),
// exactly the A operand it needs for O_l^T = H^T phi(Q)^T in the epilogue.
template <bool FP8>
__global__ __launch_bounds__(256) void fwd_mfma_kernel(FwdArgs A) {
  using L = FwdLds<FP8>;
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];

  const int lid = xcd_remap(blockIdx.x, A.nblocks);
  const int bh = lid / A.T, i = lid % A.T;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int hidx = bh % A.H;
  const int qrow = kBlock * i + 16 * w + l16;  // this lane's query token
  const int32_t* lut = A.lut + ((size_t)bh * A.T + i) * A.topk;

  // Q operand (B of S^T = K Q^T): query qrow, features 32g..32g+31 (FP8) or 32s+8g.. (bf16)
  i32x8 q8op;
  bf16x8 qop[4];
  float qscale = 1.f;
  if constexpr (FP8) {
    const uint8_t* src = A.q8 + (((size_t)bh * A.T * kBlock) + qrow) * D + 32 * g;
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint4 b = *reinterpret_cast<const uint4*>(src + 16);
    q8op = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    qscale = A.q_scale[(size_t)bh * A.T + i];
  }
  {
    // bf16 Q: sparse operand in native mode, phi(Q) input in both modes
    const bool ok = qrow < A.N;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 a = ok ? *reinterpret_cast<const uint4*>(A.q + ((size_t)bh * A.N + qrow) * D + 32 * s + 8 * g)
                         : uint4{0, 0, 0, 0};
      qop[s] = __builtin_bit_cast(bf16x8, a);
    }
  }
  const float c0 = kLog2e / sqrtf((float)D);

  f32x4 acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  float cacc[2][4][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) cacc[mt][s][e] = 0.f;
  float cz = 0.f;
  const bf16x2 one_lo = __builtin_bit_cast(bf16x2, 0x00003F80u);
  const bf16x2 one_hi = __builtin_bit_cast(bf16x2, 0x3F800000u);

  {
    TileRegs<FP8> r0;
    load_tile<FP8>(A, bh, lut[0], tid, r0);
    store_tile<FP8>(smem, tid, r0);
  }
  __syncthreads();

  for (int r = 0; r < A.topk; ++r) {
    const int j = lut[r];
    const uint8_t* stage = smem + (r & 1) * L::STAGE;
    TileRegs<FP8> nxt;
    const bool more = r + 1 < A.topk;
    if (more) load_tile<FP8>(A, bh, lut[r + 1], tid, nxt);

    // linear statistics of this routed block
    uint4 hw[2][4];
    {
      const uint16_t* hj = A.h + ((size_t)bh * A.T + j) * D * D;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          hw[mt][s] = *reinterpret_cast<const uint4*>(hj + (size_t)(32 * w + 16 * mt + l16) * D + 32 * s + 8 * g);
    }
    float zj = 0.f;
    if (tid < D) zj = A.z[((size_t)bh * A.T + j) * D + tid];

    // S^T tiles: keys 16mt + 4g + rr (rows) x queries l16 (columns)
    f32x4 S[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint8_t* krow = stage + (16 * mt + l16) * L::KSTR;
      if constexpr (FP8) {
        const uint4 a = *reinterpret_cast<const uint4*>(krow + 32 * g);
        const uint4 b = *reinterpret_cast<const uint4*>(krow + 32 * g + 16);
        const i32x8 kop = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
        S[mt] = mfma_fp8(kop, q8op, f32x4{0.f, 0.f, 0.f, 0.f});
      } else {
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 a = *reinterpret_cast<const uint4*>(krow + 64 * s + 16 * g);
          sacc = mfma_bf16(__builtin_bit_cast(bf16x8, a), qop[s], sacc);
        }
        S[mt] = sacc;
      }
    }
    float cj = c0;
    if constexpr (FP8) cj = c0 * qscale * A.k_scale[(size_t)bh * A.T + j];
    const int nvalid = min(kBlock, A.N - kBlock * j);
    if (nvalid < kBlock) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (16 * mt + 4 * g + rr >= nvalid) S[mt][rr] = -INFINITY;
    }

    // online softmax for this lane's query
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, S[mt][rr]);
    mx = rows4_max(mx);
    const float m_new = fmaxf(m_run, mx * cj);
    if (m_new > m_run) {
      const float f = exp2f(m_run - m_new);
      l_run *= f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= f;
      m_run = m_new;
    }
    float p[4][4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        p[mt][rr] = exp2f(fmaf(S[mt][rr], cj, -m_run));
        psum += p[mt][rr];
      }
    l_run += psum;
    bf16x8 pop[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t wds[4] = {pack_bf16x2(p[2 * s][0], p[2 * s][1]), pack_bf16x2(p[2 * s][2], p[2 * s][3]),
                         pack_bf16x2(p[2 * s + 1][0], p[2 * s + 1][1]),
                         pack_bf16x2(p[2 * s + 1][2], p[2 * s + 1][3])};
      pop[s] = __builtin_bit_cast(bf16x8, wds);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint8_t* vrow = stage + L::KTILE + (16 * dt + l16) * L::VSTR;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 a = *reinterpret_cast<const uint4*>(vrow + 64 * s + 16 * g);
        acc[dt] = mfma_bf16(__builtin_bit_cast(bf16x8, a), pop[s], acc[dt]);
      }
    }
    // C += h_j (bf16 -> fp32 through dot2 with (1,0) and (0,1)), c += z_j
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t wv[4] = {hw[mt][s].x, hw[mt][s].y, hw[mt][s].z, hw[mt][s].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = __builtin_bit_cast(bf16x2, wv[e]);
          cacc[mt][s][2 * e] = __builtin_amdgcn_fdot2_f32_bf16(pr, one_lo, cacc[mt][s][2 * e], false);
          cacc[mt][s][2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, one_hi, cacc[mt][s][2 * e + 1], false);
        }
      }
    cz += zj;

    if (more) store_tile<FP8>(smem + ((r + 1) & 1) * L::STAGE, tid, nxt);
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  const float l_tot = rows4_sum(l_run);
  const float inv_l = 1.f / l_tot;

  // H_i^T = h_sum - C (bf16, rows c, columns a) and Z_i = z_sum - c into LDS
  uint8_t* Hs = smem;
  float* Zs = reinterpret_cast<float*>(smem + 128 * L::HSTR);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int cr = 32 * w + 16 * mt + l16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* hs = A.h_sum + ((size_t)bh * D + cr) * D + 32 * s + 8 * g;
      const float4 x0 = *reinterpret_cast<const float4*>(hs);
      const float4 x1 = *reinterpret_cast<const float4*>(hs + 4);
      uint4 st;
      st.x = pack_bf16x2(x0.x - cacc[mt][s][0], x0.y - cacc[mt][s][1]);
      st.y = pack_bf16x2(x0.z - cacc[mt][s][2], x0.w - cacc[mt][s][3]);
      st.z = pack_bf16x2(x1.x - cacc[mt][s][4], x1.y - cacc[mt][s][5]);
      st.w = pack_bf16x2(x1.z - cacc[mt][s][6], x1.w - cacc[mt][s][7]);
      *reinterpret_cast<uint4*>(Hs + cr * L::HSTR + 64 * s + 16 * g) = st;
    }
  }
  if (tid < D) Zs[tid] = A.z_sum[(size_t)bh * D + tid] - cz;

  // phi(Q) for this lane's query over its 32 features a = 32s + 8g + e
  float qf[4][8];
  float qmax = -INFINITY;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 wv = __builtin_bit_cast(uint4, qop[s]);
    const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[s][2 * e] = bf16_lo(ww[e]);
      qf[s][2 * e + 1] = bf16_hi(ww[e]);
      qmax = fmaxf(qmax, fmaxf(qf[s][2 * e], qf[s][2 * e + 1]));
    }
  }
  qmax = rows4_max(qmax);
  float qsum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qf[s][e] = exp2f((qf[s][e] - qmax) * kLog2e);
      qsum += qf[s][e];
    }
  qsum = rows4_sum(qsum);
  const float qinv = 1.f / qsum;
  __syncthreads();   // H^T and Z in LDS
  bf16x8 phop[4];
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t wds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wds[e] = pack_bf16x2(qf[s][2 * e] * qinv, qf[s][2 * e + 1] * qinv);
      den = fmaf(bf16_lo(wds[e]), Zs[32 * s + 8 * g + 2 * e], den);
      den = fmaf(bf16_hi(wds[e]), Zs[32 * s + 8 * g + 2 * e + 1], den);
    }
    phop[s] = __builtin_bit_cast(bf16x8, wds);
  }
  den = rows4_sum(den) + A.eps;
  const float inv_den = 1.f / den;

  const bool qok = qrow < A.N;
  const float* al = A.alpha + (size_t)hidx * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    f32x4 ol = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t* hrow = Hs + (16 * dt + l16) * L::HSTR;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 a = *reinterpret_cast<const uint4*>(hrow + 64 * s + 16 * g);
      ol = mfma_bf16(__builtin_bit_cast(bf16x8, a), phop[s], ol);
    }
    const float4 a4 = *reinterpret_cast<const float4*>(al + 16 * dt + 4 * g);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
    float ov[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      ov[rr] = av[rr] * (acc[dt][rr] * inv_l) + (1.f - av[rr]) * (ol[rr] * inv_den);
    if (qok) {
      uint2 st;
      st.x = pack_bf16x2(ov[0], ov[1]);
      st.y = pack_bf16x2(ov[2], ov[3]);
      *reinterpret_cast<uint2*>(A.o + ((size_t)bh * A.N + qrow) * D + 16 * dt + 4 * g) = st;
    }
  }
  if (A.lse != nullptr) {
    // native mode scored the raw keys: log-sum-exp over K~ = K - mu is lower by q.mu/sqrt(d)
    float shift = 0.f;
    if constexpr (!FP8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 wv = __builtin_bit_cast(uint4, qop[s]);
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
        const float* mu = A.k_mean + (size_t)bh * D + 32 * s + 8 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          shift = fmaf(bf16_lo(ww[e]), mu[2 * e], shift);
          shift = fmaf(bf16_hi(ww[e]), mu[2 * e + 1], shift);
        }
      }
      shift = rows4_sum(shift) * (1.f / sqrtf((float)D));
    }
    if (g == 0 && qok) A.lse[(size_t)bh * A.N + qrow] = (m_run + log2f(l_tot)) * kLn2 - shift;
  }
}

// ---------------------------------------------------------------------------------------
// fp32, d in {64, 128}: same method with plain fp32 arithmetic.  One workgroup per
// (head, query block); 4 threads (a quad) per query, each owning D/4 output features.
// ---------------------------------------------------------------------------------------
template <int D>
struct F32Lds {
  static constexpr int TILE = 64 * D;           // floats
  static constexpr int FLOATS = 2 * TILE + 64 * D + D;
};

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                      const float* __restrict__ v, const int32_t* __restrict__ lutp,
                                                      const float* __restrict__ h, const float* __restrict__ z,
                                                      const float* __restrict__ h_sum,
                                                      const float* __restrict__ z_sum,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ k_mean, float* __restrict__ o,
                                                      float* __restrict__ lse, int N, int T, int H, int topk,
                                                      float eps) {
  constexpr int DQ = D / 4;
  __shared__ float smem[F32Lds<D>::FLOATS];
  float* Ks = smem;
  float* Vs = smem + F32Lds<D>::TILE;
  float* Ps = smem + 2 * F32Lds<D>::TILE;   // phi(Q) rows
  float* Zs = Ps + 64 * D;
  float* Hs = smem;                          // epilogue: H_i^T [D][D] over Ks and Vs

  const int bh = blockIdx.y, i = blockIdx.x, tid = threadIdx.x;
  const int ql = tid >> 2, part = tid & 3, d0 = part * DQ;
  const int qrow = kBlock * i + ql;
  const bool qok = qrow < N;
  const int32_t* lut = lutp + ((size_t)bh * T + i) * topk;
  const float c0 = kLog2e / sqrtf((float)D);

  float qv[DQ], acc[DQ];
#pragma unroll
  for (int x = 0; x < DQ; ++x) {
    qv[x] = qok ? q[((size_t)bh * N + qrow) * D + d0 + x] : 0.f;
    acc[x] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  for (int r = 0; r < topk; ++r) {
    const int j = lut[r];
    for (int x = tid; x < 64 * D; x += 256) {
      const int t = x / D, col = x % D, tok = kBlock * j + t;
      const bool ok = tok < N;
      Ks[x] = ok ? k[((size_t)bh * N + tok) * D + col] : 0.f;
      Vs[x] = ok ? v[((size_t)bh * N + tok) * D + col] : 0.f;
    }
    __syncthreads();
    const int nvalid = min(kBlock, N - kBlock * j);
    float sc[64];
    float mx = -INFINITY;
    for (int t = 0; t < 64; ++t) {
      float part_s = 0.f;
#pragma unroll
      for (int x = 0; x < DQ; ++x) part_s = fmaf(qv[x], Ks[t * D + d0 + x], part_s);
      part_s += dpp<0xB1>(part_s);
      part_s += dpp<0x4E>(part_s);
      sc[t] = t < nvalid ? part_s * c0 : -INFINITY;
      mx = fmaxf(mx, sc[t]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float f = exp2f(m_run - m_new);
    l_run *= f;
#pragma unroll
    for (int x = 0; x < DQ; ++x) acc[x] *= f;
    m_run = m_new;
    for (int t = 0; t < 64; ++t) {
      const float p = exp2f(sc[t] - m_run);
      l_run += p;
#pragma unroll
      for (int x = 0; x < DQ; ++x) acc[x] = fmaf(p, Vs[t * D + d0 + x], acc[x]);
    }
    __syncthreads();
  }

  // H_i^T = h_sum - sum over routed h_j ([c][a] layout), Z_i likewise
  for (int e = tid; e < D * D; e += 256) {
    float s = h_sum[(size_t)bh * D * D + e];
    for (int r = 0; r < topk; ++r) s -= h[((size_t)bh * T + lut[r]) * D * D + e];
    Hs[e] = s;
  }
  for (int a = tid; a < D; a += 256) {
    float s = z_sum[(size_t)bh * D + a];
    for (int r = 0; r < topk; ++r) s -= z[((size_t)bh * T + lut[r]) * D + a];
    Zs[a] = s;
  }
  // phi(Q) of this query into LDS
  float mq = -INFINITY;
#pragma unroll
  for (int x = 0; x < DQ; ++x) mq = fmaxf(mq, qv[x]);
  mq = fmaxf(mq, dpp<0xB1>(mq));
  mq = fmaxf(mq, dpp<0x4E>(mq));
  float sq = 0.f;
#pragma unroll
  for (int x = 0; x < DQ; ++x) sq += expf(qv[x] - mq);
  sq += dpp<0xB1>(sq);
  sq += dpp<0x4E>(sq);
#pragma unroll
  for (int x = 0; x < DQ; ++x) Ps[ql * D + d0 + x] = expf(qv[x] - mq) / sq;
  __syncthreads();

  float den = 0.f;
#pragma unroll
  for (int x = 0; x < DQ; ++x) den = fmaf(Ps[ql * D + d0 + x], Zs[d0 + x], den);
  den += dpp<0xB1>(den);
  den += dpp<0x4E>(den);
  den += eps;
  const float l_tot = l_run;
  const float* al = alpha + (size_t)(bh % H) * D;
#pragma unroll
  for (int x = 0; x < DQ; ++x) {
    const int cc = d0 + x;
    float num = 0.f;
    for (int a = 0; a < D; ++a) num = fmaf(Ps[ql * D + a], Hs[cc * D + a], num);
    const float os = acc[x] / l_tot, olin = num / den;
    if (qok) o[((size_t)bh * N + qrow) * D + cc] = al[cc] * os + (1.f - al[cc]) * olin;
  }
  if (lse != nullptr) {
    // the scores used the raw keys: shift the log-sum-exp to the smoothed keys K - mu
    float shift = 0.f;
#pragma unroll
    for (int x = 0; x < DQ; ++x) shift = fmaf(qv[x], k_mean[(size_t)bh * D + d0 + x], shift);
    shift += dpp<0xB1>(shift);
    shift += dpp<0x4E>(shift);
    if (part == 0 && qok) lse[(size_t)bh * N + qrow] = (m_run + log2f(l_tot)) * kLn2 - shift / sqrtf((float)D);
  }
}

hipError_t launch_fwd(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s) {
  if (g.bf16) {
    FwdArgs A;
    A.q = (const uint16_t*)t.q;
    A.k = (const uint16_t*)t.k;
    A.q8 = t.q8;
    A.k8 = t.k8;
    A.q_scale = t.q_scale;
    A.k_scale = t.k_scale;
    A.vt = ws.vt;
    A.lut = t.lut;
    A.h = (const uint16_t*)t.h;
    A.z = t.z;
    A.h_sum = t.h_sum;
    A.z_sum = t.z_sum;
    A.alpha = t.alpha;
    A.k_mean = t.k_mean;
    A.o = (uint16_t*)t.o;
    A.lse = t.lse;
    A.N = g.N;
    A.T = g.T;
    A.H = g.H;
    A.topk = g.topk;
    A.nblocks = g.BH * g.T;
    A.eps = g.eps;
    if (g.fp8)
      hipLaunchKernelGGL(fwd_mfma_kernel<true>, dim3(A.nblocks), dim3(256), 0, s, A);
    else
      hipLaunchKernelGGL(fwd_mfma_kernel<false>, dim3(A.nblocks), dim3(256), 0, s, A);
  } else {
    dim3 grid(g.T, g.BH);
    if (g.D == 128)
      hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(256), 0, s, (const float*)t.q, (const float*)t.k,
                         (const float*)t.v, t.lut, (const float*)t.h, t.z, t.h_sum, t.z_sum, t.alpha,
                         t.k_mean, (float*)t.o, t.lse, g.N, g.T, g.H, g.topk, g.eps);
    else
      hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(256), 0, s, (const float*)t.q, (const float*)t.k,
                         (const float*)t.v, t.lut, (const float*)t.h, t.z, t.h_sum, t.z_sum, t.alpha,
                         t.k_mean, (float*)t.o, t.lse, g.N, g.T, g.H, g.topk, g.eps);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Diagnostic: one wave, one matrix-core instruction, C = 0.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void selftest_mfma_kernel(int which, const uint4* a, const uint4* b, float4* d) {
  const int l = threadIdx.x;
  f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
  if (which == 0) {
    r = mfma_bf16(__builtin_bit_cast(bf16x8, a[l]), __builtin_bit_cast(bf16x8, b[l]), r);
  } else {
    const uint4 a0 = a[2 * l], a1 = a[2 * l + 1], b0 = b[2 * l], b1 = b[2 * l + 1];
    const i32x8 ao = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 bo = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    r = mfma_fp8(ao, bo, r);
  }
  d[l] = make_float4(r[0], r[1], r[2], r[3]);
}

hipError_t launch_selftest_mfma(int which, const void* a, const void* b, float* d, hipStream_t s) {
  hipLaunchKernelGGL(selftest_mfma_kernel, dim3(1), dim3(64), 0, s, which, (const uint4*)a, (const uint4*)b,
                     (float4*)d);
  return hipGetLastError();
}

}  // namespace sla2
