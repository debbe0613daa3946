// SLA2 backward pass (bf16 inputs, FP8 e4m3 Q.K^T forward, d = 128): dQ, dK, dV, dalpha of
// L = sum(dO * O) with the routing held fixed.
//
// Pages: "SLA2: Sparse-Linear Attention with Learnable Routing and QAT", section 3 (O =
// alpha * O_s + (1 - alpha) * O_l), section 5 (QAT: low-bit forward, 16-bit backward),
// appendix A (gradients of Q, K, V, phi(Q), phi(K) derived by hand; dH_i, dZ_i formed per query
// block and accumulated for each key block over the query blocks that do not route to it);
// "SLA: Beyond Sparsity in Diffusion Transformers...", section 4 (the sparse branch follows
// the FlashAttention backward; the linear branch goes through dH_i, dZ_i, symmetric to the
// forward).  Straight-through quantiser: dQ' passes to Q and dK' to K~.
//
// Per query block i (bwd_query_kernel), over its routed key blocks:
//   pass A: S = Q' K'^T / sqrt(d), P = exp(S - lse), O_s = P V, then Dq = rowsum(dO_s * O_s);
//   linear: H_i, Z_i (totals minus the routed h_j, z_j), O_l, dalpha, dnum = dO_l / den,
//           dden = -(dO_l . O_l) / den, dphi(q) = dnum H_i^T + dden Z_i, dH_i = phi(q)^T dnum,
//           dZ_i = dden^T phi(q);
//   pass B: dP = dO_s V^T, dS = P (dP - Dq), dQ' = dS K' / sqrt(d).
// Per key block j (bwd_key_kernel), over the query blocks that route to it:
//   dV = P^T dO_s, dK' = dS^T Q' / sqrt(d); linear: dh_j = dH_tot - sum of dH_i over those
//   query blocks (the rest are the ones that do not route to j), dz_j likewise,
//   dphi(k) = V dh_j^T + dz_j, dV += phi(k) dh_j.
// Then dK = dK~ - mean over tokens (key smoothing) and dalpha summed over tokens and batch.
//
// Matrix products run on the bf16 16x16x32 matrix cores (the scores on the e4m3 16x16x128
// ones, exactly as the forward computed them) with both operands read from LDS tiles that hold
// the contraction index contiguous: A as rows of the left factor, B as rows of the right
// factor's transpose.  Tiles are staged synchronously; this first version favours a plain
// structure over overlap.
#include <math.h>

#include "sla2_device.hpp"
#include "sla2_internal.hpp"

namespace sla2 {

namespace {

constexpr int kD = 128;
constexpr int kNT = 256;

// Row-major LDS tile of RB-byte rows whose 16-byte chunks are XOR-swizzled by the row index:
// 16 lanes reading one chunk column of 16 consecutive rows hit distinct banks.
template <int RB>
struct LTile {
  uint8_t* p;
  __device__ __forceinline__ uint8_t* chunk(int r, int c) const {
    constexpr int NC = RB / 16;
    return p + r * RB + 16 * (c ^ (r & (NC - 1)));
  }
  __device__ __forceinline__ uint16_t* el16(int r, int e) const {   // bf16 element e of row r
    return reinterpret_cast<uint16_t*>(chunk(r, e >> 3)) + (e & 7);
  }
  __device__ __forceinline__ bf16x8 op(int r, int k0) const {       // 8 bf16 from element k0
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(chunk(r, k0 >> 3)));
  }
  __device__ __forceinline__ i32x8 op8(int r, int g) const {        // 32 e4m3 codes, bytes 32g..
    const u32x4 a = *reinterpret_cast<const u32x4*>(chunk(r, 2 * g));
    const u32x4 b = *reinterpret_cast<const u32x4*>(chunk(r, 2 * g + 1));
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
};

// rows x RB bytes from global rows of stride ld bytes; rows >= nvalid are zero
template <int RB>
__device__ __forceinline__ void stage(LTile<RB> dst, const uint8_t* src, size_t ld, int rows, int nvalid, int tid) {
  constexpr int NC = RB / 16;
  for (int x = tid; x < rows * NC; x += kNT) {
    const int r = x / NC, c = x % NC;
    const u32x4 v = r < nvalid ? *reinterpret_cast<const u32x4*>(src + (size_t)r * ld + 16 * c) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(dst.chunk(r, c)) = v;
  }
}

// D(16 x 16) += A(16 x K) B(K x 16), A rows m0.. of At (k contiguous), B^T rows n0.. of Bt
template <int K, int RBA, int RBB>
__device__ __forceinline__ f32x4 mm(const LTile<RBA>& At, int m0, const LTile<RBB>& Bt, int n0, int l16, int g,
                                    f32x4 c) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) c = mfma_bf16(At.op(m0 + l16, k0 + 8 * g), Bt.op(n0 + l16, k0 + 8 * g), c);
  return c;
}

// e4m3 (OCP: bias 7, no infinities, 0x7f / 0xff NaN never produced by the quantiser)
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e ? ldexpf(1.f + 0.125f * (float)m, (int)e - 7) : ldexpf((float)m, -9);
  return (b & 0x80u) ? -mag : mag;
}

// column position of key (or query) x of a 64-block in the forward's V^T tiles: within each
// 32-half, keys 4gg + e sit at 8gg + e and keys 16 + 4gg + e at 8gg + 4 + e
__device__ __forceinline__ int vt_pos(int x) {
  const int s = x >> 5, rem = x & 31, h = rem >> 4, gg = (rem & 15) >> 2, e = rem & 3;
  return 32 * s + 8 * gg + 4 * h + e;
}

struct BwdArgs {
  const uint16_t* q;       // bf16 [BH, N, D]
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* alpha;      // [H, D]
  const float* k_mean;     // [BH, D]
  const uint8_t* q8;       // [BH, 64T, D]
  const uint8_t* k8;
  const float* q_scale;    // [BH, T]
  const float* k_scale;
  const float* lse;        // [BH, N]
  const int32_t* lut;      // [BH, T, topk]
  const uint8_t* mask;     // [BH, T, T]
  const uint16_t* h;       // bf16 [BH, T, D, D], h[j][c][a]
  const float* z;          // [BH, T, D]
  const float* h_sum;      // [BH, D, D] (transposed like h)
  const float* z_sum;      // [BH, D]
  const uint16_t* vt;      // forward workspace: [BH, T, D, 64] V^T tiles, keys at vt_pos
  // backward workspace
  uint16_t* dos;           // [BH, 64T, D] alpha * dO (rows past N zero)
  uint16_t* dot;           // [BH, T, D, 64] dos transposed
  uint16_t* qt;            // [BH, T, D, 64] Q'^T (dequantised e4m3)
  uint16_t* kt;            // [BH, T, D, 64] K'^T
  int32_t* inv;            // [BH, T, T] query blocks routing to key block j, ascending
  int32_t* inv_cnt;        // [BH, T]
  float* dsum;             // [BH, 64T] rowsum(dO_s * O_s)
  float* dH;               // [BH, T, D, D] dH_i[a][c]
  float* dZ;               // [BH, T, D]
  float* dH_tot;           // [BH, D, D]
  float* dZ_tot;           // [BH, D]
  float* dalpha_part;      // [BH, T, D]
  float* dkt;              // [BH, 64T, D] dK~ (fp32)
  float* colsum_part;      // [BH, NCH, D]
  float* dk_mean;          // [BH, D]
  // outputs
  uint16_t* dq;            // bf16 [BH, N, D]
  uint16_t* dk;
  uint16_t* dv;
  float* dalpha;           // [H, D]
  int B, H, N, T, topk, nch;
  float eps;
  int smooth_k;
};

// ---------------------------------------------------------------------------------------
// Per (head, 64-token block b): alpha * dO rows and their transpose, and the transposed
// dequantised e4m3 tiles of Q and K~.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs A) {
  __shared__ uint16_t tr[kD * 64];   // [row c][col x], plain row-major
  const int b = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, hidx = bh % A.H;
  const int x = tid >> 2, c0 = 32 * (tid & 3);   // token x of the block, features c0..c0+31
  const int tok = 64 * b + x;
  const size_t row = (size_t)bh * A.T * 64 + tok;
  auto flush = [&](uint16_t* dst) {   // tr -> dst[bh][b][c][x], 16-byte chunks
    __syncthreads();
    uint16_t* base = dst + ((size_t)bh * A.T + b) * kD * 64;
    for (int e = tid; e < kD * 64 / 8; e += kNT)
      reinterpret_cast<u32x4*>(base)[e] = reinterpret_cast<const u32x4*>(tr)[e];
    __syncthreads();
  };
  // alpha * dO
  {
    uint16_t out[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int c = c0 + e;
      float val = 0.f;
      if (tok < A.N) val = A.alpha[(size_t)hidx * kD + c] * bf16_to_f32(A.dout[((size_t)bh * A.N + tok) * kD + c]);
      out[e] = f32_to_bf16(val);
      tr[c * 64 + x] = out[e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      reinterpret_cast<u32x4*>(A.dos + row * kD + c0)[u] = reinterpret_cast<const u32x4*>(out)[u];
    flush(A.dot);
  }
  // Q' and K' = e4m3 code * block scale (pad rows hold code 0)
  for (int which = 0; which < 2; ++which) {
    const uint8_t* codes = (which == 0 ? A.q8 : A.k8) + row * kD + c0;
    const float sc = (which == 0 ? A.q_scale : A.k_scale)[(size_t)bh * A.T + b];
#pragma unroll
    for (int e = 0; e < 32; ++e) tr[(c0 + e) * 64 + x] = f32_to_bf16(e4m3_value(codes[e]) * sc);
    flush(which == 0 ? A.qt : A.kt);
  }
}

// Query blocks that route to key block j, ascending: one wave per (head, j) scans column j of
// the mask with ballots.
__global__ __launch_bounds__(64) void bwd_invlut_kernel(BwdArgs A) {
  const int j = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const uint8_t* col = A.mask + (size_t)bh * A.T * A.T + j;
  int32_t* out = A.inv + ((size_t)bh * A.T + j) * A.T;
  int base = 0;
  for (int i0 = 0; i0 < A.T; i0 += 64) {
    const int i = i0 + lane;
    const bool on = i < A.T && col[(size_t)i * A.T] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
    if (on) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = i;
    base += __popcll(bal);
  }
  if (lane == 0) A.inv_cnt[(size_t)bh * A.T + j] = base;
}

// ---------------------------------------------------------------------------------------
// Query side.  Wave w owns queries 16w..16w+15 of block i; results in the matrix-core output
// layout: lane (g = l/16, l16 = l%16) holds rows 16w + 4g + r (r < 4) of column l16 of each
// 16-wide column tile.
// ---------------------------------------------------------------------------------------
namespace qlds {
constexpr int QS = 0;                 // Q8 rows of block i        64 x 128 B
constexpr int DOS = QS + 8192;        // alpha * dO rows           64 x 256 B
constexpr int SMALL = DOS + 16384;    // lse, Dq, den, m, 1/s, dden, Z_i, alpha partials
constexpr int U = SMALL + 4096;       // union of the phases
// sparse phases
constexpr int PS = U;                 // P or dS                   64 x 128 B
constexpr int KS = PS + 8192;         // K8 rows of block j        64 x 128 B
constexpr int VT = KS + 8192;         // V^T (forward tile)        128 x 128 B
constexpr int VS = VT + 16384;        // V rows                    64 x 256 B
constexpr int KT = VS + 16384;        // K'^T                      128 x 128 B
// linear phase
constexpr int HT = U;                 // H_i^T [c][a]              128 x 256 B
constexpr int HN = HT + 32768;        // H_i [a][c]                128 x 256 B
constexpr int PHQ = HN + 32768;       // phi(q) [q][a]             64 x 256 B
constexpr int PHQT = PHQ + 16384;     // phi(q)^T [a][q]           128 x 128 B
constexpr int DNUM = PHQT + 16384;    // dnum [q][c]               64 x 256 B
constexpr int DNUMT = DNUM + 16384;   // dnum^T [c][q]             128 x 128 B
constexpr int BYTES = DNUMT + 16384;
static_assert(KT + 16384 <= BYTES, "sparse phase fits the union");
}  // namespace qlds

__global__ __launch_bounds__(256, 1) void bwd_query_kernel(BwdArgs A) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[qlds::BYTES];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4, hidx = bh % A.H;
  const int q0 = 16 * w;
  const int T = A.T, topk = A.topk;
  float* lseS = reinterpret_cast<float*>(sm + qlds::SMALL);
  float* dqS = lseS + 64;
  float* denS = dqS + 64;
  float* mqS = denS + 64;
  float* isS = mqS + 64;
  float* ddenS = isS + 64;
  float* ZS = ddenS + 64;            // 128
  float* alS = ZS + 128;             // 4 x 128
  const LTile<128> QS{sm + qlds::QS}, PS{sm + qlds::PS}, KS{sm + qlds::KS}, VT{sm + qlds::VT}, KT{sm + qlds::KT};
  const LTile<256> DOS{sm + qlds::DOS}, VS{sm + qlds::VS}, HT{sm + qlds::HT}, HN{sm + qlds::HN},
      PHQ{sm + qlds::PHQ}, DNUM{sm + qlds::DNUM};
  const LTile<128> PHQT{sm + qlds::PHQT}, DNUMT{sm + qlds::DNUMT};
  const int32_t* lut = A.lut + ((size_t)bh * T + i) * topk;
  const float inv_sqrt_d = 1.f / sqrtf((float)kD);
  const int nq = min(64, A.N - 64 * i);   // valid queries of this block

  stage<128>(QS, A.q8 + ((size_t)bh * T * 64 + 64 * i) * kD, kD, 64, 64, tid);
  stage<256>(DOS, reinterpret_cast<const uint8_t*>(A.dos + ((size_t)bh * T * 64 + 64 * i) * kD), 2 * kD, 64, 64, tid);
  if (tid < 64) lseS[tid] = tid < nq ? A.lse[(size_t)bh * A.N + 64 * i + tid] : 0.f;
  __syncthreads();
  const float qsc = A.q_scale[(size_t)bh * T + i];

  // scores of this wave's queries against key block j: S[nt] = 16 x 16 tiles (keys 16nt..)
  auto scores = [&](int j, f32x4 (&S)[4]) {
    const float cj = kLog2e * inv_sqrt_d * qsc * A.k_scale[(size_t)bh * T + j];
    const int nk = min(64, A.N - 64 * j);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 s = mfma_fp8(QS.op8(q0 + l16, g), KS.op8(16 * nt + l16, g), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = q0 + 4 * g + r, key = 16 * nt + l16;
        const bool ok = qq < nq && key < nk;
        s[r] = ok ? __builtin_amdgcn_exp2f(s[r] * cj - lseS[qq] * kLog2e) : 0.f;   // P
      }
      S[nt] = s;
    }
  };

  // ---------------- pass A: O_s and Dq
  f32x4 os[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) os[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < topk; ++r) {
    const int j = lut[r];
    stage<128>(KS, A.k8 + ((size_t)bh * T * 64 + 64 * j) * kD, kD, 64, 64, tid);
    stage<128>(VT, reinterpret_cast<const uint8_t*>(A.vt + ((size_t)bh * T + j) * kD * 64), 128, 128, 128, tid);
    __syncthreads();
    f32x4 P[4];
    scores(j, P);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) *PS.el16(q0 + 4 * g + rr, vt_pos(16 * nt + l16)) = f32_to_bf16(P[nt][rr]);
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) os[nt] = mm<64>(PS, q0, VT, 16 * nt, l16, g, os[nt]);
    __syncthreads();
  }
  // Dq = sum_c dO_s * O_s
  {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part[rr] += bf16_to_f32(*DOS.el16(q0 + 4 * g + rr, 16 * nt + l16)) * os[nt][rr];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float dsum = row16_sum(part[rr]);
      if (l16 == 0) {
        dqS[q0 + 4 * g + rr] = dsum;
        if (q0 + 4 * g + rr < nq) A.dsum[(size_t)bh * T * 64 + 64 * i + q0 + 4 * g + rr] = dsum;
      }
    }
  }

  // ---------------- linear branch
  // Z_i and H_i^T: totals minus the routed blocks
  if (tid < kD) {
    float zz = A.z_sum[(size_t)bh * kD + tid];
    for (int r = 0; r < topk; ++r) zz -= A.z[((size_t)bh * T + lut[r]) * kD + tid];
    ZS[tid] = zz;
  }
  {
    const int c = tid >> 1, a0 = 64 * (tid & 1);
    float hh[64];
    const float* hs = A.h_sum + (size_t)bh * kD * kD + c * kD + a0;
#pragma unroll
    for (int e = 0; e < 64; ++e) hh[e] = hs[e];
    for (int r = 0; r < topk; ++r) {
      const u32x4* hj = reinterpret_cast<const u32x4*>(A.h + (((size_t)bh * T + lut[r]) * kD + c) * kD + a0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4 wv = hj[u];
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hh[8 * u + 2 * e] -= bf16_lo(ww[e]);
          hh[8 * u + 2 * e + 1] -= bf16_hi(ww[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const uint16_t bv = f32_to_bf16(hh[e]);
      *HT.el16(c, a0 + e) = bv;
      *HN.el16(a0 + e, c) = bv;
    }
  }
  __syncthreads();
  // phi(q): four threads per query row (32 features each); den = phi(q).Z_i + eps
  {
    const int qq = tid >> 2, a0 = 32 * (tid & 3);
    const int tok = min(64 * i + qq, A.N - 1);
    const uint16_t* qr = A.q + ((size_t)bh * A.N + tok) * kD + a0;
    float x[32];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = bf16_to_f32(qr[e]);
      mx = fmaxf(mx, x[e]);
    }
    mx = fmaxf(mx, dpp<0xB1>(mx));
    mx = fmaxf(mx, dpp<0x4E>(mx));
    float sm_ = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = __expf(x[e] - mx);
      sm_ += x[e];
    }
    sm_ += dpp<0xB1>(sm_);
    sm_ += dpp<0x4E>(sm_);
    const float is = 1.f / sm_;
    float dz = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float ph = x[e] * is;
      dz = fmaf(ph, ZS[a0 + e], dz);
      const uint16_t bv = f32_to_bf16(ph);
      *PHQ.el16(qq, a0 + e) = bv;
      *PHQT.el16(a0 + e, qq) = bv;
    }
    dz += dpp<0xB1>(dz);
    dz += dpp<0x4E>(dz);
    if ((tid & 3) == 0) {
      denS[qq] = dz + A.eps;
      mqS[qq] = mx;
      isS[qq] = is;
    }
  }
  __syncthreads();
  // O_l, dalpha, dnum, dden.  With every block routed the linear branch is an empty sum: O_l
  // and its gradients are 0 (the complement form would leave rounding amplified by 1/eps).
  const bool lin = topk < T;
  {
    float alp[4][8], ddp[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) ddp[rr] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
      num = mm<128>(PHQ, q0, HT, 16 * nt, l16, g, num);
      const int c = 16 * nt + l16;
      const float al = A.alpha[(size_t)hidx * kD + c];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int qq = q0 + 4 * g + rr;
        const bool ok = qq < nq;
        const float den = denS[qq];
        const float ol = lin ? num[rr] / den : 0.f;
        const float dO = ok ? bf16_to_f32(A.dout[((size_t)bh * A.N + 64 * i + qq) * kD + c]) : 0.f;
        alp[rr][nt] = dO * (os[nt][rr] - ol);
        const float dol = (1.f - al) * dO;
        const float dn = lin ? dol / den : 0.f;
        ddp[rr] = fmaf(-dol, ol, ddp[rr]);
        const uint16_t bv = f32_to_bf16(dn);
        *DNUM.el16(qq, c) = bv;
        *DNUMT.el16(c, qq) = bv;
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float t = row16_sum(ddp[rr]);
      if (l16 == 0) ddenS[q0 + 4 * g + rr] = t / denS[q0 + 4 * g + rr];
    }
    // dalpha partial of this wave: sum over its 16 queries, per feature
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float t = rows4_sum(alp[0][nt] + alp[1][nt] + alp[2][nt] + alp[3][nt]);
      if (g == 0) alS[w * kD + 16 * nt + l16] = t;
    }
  }
  __syncthreads();
  if (tid < kD)
    A.dalpha_part[((size_t)bh * T + i) * kD + tid] = (alS[tid] + alS[kD + tid]) + (alS[2 * kD + tid] + alS[3 * kD + tid]);
  // dphi(q) = dnum H_i^T + dden Z_i, then the softmax backward -> dq (linear part)
  f32x4 dql[8];
  {
    float dphi[8][4], ph[8][4], dot_[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
      t = mm<128>(DNUM, q0, HN, 16 * nt, l16, g, t);
      const int a = 16 * nt + l16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int qq = q0 + 4 * g + rr;
        const int tok = min(64 * i + qq, A.N - 1);
        dphi[nt][rr] = t[rr] + ddenS[qq] * ZS[a];
        ph[nt][rr] = __expf(bf16_to_f32(A.q[((size_t)bh * A.N + tok) * kD + a]) - mqS[qq]) * isS[qq];
        dot_[rr] = fmaf(ph[nt][rr], dphi[nt][rr], dot_[rr]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) dot_[rr] = row16_sum(dot_[rr]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dql[nt][rr] = ph[nt][rr] * (dphi[nt][rr] - dot_[rr]);
  }
  // dH_i = phi(q)^T dnum (wave w: rows a of tiles 2w, 2w+1), dZ_i = dden^T phi(q)
  {
    float* dHi = A.dH + ((size_t)bh * T + i) * kD * kD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int a0 = 16 * (2 * w + mt);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
        t = mm<64>(PHQT, a0, DNUMT, 16 * nt, l16, g, t);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) dHi[(size_t)(a0 + 4 * g + rr) * kD + 16 * nt + l16] = t[rr];
      }
    }
    if (tid < kD) {
      float zz = 0.f;
      for (int qq = 0; qq < nq; ++qq) {
        const float ph = __expf(bf16_to_f32(A.q[((size_t)bh * A.N + 64 * i + qq) * kD + tid]) - mqS[qq]) * isS[qq];
        zz = fmaf(ddenS[qq], ph, zz);
      }
      A.dZ[((size_t)bh * T + i) * kD + tid] = zz;
    }
  }
  __syncthreads();

  // ---------------- pass B: dQ' = dS K' / sqrt(d)
  f32x4 dqs[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) dqs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < topk; ++r) {
    const int j = lut[r];
    const int nk = min(64, A.N - 64 * j);
    stage<128>(KS, A.k8 + ((size_t)bh * T * 64 + 64 * j) * kD, kD, 64, 64, tid);
    stage<256>(VS, reinterpret_cast<const uint8_t*>(A.v + ((size_t)bh * A.N + 64 * j) * kD), 2 * kD, 64, nk, tid);
    stage<128>(KT, reinterpret_cast<const uint8_t*>(A.kt + ((size_t)bh * T + j) * kD * 64), 128, 128, 128, tid);
    __syncthreads();
    f32x4 P[4];
    scores(j, P);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
      dp = mm<128>(DOS, q0, VS, 16 * nt, l16, g, dp);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int qq = q0 + 4 * g + rr;
        *PS.el16(qq, 16 * nt + l16) = f32_to_bf16(P[nt][rr] * (dp[rr] - dqS[qq]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) dqs[nt] = mm<64>(PS, q0, KT, 16 * nt, l16, g, dqs[nt]);
    __syncthreads();
  }

  // dq = dQ' / sqrt(d) + dq (linear)
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int qq = q0 + 4 * g + rr;
      if (qq < nq)
        A.dq[((size_t)bh * A.N + 64 * i + qq) * kD + 16 * nt + l16] = f32_to_bf16(dqs[nt][rr] * inv_sqrt_d + dql[nt][rr]);
    }
}

// ---------------------------------------------------------------------------------------
// Key side.  Wave w owns keys 16w..16w+15 of block j (rows of every product below).
// ---------------------------------------------------------------------------------------
namespace klds {
constexpr int KS = 0;                 // K8 rows of block j        64 x 128 B
constexpr int VS = KS + 8192;         // V rows of block j         64 x 256 B
constexpr int SMALL = VS + 16384;     // lse_i, Dq_i, dz_j, phi(k) max / inverse sums
constexpr int U = SMALL + 4096;
// sparse phase
constexpr int QS = U;                 // Q8 rows of block i        64 x 128 B
constexpr int DOS = QS + 8192;        // alpha * dO rows           64 x 256 B
constexpr int QT = DOS + 16384;       // Q'^T                      128 x 128 B
constexpr int DOT = QT + 16384;       // (alpha * dO)^T            128 x 128 B
constexpr int PS = DOT + 16384;       // P^T [key][q]              64 x 128 B
constexpr int DSS = PS + 8192;        // dS^T [key][q]             64 x 128 B
// linear phase
constexpr int DHN = U;                // dh_j [a][c]               128 x 256 B
constexpr int DHT = DHN + 32768;      // dh_j^T [c][a]             128 x 256 B
constexpr int PHK = DHT + 32768;      // phi(k) [key][a]           64 x 256 B
constexpr int BYTES = PHK + 16384;
static_assert(DSS + 8192 <= BYTES, "sparse phase fits the union");
}  // namespace klds

__global__ __launch_bounds__(256, 1) void bwd_key_kernel(BwdArgs A) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[klds::BYTES];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int k0 = 16 * w;
  const int T = A.T;
  float* lseS = reinterpret_cast<float*>(sm + klds::SMALL);
  float* dqS = lseS + 64;
  float* dzS = dqS + 64;      // 128
  float* mkS = dzS + 128;     // 64
  float* isS = mkS + 64;      // 64
  const LTile<128> KS{sm + klds::KS}, QS{sm + klds::QS}, QT{sm + klds::QT}, DOT{sm + klds::DOT}, PS{sm + klds::PS},
      DSS{sm + klds::DSS};
  const LTile<256> VS{sm + klds::VS}, DOS{sm + klds::DOS}, DHN{sm + klds::DHN}, DHT{sm + klds::DHT},
      PHK{sm + klds::PHK};
  const float inv_sqrt_d = 1.f / sqrtf((float)kD);
  const int nk = min(64, A.N - 64 * j);
  const float ksc = A.k_scale[(size_t)bh * T + j];
  const int cnt = A.inv_cnt[(size_t)bh * T + j];
  const int32_t* inv = A.inv + ((size_t)bh * T + j) * T;

  stage<128>(KS, A.k8 + ((size_t)bh * T * 64 + 64 * j) * kD, kD, 64, 64, tid);
  stage<256>(VS, reinterpret_cast<const uint8_t*>(A.v + ((size_t)bh * A.N + 64 * j) * kD), 2 * kD, 64, nk, tid);

  f32x4 dv[8], dk[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    dv[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dk[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int x = 0; x < cnt; ++x) {
    const int i = inv[x];
    const int nq = min(64, A.N - 64 * i);
    __syncthreads();   // the previous block's tiles are consumed
    stage<128>(QS, A.q8 + ((size_t)bh * T * 64 + 64 * i) * kD, kD, 64, 64, tid);
    stage<256>(DOS, reinterpret_cast<const uint8_t*>(A.dos + ((size_t)bh * T * 64 + 64 * i) * kD), 2 * kD, 64, 64, tid);
    stage<128>(QT, reinterpret_cast<const uint8_t*>(A.qt + ((size_t)bh * T + i) * kD * 64), 128, 128, 128, tid);
    stage<128>(DOT, reinterpret_cast<const uint8_t*>(A.dot + ((size_t)bh * T + i) * kD * 64), 128, 128, 128, tid);
    if (tid < 64) {
      lseS[tid] = tid < nq ? A.lse[(size_t)bh * A.N + 64 * i + tid] : 0.f;
      dqS[tid] = tid < nq ? A.dsum[(size_t)bh * T * 64 + 64 * i + tid] : 0.f;
    }
    __syncthreads();
    const float cij = kLog2e * inv_sqrt_d * ksc * A.q_scale[(size_t)bh * T + i];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 s = mfma_fp8(KS.op8(k0 + l16, g), QS.op8(16 * nt + l16, g), f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
      dp = mm<128>(VS, k0, DOS, 16 * nt, l16, g, dp);
      const int qq = 16 * nt + l16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = k0 + 4 * g + rr;
        const bool ok = qq < nq && key < nk;
        const float p = ok ? __builtin_amdgcn_exp2f(s[rr] * cij - lseS[qq] * kLog2e) : 0.f;
        *PS.el16(key, qq) = f32_to_bf16(p);
        *DSS.el16(key, qq) = f32_to_bf16(p * (dp[rr] - dqS[qq]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      dv[nt] = mm<64>(PS, k0, DOT, 16 * nt, l16, g, dv[nt]);
      dk[nt] = mm<64>(DSS, k0, QT, 16 * nt, l16, g, dk[nt]);
    }
  }
  __syncthreads();

  // ---------------- linear branch
  // dh_j = dH_tot - sum of dH_i over the query blocks routing to j; dz_j likewise
  {
    const int a = tid >> 1, c0 = 64 * (tid & 1);
    float dd[64];
    const float* tot = A.dH_tot + (size_t)bh * kD * kD + a * kD + c0;
#pragma unroll
    for (int e = 0; e < 64; ++e) dd[e] = tot[e];
    for (int x = 0; x < cnt; ++x) {
      const f32x4* di = reinterpret_cast<const f32x4*>(A.dH + (((size_t)bh * T + inv[x]) * kD + a) * kD + c0);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const f32x4 t = di[u];
#pragma unroll
        for (int e = 0; e < 4; ++e) dd[4 * u + e] -= t[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const uint16_t bv = f32_to_bf16(dd[e]);
      *DHN.el16(a, c0 + e) = bv;
      *DHT.el16(c0 + e, a) = bv;
    }
  }
  if (tid < kD) {
    float zz = A.dZ_tot[(size_t)bh * kD + tid];
    for (int x = 0; x < cnt; ++x) zz -= A.dZ[((size_t)bh * T + inv[x]) * kD + tid];
    dzS[tid] = zz;
  }
  // phi(k~): four threads per key row
  const float* mu = A.k_mean + (size_t)bh * kD;
  {
    const int kk = tid >> 2, a0 = 32 * (tid & 3);
    const int tok = min(64 * j + kk, A.N - 1);
    const uint16_t* kr = A.k + ((size_t)bh * A.N + tok) * kD + a0;
    float x[32];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = bf16_to_f32(kr[e]) - mu[a0 + e];
      mx = fmaxf(mx, x[e]);
    }
    mx = fmaxf(mx, dpp<0xB1>(mx));
    mx = fmaxf(mx, dpp<0x4E>(mx));
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = __expf(x[e] - mx);
      s += x[e];
    }
    s += dpp<0xB1>(s);
    s += dpp<0x4E>(s);
    const float is = 1.f / s;
#pragma unroll
    for (int e = 0; e < 32; ++e) *PHK.el16(kk, a0 + e) = f32_to_bf16(kk < nk ? x[e] * is : 0.f);
    if ((tid & 3) == 0) {
      mkS[kk] = mx;
      isS[kk] = is;
    }
  }
  __syncthreads();
  // dphi(k) = V dh_j^T + dz_j -> dk~ (linear part); dV += phi(k) dh_j
  float dkl[8][4];
  {
    float dphi[8][4], ph[8][4], dot_[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
      t = mm<128>(VS, k0, DHN, 16 * nt, l16, g, t);
      dv[nt] = mm<128>(PHK, k0, DHT, 16 * nt, l16, g, dv[nt]);
      const int a = 16 * nt + l16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int kk = k0 + 4 * g + rr;
        const int tok = min(64 * j + kk, A.N - 1);
        dphi[nt][rr] = t[rr] + dzS[a];
        ph[nt][rr] = __expf(bf16_to_f32(A.k[((size_t)bh * A.N + tok) * kD + a]) - mu[a] - mkS[kk]) * isS[kk];
        dot_[rr] = fmaf(ph[nt][rr], dphi[nt][rr], dot_[rr]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) dot_[rr] = row16_sum(dot_[rr]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dkl[nt][rr] = ph[nt][rr] * (dphi[nt][rr] - dot_[rr]);
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int kk = k0 + 4 * g + rr, c = 16 * nt + l16;
      if (kk < nk) {
        A.dv[((size_t)bh * A.N + 64 * j + kk) * kD + c] = f32_to_bf16(dv[nt][rr]);
        A.dkt[((size_t)bh * T * 64 + 64 * j + kk) * kD + c] = dk[nt][rr] * inv_sqrt_d + dkl[nt][rr];
      }
    }
}

// Column sums of dK~ over chunks of 256 tokens, then per head: mean over the N tokens.
__global__ __launch_bounds__(256) void bwd_colsum_kernel(BwdArgs A) {
  __shared__ float red[2][kD];
  const int ch = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c = tid & (kD - 1), half = tid >> 7;
  float s = 0.f;
  const int r0 = 256 * ch, r1 = min(A.N, r0 + 256);
  for (int r = r0 + half; r < r1; r += 2) s += A.dkt[((size_t)bh * A.T * 64 + r) * kD + c];
  red[half][c] = s;
  __syncthreads();
  if (tid < kD) A.colsum_part[((size_t)bh * A.nch + ch) * kD + tid] = red[0][tid] + red[1][tid];
}

// mean over the N tokens of dK~ (zero without key smoothing), from the chunk sums in fixed order
__global__ __launch_bounds__(128) void bwd_mean_kernel(BwdArgs A) {
  const int bh = blockIdx.x, c = threadIdx.x;
  float s = 0.f;
  if (A.smooth_k)
    for (int ch = 0; ch < A.nch; ++ch) s += A.colsum_part[((size_t)bh * A.nch + ch) * kD + c];
  A.dk_mean[(size_t)bh * kD + c] = A.smooth_k ? s / (float)A.N : 0.f;
}

// dK = dK~ - mean: 16 bytes of a row per thread
__global__ __launch_bounds__(256) void bwd_dk_kernel(BwdArgs A) {
  const int bh = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;   // chunk of 8 features
  const int r = e >> 4, c0 = 8 * (e & 15);
  if (r >= A.N) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(A.dkt + ((size_t)bh * A.T * 64 + r) * kD + c0);
  const f32x4* mu = reinterpret_cast<const f32x4*>(A.dk_mean + (size_t)bh * kD + c0);
  const f32x4 a = src[0] - mu[0], b = src[1] - mu[1];
  u32x4 out;
  out.x = pack_bf16x2(a.x, a.y);
  out.y = pack_bf16x2(a.z, a.w);
  out.z = pack_bf16x2(b.x, b.y);
  out.w = pack_bf16x2(b.z, b.w);
  *reinterpret_cast<u32x4*>(A.dk + ((size_t)bh * A.N + r) * kD + c0) = out;
}

// dalpha[h][c] = sum over batch and query blocks of the per-block partials: 8 partial sums
// per feature over interleaved blocks, combined in fixed order
__global__ __launch_bounds__(1024) void bwd_dalpha_kernel(BwdArgs A) {
  __shared__ float red[8][kD];
  const int hidx = blockIdx.x, c = threadIdx.x & (kD - 1), u = threadIdx.x >> 7;
  float s = 0.f;
  for (int b = 0; b < A.B; ++b) {
    const int bh = b * A.H + hidx;
    for (int i = u; i < A.T; i += 8) s += A.dalpha_part[((size_t)bh * A.T + i) * kD + c];
  }
  red[u][c] = s;
  __syncthreads();
  if (u == 0) {
    float t = 0.f;
    for (int k = 0; k < 8; ++k) t += red[k][c];
    A.dalpha[(size_t)hidx * kD + c] = t;
  }
}

}  // namespace

size_t bwd_workspace_layout(const Geometry& g, BwdWorkspace* ws, char* base) {
  const size_t BH = g.BH, T = g.T, D = g.D;
  const size_t nch = (g.N + 255) / 256;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return base ? base + o : nullptr;
  };
  BwdWorkspace w;
  w.dos = (uint16_t*)take(BH * T * 64 * D * 2);
  w.dot = (uint16_t*)take(BH * T * D * 64 * 2);
  w.qt = (uint16_t*)take(BH * T * D * 64 * 2);
  w.kt = (uint16_t*)take(BH * T * D * 64 * 2);
  w.inv = (int32_t*)take(BH * T * T * 4);
  w.inv_cnt = (int32_t*)take(BH * T * 4);
  w.dsum = (float*)take(BH * T * 64 * 4);
  w.dH = (float*)take(BH * T * D * D * 4);
  w.dZ = (float*)take(BH * T * D * 4);
  w.dH_tot = (float*)take(BH * D * D * 4);
  w.dZ_tot = (float*)take(BH * D * 4);
  w.dalpha_part = (float*)take(BH * T * D * 4);
  w.dkt = (float*)take(BH * T * 64 * D * 4);
  w.colsum_part = (float*)take(BH * nch * D * 4);
  w.dk_mean = (float*)take(BH * D * 4);
  if (ws) *ws = w;
  return off;
}

hipError_t launch_bwd(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const BwdWorkspace& bw,
                      const void* dout, void* dq, void* dk, void* dv, float* dalpha, hipStream_t s) {
  BwdArgs A;
  A.q = (const uint16_t*)t.q;
  A.k = (const uint16_t*)t.k;
  A.v = (const uint16_t*)t.v;
  A.dout = (const uint16_t*)dout;
  A.alpha = t.alpha;
  A.k_mean = t.k_mean;
  A.q8 = t.q8;
  A.k8 = t.k8;
  A.q_scale = t.q_scale;
  A.k_scale = t.k_scale;
  A.lse = t.lse;
  A.lut = t.lut;
  A.mask = t.mask;
  A.h = (const uint16_t*)t.h;
  A.z = t.z;
  A.h_sum = t.h_sum;
  A.z_sum = t.z_sum;
  A.vt = ws.vt;
  A.dos = bw.dos;
  A.dot = bw.dot;
  A.qt = bw.qt;
  A.kt = bw.kt;
  A.inv = bw.inv;
  A.inv_cnt = bw.inv_cnt;
  A.dsum = bw.dsum;
  A.dH = bw.dH;
  A.dZ = bw.dZ;
  A.dH_tot = bw.dH_tot;
  A.dZ_tot = bw.dZ_tot;
  A.dalpha_part = bw.dalpha_part;
  A.dkt = bw.dkt;
  A.colsum_part = bw.colsum_part;
  A.dk_mean = bw.dk_mean;
  A.dq = (uint16_t*)dq;
  A.dk = (uint16_t*)dk;
  A.dv = (uint16_t*)dv;
  A.dalpha = dalpha;
  A.B = g.B;
  A.H = g.H;
  A.N = g.N;
  A.T = g.T;
  A.topk = g.topk;
  A.nch = (g.N + 255) / 256;
  A.eps = g.eps;
  A.smooth_k = g.smooth_k ? 1 : 0;
  const dim3 blocks(g.T, g.BH);
  hipLaunchKernelGGL(bwd_prep_kernel, blocks, dim3(256), 0, s, A);
  hipLaunchKernelGGL(bwd_invlut_kernel, blocks, dim3(64), 0, s, A);
  hipLaunchKernelGGL(bwd_query_kernel, blocks, dim3(256), 0, s, A);
  hipError_t e = launch_sum_parts(bw.dH, bw.dZ, g.T, g.D, g.BH, bw.dH_tot, bw.dZ_tot, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_key_kernel, blocks, dim3(256), 0, s, A);
  hipLaunchKernelGGL(bwd_colsum_kernel, dim3(A.nch, g.BH), dim3(256), 0, s, A);
  hipLaunchKernelGGL(bwd_mean_kernel, dim3(g.BH), dim3(128), 0, s, A);
  hipLaunchKernelGGL(bwd_dk_kernel, dim3((g.N * 16 + 255) / 256, g.BH), dim3(256), 0, s, A);
  hipLaunchKernelGGL(bwd_dalpha_kernel, dim3(g.H), dim3(1024), 0, s, A);
  return hipGetLastError();
}

}  // namespace sla2
