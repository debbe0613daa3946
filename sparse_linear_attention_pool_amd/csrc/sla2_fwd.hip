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
  const uint8_t* phik8;   // [BH, T*64, D] e4m3 codes of phi(K~)
  const float* phik_scale;  // [BH, T]
  const int32_t* lut;     // [BH, T, topk]
  const float* h_sum;     // [BH, D, D]
  const float* z_sum;     // [BH, D]
  const float* alpha;     // [H, D]
  const float* k_mean;    // [BH, D] (lse of the native mode is shifted to the smoothed keys)
  uint16_t* o;            // [BH, N, D]
  float* lse;             // [BH, N] or null
  int N, T, H, topk, nblocks;
  float eps;
};

// LDS geometry of one staged key block (bytes).  Rows are stored unpadded with the 16-byte
// chunks of each row permuted (physical chunk = logical chunk XOR (row mod 8), mod 16 for
// 256-byte rows), so that the 16-byte operand reads of 8 consecutive lanes (8 consecutive
// rows, same logical chunk) hit distinct banks.
template <bool FP8>
struct FwdLds {
  static constexpr int KROW = FP8 ? 128 : 256;    // one key row: 128 e4m3 codes or 128 bf16
  static constexpr int KTILE = 64 * KROW;
  static constexpr int PTILE = 64 * 128;          // e4m3 codes of phi(K~): 64 keys x 128
  static constexpr int VTILE = 128 * 128;         // V^T: 128 rows (features) x 64 bf16 keys
  static constexpr int POFF = KTILE, VOFF = KTILE + PTILE;
  static constexpr int STAGE = KTILE + PTILE + VTILE;
  static constexpr int BYTES = 2 * STAGE;         // the tile being read, the tile being written
  static constexpr int KLOADS = KTILE / 4096;     // 16-byte loads per thread per tile part
  static constexpr int PLOADS = PTILE / 4096;
  static constexpr int VLOADS = VTILE / 4096;
  static_assert(128 * 256 + 512 <= BYTES, "epilogue H^T tile must fit in the staging buffers");
};

// Barrier for LDS hand-offs inside the routed-block loop: this wave's LDS writes are retired,
// then all waves meet.  Unlike __syncthreads() it does not drain the vector-memory loads in
// flight (the prefetched tile), which the compiler waits for where they are used.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 0xF | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// This thread's share of one key block's tiles, in registers.
template <bool FP8>
struct TileRegs {
  u32x4 kk[FwdLds<FP8>::KLOADS];
  u32x4 pp[FwdLds<FP8>::PLOADS];
  u32x4 vv[FwdLds<FP8>::VLOADS];
};

// Thread tid moves the 16-byte chunks q = tid + 256p: K row q / (chunks per row), logical
// chunk q % (chunks per row); phi(K~) codes row q / 8, chunk q % 8; V^T row q / 8, chunk q % 8.
template <bool FP8>
__device__ __forceinline__ void load_tile(const FwdArgs& A, int bh, int j, int tid, TileRegs<FP8>& t) {
  using L = FwdLds<FP8>;
  constexpr int D = 128;
  static_for<L::KLOADS>([&](auto P) {
    const int qd = tid + 256 * P;
    if constexpr (FP8) {
      const int row = qd >> 3, lc = qd & 7;
      t.kk[P] = *reinterpret_cast<const u32x4*>(A.k8 + (((size_t)bh * A.T + j) * kBlock + row) * D + 16 * lc);
    } else {
      const int row = qd >> 4, lc = qd & 15;
      const int tok = min(kBlock * j + row, A.N - 1);   // rows past N: any finite row, masked later
      t.kk[P] = *reinterpret_cast<const u32x4*>(A.k + ((size_t)bh * A.N + tok) * D + 8 * lc);
    }
  });
  static_for<L::PLOADS>([&](auto P) {
    const int qd = tid + 256 * P, row = qd >> 3, lc = qd & 7;
    t.pp[P] = *reinterpret_cast<const u32x4*>(A.phik8 + (((size_t)bh * A.T + j) * kBlock + row) * D + 16 * lc);
  });
  static_for<L::VLOADS>([&](auto P) {
    const int qd = tid + 256 * P, row = qd >> 3, lc = qd & 7;
    t.vv[P] = *reinterpret_cast<const u32x4*>(A.vt + (((size_t)bh * A.T + j) * D + row) * kBlock + 8 * lc);
  });
}

template <bool FP8>
__device__ __forceinline__ void store_tile(uint8_t* stage, int tid, const TileRegs<FP8>& t) {
  using L = FwdLds<FP8>;
  static_for<L::KLOADS>([&](auto P) {
    const int qd = tid + 256 * P;
    if constexpr (FP8) {
      const int row = qd >> 3, lc = qd & 7;
      *reinterpret_cast<u32x4*>(stage + row * L::KROW + 16 * (lc ^ (row & 7))) = t.kk[P];
    } else {
      const int row = qd >> 4, lc = qd & 15;
      *reinterpret_cast<u32x4*>(stage + row * L::KROW + 16 * (lc ^ (row & 15))) = t.kk[P];
    }
  });
  static_for<L::PLOADS>([&](auto P) {
    const int qd = tid + 256 * P, row = qd >> 3, lc = qd & 7;
    *reinterpret_cast<u32x4*>(stage + L::POFF + row * 128 + 16 * (lc ^ (row & 7))) = t.pp[P];
  });
  static_for<L::VLOADS>([&](auto P) {
    const int qd = tid + 256 * P, row = qd >> 3, lc = qd & 7;
    *reinterpret_cast<u32x4*>(stage + L::VOFF + row * 128 + 16 * (lc ^ (row & 7))) = t.vv[P];
  });
}

// 32 e4m3 codes of one 128-byte LDS row (logical chunks 2g and 2g+1): the A operand of a
// 16x16x128 matrix-core product for row `row`.
__device__ __forceinline__ i32x8 lds_fp8_row(const uint8_t* base, int row, int g) {
  const uint8_t* r = base + row * 128;
  const u32x4 a = *reinterpret_cast<const u32x4*>(r + 16 * ((2 * g) ^ (row & 7)));
  const u32x4 b = *reinterpret_cast<const u32x4*>(r + 16 * ((2 * g + 1) ^ (row & 7)));
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

constexpr int kLutCache = 512;   // routed blocks whose index and scales are cached in LDS

// Per-lane state of the routed-block loop (one query per lane, see the kernel comment).
struct FwdState {
  f32x4 acc[8];          // O_s^T: sum_s p_s V_s, features 16dt + 4g + rr
  f32x4 accl[8];         // sum over routed keys of (phi(q).phi(k_s)) V_s, same layout
  float m_run, l_run;    // running max (log2 units) and this lane's partial sum of p
  float a_run;           // this lane's partial sum of phi(q).phi(k_s) over routed keys
};

// One routed block, the r-th LUT entry, whose tile is in LDS stage r % 2.  t holds the tile
// of block r+1 (loaded one iteration earlier); at the end it goes to the other stage and t is
// refilled with the tile of block r+2.  mask: the block may be partial (only the last LUT
// entry can be: LUT rows are ascending and only block T-1 is partial).
template <bool FP8, bool LUT_LDS>
__device__ __forceinline__ void fwd_iteration(const FwdArgs& A, FwdState& st, uint8_t* smem, const int* lutS,
                                              const float* kscS, const float* pscS, const int32_t* lutG, int r,
                                              int topk, int bh, int l16, int g, int tid, const i32x8& q8op,
                                              const bf16x8 (&qop)[4], const i32x8& phq8op, float cq, float cphq,
                                              bool mask, TileRegs<FP8>& t) {
  using L = FwdLds<FP8>;
  // the LUT row comes from the LDS cache, or from global memory when it is longer than the
  // cache (a separate instantiation, so no load ever has to serve both address spaces)
  auto lut_at = [&](int x) {
    if constexpr (LUT_LDS) return lutS[x];
    else return lutG[x];
  };
  const int j = lut_at(r);
  const uint8_t* stage = smem + (r & 1) * L::STAGE;

  // ---- S^T = K_j Q^T and Ph^T = phi(K_j) phi(Q)^T: keys 16mt + 4g + rr x queries l16.
  // Operand reads run one key tile ahead of the matrix-core products (read tile mt+1, then
  // multiply tile mt); the scheduling fences keep the compiler from hoisting every read,
  // which would hold all operands of the block in registers at once.
  f32x4 S[4], Ph[4];
  if constexpr (FP8) {
    i32x8 ka = lds_fp8_row(stage, l16, g), pa = lds_fp8_row(stage + L::POFF, l16, g);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      i32x8 kb = ka, pb = pa;
      if (mt < 3) {
        kb = lds_fp8_row(stage, 16 * (mt + 1) + l16, g);
        pb = lds_fp8_row(stage + L::POFF, 16 * (mt + 1) + l16, g);
      }
      S[mt] = mfma_fp8(ka, q8op, f32x4{0.f, 0.f, 0.f, 0.f});
      Ph[mt] = mfma_fp8(pa, phq8op, f32x4{0.f, 0.f, 0.f, 0.f});
      __builtin_amdgcn_sched_barrier(0);
      ka = kb;
      pa = pb;
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 16 * mt + l16;
      const uint8_t* krow = stage + row * L::KROW;
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 16 * ((4 * s + g) ^ (row & 15)));
        sacc = mfma_bf16(__builtin_bit_cast(bf16x8, a), qop[s], sacc);
      }
      S[mt] = sacc;
      Ph[mt] = mfma_fp8(lds_fp8_row(stage + L::POFF, row, g), phq8op, f32x4{0.f, 0.f, 0.f, 0.f});
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float cj = cq, pj;
  if constexpr (LUT_LDS) {
    if constexpr (FP8) cj = cq * kscS[r];
    pj = cphq * pscS[r];
  } else {
    if constexpr (FP8) cj = cq * A.k_scale[(size_t)bh * A.T + j];
    pj = cphq * A.phik_scale[(size_t)bh * A.T + j];
  }
  if (mask) {   // phi codes of keys past N are zero already; only the scores need it
    const int nvalid = min(kBlock, A.N - kBlock * j);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (16 * mt + 4 * g + rr >= nvalid) S[mt][rr] = -INFINITY;
  }

  // ---- online softmax for this lane's query.  The running max is only raised when the
  // block max exceeds it by more than 8 (log2 units), so p <= 256; the rescale is skipped
  // by the whole wave when no lane needs it.
  float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                   fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
  mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(S[2][0], S[2][1]), fmaxf(S[2][2], S[2][3])),
                       fmaxf(fmaxf(S[3][0], S[3][1]), fmaxf(S[3][2], S[3][3]))));
  mx = rows4_max(mx) * cj;
  const bool raise = mx > st.m_run + 8.f;
  if (__builtin_amdgcn_ballot_w64(raise) != 0) {
    const float mnew = raise ? mx : st.m_run;
    const float f = __builtin_amdgcn_exp2f(st.m_run - mnew);
    st.l_run *= f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acc[dt] *= f;
    st.m_run = mnew;
  }
  float psum = 0.f, asum = 0.f;
  bf16x8 pop[2], aop[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float pv[8], av[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        pv[4 * h + rr] = __builtin_amdgcn_exp2f(fmaf(S[2 * s + h][rr], cj, -st.m_run));
        av[4 * h + rr] = Ph[2 * s + h][rr] * pj;
        psum += pv[4 * h + rr];
        asum += av[4 * h + rr];
      }
    const uint32_t pw[4] = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                            pack_bf16x2(pv[6], pv[7])};
    const uint32_t aw[4] = {pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]), pack_bf16x2(av[4], av[5]),
                            pack_bf16x2(av[6], av[7])};
    pop[s] = __builtin_bit_cast(bf16x8, pw);
    aop[s] = __builtin_bit_cast(bf16x8, aw);
  }
  st.l_run += psum;
  st.a_run += asum;

  // ---- O_s^T += V^T P^T and O_corr^T += V^T Ph^T, sharing each V^T operand read; reads run
  // one feature tile ahead of the products
  auto vread = [&](int dt, int s) {
    const int row = 16 * dt + l16;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stage + L::VOFF + row * 128 +
                                                                     16 * ((4 * s + g) ^ (row & 7))));
  };
  bf16x8 v0 = vread(0, 0), v1 = vread(0, 1);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    bf16x8 n0 = v0, n1 = v1;
    if (dt < 7) {
      n0 = vread(dt + 1, 0);
      n1 = vread(dt + 1, 1);
    }
    st.acc[dt] = mfma_bf16(v0, pop[0], st.acc[dt]);
    st.accl[dt] = mfma_bf16(v0, aop[0], st.accl[dt]);
    st.acc[dt] = mfma_bf16(v1, pop[1], st.acc[dt]);
    st.accl[dt] = mfma_bf16(v1, aop[1], st.accl[dt]);
    __builtin_amdgcn_sched_barrier(0);
    v0 = n0;
    v1 = n1;
  }

  // ---- the tile of block r+1 goes to the other stage (its previous tile, block r-1, was
  // consumed before the last barrier); t is refilled with the tile of block r+2
  if (r + 1 < topk) store_tile<FP8>(smem + ((r + 1) & 1) * L::STAGE, tid, t);
  if (r + 2 < topk) load_tile<FP8>(A, bh, lut_at(r + 2), tid, t);
  lds_barrier();
}

// One workgroup (4 waves) per (head, query block).  Wave w owns queries 16w..16w+15 and
// computes S^T = K_j Q_w^T so that each lane holds one query (l % 16) and 16 of the block's
// keys (16mt + 4(l/16) + rr): the softmax state is per lane, and P feeds the P.V product as
// the B operand of O^T = V^T P^T without a transpose.
// The linear branch needs, for the unrouted blocks, phi(q) H_i and phi(q).Z_i with
// H_i = h_sum - sum over routed j of h_j.  The routed part phi(q) h_j = (phi(q) phi(K_j)^T) V_j
// is evaluated by re-association over the same routed keys and V^T tiles as the sparse
// branch, with phi(K~) and phi(q) as e4m3 codes (phi(q) scaled per query).
// Pipeline per routed block r: compute on the LDS tile of block r, write the tile of block
// r+1 (loaded one iteration earlier) to the other LDS stage, load the tile of block r+2.
template <bool FP8, bool LUT_LDS>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(FwdArgs A) {
  using L = FwdLds<FP8>;
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::BYTES];
  __shared__ int lutS[kLutCache];
  __shared__ float kscS[kLutCache];
  __shared__ float pscS[kLutCache];

  const int lid = xcd_remap(blockIdx.x, A.nblocks);
  const int bh = lid / A.T, i = lid % A.T;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int hidx = bh % A.H;
  const int qrow = kBlock * i + 16 * w + l16;  // this lane's query token
  const bool qok = qrow < A.N;
  const int32_t* lutG = A.lut + ((size_t)bh * A.T + i) * A.topk;
  const int topk = A.topk;

  if constexpr (LUT_LDS) {
    for (int x = tid; x < topk; x += 256) {
      const int j = lutG[x];
      lutS[x] = j;
      if constexpr (FP8) kscS[x] = A.k_scale[(size_t)bh * A.T + j];
      pscS[x] = A.phik_scale[(size_t)bh * A.T + j];
    }
  }
  __syncthreads();
  auto lut0 = [&](int x) {
    if constexpr (LUT_LDS) return lutS[x];
    else return lutG[x];
  };
  // the last routed block is partial iff it is block T-1 and N is not a multiple of 64
  const bool last_partial = (lut0(topk - 1) == A.T - 1) && (A.N % kBlock != 0);

  // prologue: tile of block 0 -> registers (-> LDS stage 0 below), then tile of block 1
  TileRegs<FP8> t;
  load_tile<FP8>(A, bh, lut0(0), tid, t);

  // Q operands (B of S^T = K Q^T): FP8 codes of features 32g..32g+31, or bf16 features 32s+8g+e
  i32x8 q8op = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  bf16x8 qop[4];
  float cq = kLog2e / sqrtf((float)D);
  if constexpr (FP8) {
    const uint8_t* src = A.q8 + (((size_t)bh * A.T * kBlock) + qrow) * D + 32 * g;
    const u32x4 a = *reinterpret_cast<const u32x4*>(src);
    const u32x4 b = *reinterpret_cast<const u32x4*>(src + 16);
    q8op = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    cq *= A.q_scale[(size_t)bh * A.T + i];
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 a = qok ? *reinterpret_cast<const u32x4*>(A.q + ((size_t)bh * A.N + qrow) * D + 32 * s + 8 * g)
                          : u32x4{0, 0, 0, 0};
      qop[s] = __builtin_bit_cast(bf16x8, a);
    }
  }
  // phi(q) as e4m3 codes of features 32g..32g+31 with one max/448 scale for this query
  i32x8 phq8op;
  float cphq;
  {
    float x[32];
    const uint16_t* qsrc = A.q + ((size_t)bh * A.N + qrow) * D + 32 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = qok ? *reinterpret_cast<const u32x4*>(qsrc + 8 * c) : u32x4{0, 0, 0, 0};
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = bf16_lo(vw[e]);
        x[8 * c + 2 * e + 1] = bf16_hi(vw[e]);
      }
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, x[e]);
    mx = rows4_max(mx);
    float sm = 0.f, pmx = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = __builtin_amdgcn_exp2f((x[e] - mx) * kLog2e);
      sm += x[e];
      pmx = fmaxf(pmx, x[e]);
    }
    sm = rows4_sum(sm);
    pmx = rows4_max(pmx) / sm;                 // max of phi(q)
    float sp = __fdiv_rn(pmx, kFp8Max);
    if (!(sp > 0.f)) sp = 1.f;
    const float inv = 1.f / (sm * sp);          // code = phi / sp = e / (sum * sp)
    uint32_t wds[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      wds[c] = pack_fp8x4(clamp_fp8(x[4 * c] * inv), clamp_fp8(x[4 * c + 1] * inv), clamp_fp8(x[4 * c + 2] * inv),
                          clamp_fp8(x[4 * c + 3] * inv));
    phq8op = i32x8{(int)wds[0], (int)wds[1], (int)wds[2], (int)wds[3], (int)wds[4], (int)wds[5], (int)wds[6], (int)wds[7]};
    cphq = sp;
  }

  FwdState st;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.accl[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.a_run = 0.f;

  store_tile<FP8>(smem, tid, t);
  if (topk > 1) load_tile<FP8>(A, bh, lut0(1), tid, t);
  lds_barrier();

  for (int r = 0; r < topk; ++r)
    fwd_iteration<FP8, LUT_LDS>(A, st, smem, lutS, kscS, pscS, lutG, r, topk, bh, l16, g, tid, q8op, qop, phq8op, cq,
                                cphq, last_partial && r == topk - 1, t);

  // ---------------- epilogue ----------------
  const float l_tot = rows4_sum(st.l_run);
  const float a_tot = rows4_sum(st.a_run);
  const float inv_l = 1.f / l_tot;

  // H^T = h_sum (bf16, rows c, columns a; 256-byte rows, chunk k stored at k ^ (row % 16)) and
  // Z = z_sum into LDS; every wave needs all of them.
  uint8_t* Hs = smem;
  float* Zs = reinterpret_cast<float*>(smem + 128 * 256);
  {
    const float* hsum = A.h_sum + (size_t)bh * D * D;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int qd = tid + 256 * p;          // 8 features of row qd / 16, chunk qd % 16
      const int cr = qd >> 4, ch = qd & 15;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(hsum + cr * D + 8 * ch);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(hsum + cr * D + 8 * ch + 4);
      u32x4 hv;
      hv.x = pack_bf16x2(x0.x, x0.y);
      hv.y = pack_bf16x2(x0.z, x0.w);
      hv.z = pack_bf16x2(x1.x, x1.y);
      hv.w = pack_bf16x2(x1.z, x1.w);
      *reinterpret_cast<u32x4*>(Hs + cr * 256 + 16 * (ch ^ (cr & 15))) = hv;
    }
    if (tid < D) Zs[tid] = A.z_sum[(size_t)bh * D + tid];
  }
  // phi(q) in bf16 as the B operand of O_l^T = H^T phi(Q)^T: features a = 32s + 8g + e
  float qf[4][8];
  {
    float qmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = qok ? *reinterpret_cast<const u32x4*>(A.q + ((size_t)bh * A.N + qrow) * D + 32 * s + 8 * g)
                          : u32x4{0, 0, 0, 0};
      const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
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
        qf[s][e] = __builtin_amdgcn_exp2f((qf[s][e] - qmax) * kLog2e);
        qsum += qf[s][e];
      }
    qsum = rows4_sum(qsum);
    const float qinv = 1.f / qsum;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] *= qinv;
  }
  __syncthreads();   // H^T and Z in LDS
  bf16x8 phop[4];
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t wds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wds[e] = pack_bf16x2(qf[s][2 * e], qf[s][2 * e + 1]);
      den = fmaf(bf16_lo(wds[e]), Zs[32 * s + 8 * g + 2 * e], den);
      den = fmaf(bf16_hi(wds[e]), Zs[32 * s + 8 * g + 2 * e + 1], den);
    }
    phop[s] = __builtin_bit_cast(bf16x8, wds);
  }
  // denominator over the unrouted keys: phi(q).Z_tot - sum over routed keys of phi(q).phi(k)
  den = rows4_sum(den) - a_tot + A.eps;
  const float inv_den = 1.f / den;

  const float* al = A.alpha + (size_t)hidx * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    f32x4 ol = f32x4{0.f, 0.f, 0.f, 0.f};
    const int hr = 16 * dt + l16;
    const uint8_t* hrow = Hs + hr * 256;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(hrow + 16 * ((4 * s + g) ^ (hr & 15)));
      ol = mfma_bf16(__builtin_bit_cast(bf16x8, a), phop[s], ol);
    }
    const f32x4 a4 = *reinterpret_cast<const f32x4*>(al + 16 * dt + 4 * g);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
    float ov[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      ov[rr] = av[rr] * (st.acc[dt][rr] * inv_l) + (1.f - av[rr]) * ((ol[rr] - st.accl[dt][rr]) * inv_den);
    if (qok) {
      u32x2 sv;
      sv.x = pack_bf16x2(ov[0], ov[1]);
      sv.y = pack_bf16x2(ov[2], ov[3]);
      *reinterpret_cast<u32x2*>(A.o + ((size_t)bh * A.N + qrow) * D + 16 * dt + 4 * g) = sv;
    }
  }
  if (A.lse != nullptr) {
    // native mode scored the raw keys: log-sum-exp over K~ = K - mu is lower by q.mu/sqrt(d)
    float shift = 0.f;
    if constexpr (!FP8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 wv = __builtin_bit_cast(u32x4, qop[s]);
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
    if (g == 0 && qok) A.lse[(size_t)bh * A.N + qrow] = (st.m_run + log2f(l_tot)) * kLn2 - shift;
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
    A.phik8 = ws.phik8;
    A.phik_scale = ws.phik_scale;
    A.lut = t.lut;
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
    const bool lds_lut = g.topk <= kLutCache;
    if (g.fp8) {
      if (lds_lut) hipLaunchKernelGGL((fwd_mfma_kernel<true, true>), dim3(A.nblocks), dim3(256), 0, s, A);
      else hipLaunchKernelGGL((fwd_mfma_kernel<true, false>), dim3(A.nblocks), dim3(256), 0, s, A);
    } else {
      if (lds_lut) hipLaunchKernelGGL((fwd_mfma_kernel<false, true>), dim3(A.nblocks), dim3(256), 0, s, A);
      else hipLaunchKernelGGL((fwd_mfma_kernel<false, false>), dim3(A.nblocks), dim3(256), 0, s, A);
    }
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
__global__ __launch_bounds__(64) void selftest_mfma_kernel(int which, const u32x4* a, const u32x4* b, float4* d) {
  const int l = threadIdx.x;
  f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
  if (which == 2) {
    const f64x4 r64 = mfma_f64(reinterpret_cast<const double*>(a)[l], reinterpret_cast<const double*>(b)[l],
                               f64x4{0.0, 0.0, 0.0, 0.0});
    double* d64 = reinterpret_cast<double*>(d);
    d64[4 * l + 0] = r64[0];
    d64[4 * l + 1] = r64[1];
    d64[4 * l + 2] = r64[2];
    d64[4 * l + 3] = r64[3];
    return;
  }
  if (which == 0) {
    r = mfma_bf16(__builtin_bit_cast(bf16x8, a[l]), __builtin_bit_cast(bf16x8, b[l]), r);
  } else {
    const u32x4 a0 = a[2 * l], a1 = a[2 * l + 1], b0 = b[2 * l], b1 = b[2 * l + 1];
    const i32x8 ao = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 bo = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    r = mfma_fp8(ao, bo, r);
  }
  d[l] = make_float4(r[0], r[1], r[2], r[3]);
}

hipError_t launch_selftest_mfma(int which, const void* a, const void* b, void* d, hipStream_t s) {
  hipLaunchKernelGGL(selftest_mfma_kernel, dim3(1), dim3(64), 0, s, which, (const u32x4*)a, (const u32x4*)b,
                     (float4*)d);
  return hipGetLastError();
}

}  // namespace sla2
