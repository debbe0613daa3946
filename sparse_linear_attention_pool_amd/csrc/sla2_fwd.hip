// SLA2 fused forward: for each query block i, over the routed key blocks j in LUT order,
//   S = Q_i K_j^T / sqrt(d) (FP8 e4m3 codes times the two block scales, or bf16),
//   online softmax (running max and sum, exp2 with log2(e) folded into the scale),
//   acc += P V_j (bf16 matrix cores, or e4m3 P and V with power-of-two scales in the low-bit
//   P.V mode);
// then O_s = acc / l and the linear branch over the unrouted blocks,
//   O_l = phi(Q_i) H_i / (phi(Q_i) Z_i + eps), H_i = h_sum - sum_{j routed} h_j, Z_i likewise,
// and O = alpha * O_s + (1 - alpha) * O_l.  The fp32 kernel gathers the routed h_j, z_j.  The
// matrix-core kernel never reads h_j: it adds phi(Q_i) times the routed part of H by
// re-association, sum_{j routed} (phi(Q_i) phi(K~_j)^T) V_j, over the same key and V^T tiles as
// the sparse branch, and takes Z_R(i) = sum_{j routed} z_j from the precompute.  With a large
// share of the blocks routed it sums phi(Q_i) H_i over the unrouted blocks directly instead.
//
// Pages: "SLA2: Sparse-Linear Attention with Learnable Routing and QAT", section 3 (sparse
// attention only where M = 1 on FlashAttention-style computation; linear branch from the
// M = 0 statistics; O = alpha * O_s + (1 - alpha) * O_l), section 5 (low-bit Q.K^T, and P
// and V, with scales), section 6 (M = 1 blocks: sparse scores and values; M = 0 blocks: linear
// statistics); "SLA: Beyond Sparsity in Diffusion Transformers...", section 3 figure
// (O_s = diag(l)^-1 O_acc, O_l = phi(Q_i) H_i / (phi(Q_i) Z_i)), section 4 (online softmax
// with a running max, 1e-5 in the linear denominator), section 7 (the loop walks a LUT of
// routed block indices; exp2 with log2(e) folded into the score scale).
#include <math.h>

#include "sla2_device.hpp"
#include "sla2_internal.hpp"
#include "sla2_lds.hpp"

namespace sla2 {

struct FwdArgs {
  const uint16_t* q;      // bf16 [BH, N, D]
  const uint16_t* k;      // bf16 [BH, N, D] (native Q.K^T only)
  const uint8_t* q8;      // [BH, T*64, D]
  const uint8_t* k8;
  const float* q_scale;   // [BH, T]
  const float* k_scale;
  const uint16_t* vt;     // [BH, T, D, 64] bf16, or e4m3 bytes with low-bit P.V
  const uint16_t* v;      // bf16 [BH, N, D]: V rows, read by the low-bit mode's unrouted-block loop
  const uint8_t* vexp;    // low-bit P.V: [BH, T, D] biased exponents of the V scales
  const uint8_t* phik8;   // [BH, T*64, D] e4m3 codes of 448 phi(K~), features permuted
  const int32_t* lut;     // [BH, T, topk]
  const uint16_t* hbf;    // [BH, D, D] bf16 LDS image of H^T = h_sum (see Workspace::hbf)
  const float* zblk;      // [BH, T, D] z_j of every key block
  float* zrout;           // [BH, T, D] Z_R(i) = sum of z_j over the routed blocks of row i, stored
                          // for the backward pass with os (else unused)
  const float* z_sum;     // [BH, D]
  const float* alpha;     // [H, D]
  const float* k_mean;    // [BH, D] (lse of the native mode is shifted to the smoothed keys)
  uint16_t* o;            // [BH, N, D]
  float* lse;             // [BH, N] or null
  uint16_t* os;           // [BH, N, D] O_s for the backward pass, or null (then ol, inv_den too)
  uint16_t* ol;           // [BH, N, D] O_l
  float* inv_den;         // [BH, 64T] 1 / (phi(q).Z_i + eps)
  int N, T, H, topk, nblocks;
  float eps;
};

// LDS geometry of one staged key block (bytes) for a workgroup of NT threads.  Rows are stored
// unpadded with the 16-byte chunks of each row permuted (physical chunk = logical chunk XOR
// (row mod 8), mod 16 for 256-byte rows), so that the 16-byte operand reads of consecutive
// lanes (consecutive rows, same logical chunk) hit distinct banks.
template <bool FP8, int NT, bool PV8 = false>
struct FwdLds {
  static constexpr int KROW = FP8 ? 128 : 256;    // one key row: 128 e4m3 codes or 128 bf16
  static constexpr int KTILE = 64 * KROW;
  static constexpr int PTILE = 64 * 128;          // e4m3 codes of phi(K~): 64 keys x 128
  // V^T: 128 rows (features) x 64 keys, bf16 (128-byte rows) or e4m3 (64-byte rows, physical
  // chunk = logical chunk XOR ((row / 4) mod 4)), then the 128 exponent bytes of its scales
  static constexpr int VROW = PV8 ? 64 : 128;
  static constexpr int VTILE = 128 * VROW;
  static constexpr int VEBYTES = PV8 ? 128 : 0;
  static constexpr int POFF = KTILE, VOFF = KTILE + PTILE, VEOFF = VOFF + VTILE;
  static constexpr int TILE = VEOFF + VEBYTES;
  static constexpr int STAGE = TILE > 128 * 256 ? TILE : 128 * 256;   // also holds the epilogue's H^T
  static constexpr int KLOADS = KTILE / (16 * NT);   // 16-byte loads per thread per tile part
  static constexpr int PLOADS = PTILE / (16 * NT);
  static constexpr int VLOADS = VTILE / (16 * NT);
};

// This thread's share of one key block's tiles, in registers.
struct TileSrc {
  __amdgpu_buffer_rsrc_t k, phik8, vt, hbf;   // k: e4m3 codes of K~ (FP8) or bf16 K (native)
  __amdgpu_buffer_rsrc_t vexp;                // low-bit P.V: exponents of the V scales
  __amdgpu_buffer_rsrc_t vrows;               // low-bit P.V: the bf16 V rows of this head
};

__device__ __forceinline__ TileSrc tile_src(const FwdArgs& A, int bh) {
  constexpr int D = 128;
  const size_t head = (size_t)bh * A.T * kBlock * D;   // elements of one head's tiles
  const int bytes8 = A.T * kBlock * D;                 // <= 4096 * 8 KB
  TileSrc s;
  s.k = A.k8 != nullptr ? __builtin_amdgcn_make_buffer_rsrc((void*)(A.k8 + head), 0, bytes8, 0x00020000)
                        : __builtin_amdgcn_make_buffer_rsrc((void*)(A.k + (size_t)bh * A.N * D), 0, A.N * D * 2, 0x00020000);
  s.phik8 = __builtin_amdgcn_make_buffer_rsrc((void*)(A.phik8 + head), 0, bytes8, 0x00020000);
  if (A.vexp != nullptr) {   // e4m3 V^T tiles: one byte per element
    s.vt = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)A.vt + head), 0, bytes8, 0x00020000);
    s.vexp = __builtin_amdgcn_make_buffer_rsrc((void*)(A.vexp + (size_t)bh * A.T * D), 0, A.T * D, 0x00020000);
    s.vrows = __builtin_amdgcn_make_buffer_rsrc((void*)(A.v + (size_t)bh * A.N * D), 0, A.N * D * 2, 0x00020000);
  } else {
    s.vt = __builtin_amdgcn_make_buffer_rsrc((void*)(A.vt + head), 0, 2 * bytes8, 0x00020000);
    s.vexp = s.vt;
    s.vrows = s.vt;
  }
  s.hbf = __builtin_amdgcn_make_buffer_rsrc((void*)(A.hbf + (size_t)bh * D * D), 0, 2 * D * D, 0x00020000);
  return s;
}

// The tile of key block j (K, phi(K~) codes, V^T) into the LDS stage at `stage`; without the
// keys (WITH_K false) for the linear branch alone.
template <bool FP8, int NT, bool PV8, bool WITH_K = true>
__device__ __forceinline__ void dma_tile(const FwdArgs& A, const TileSrc& src, int j, int tid, uint8_t* stage) {
  using L = FwdLds<FP8, NT, PV8>;
  constexpr int D = 128;
  const int wofs = 1024 * __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's 1 KB of each group
  if constexpr (WITH_K) static_for<L::KLOADS>([&](auto P) {
    const int qd = tid + NT * P;
    uint8_t* dst = stage + 16 * NT * P + wofs;
    if constexpr (FP8) {
      const int row = qd >> 3, pc = qd & 7;
      lds_dma(src.k, dst, row * 128 + 16 * fp8_chunk(row, pc), j * (kBlock * D));
    } else {
      const int row = qd >> 4, pc = qd & 15;
      const int tok = min(kBlock * j + row, A.N - 1);   // rows past N: any finite row, masked later
      lds_dma(src.k, dst, tok * (2 * D) + 16 * (pc ^ (row & 15)), 0);
    }
  });
  static_for<L::PLOADS>([&](auto P) {
    const int qd = tid + NT * P, row = qd >> 3, pc = qd & 7;
    lds_dma(src.phik8, stage + L::POFF + 16 * NT * P + wofs, row * 128 + 16 * fp8_chunk(row, pc), j * (kBlock * D));
  });
  if constexpr (PV8) {
    static_for<L::VLOADS>([&](auto P) {
      const int qd = tid + NT * P, row = qd >> 2, pc = qd & 3;
      lds_dma(src.vt, stage + L::VOFF + 16 * NT * P + wofs, row * 64 + 16 * (pc ^ ((row >> 2) & 3)), j * (kBlock * D));
    });
    if (tid < L::VEBYTES / 16) lds_dma(src.vexp, stage + L::VEOFF, 16 * tid, j * D);   // wave 0, 8 lanes
  } else {
    static_for<L::VLOADS>([&](auto P) {
      const int qd = tid + NT * P, row = qd >> 3, pc = qd & 7;
      lds_dma(src.vt, stage + L::VOFF + 16 * NT * P + wofs, row * 128 + 16 * (pc ^ (row & 7)), j * (2 * kBlock * D));
    });
  }
}

// What the unrouted-block loop reads of key block j: the phi codes and V.  bf16 modes take the
// V^T tile; the low-bit P.V mode takes the bf16 V rows from the input (256-byte rows, chunk k of
// row r at chunk k ^ (r % 16), in the stage's V region and after it: 16 KB), so that the linear
// branch keeps bf16 V there.  Rows past N load row N-1 (their phi codes are zero).
template <bool FP8, int NT, bool PV8>
__device__ __forceinline__ void dma_lin(const FwdArgs& A, const TileSrc& src, int j, int tid, uint8_t* stage) {
  if constexpr (PV8) {
    using L = FwdLds<FP8, NT, PV8>;
    constexpr int D = 128;
    static_assert(L::VOFF + 64 * 256 <= L::STAGE, "bf16 V rows fit after the phi codes");
    const int wofs = 1024 * __builtin_amdgcn_readfirstlane(tid >> 6);
    static_for<L::PLOADS>([&](auto P) {
      const int qd = tid + NT * P, row = qd >> 3, pc = qd & 7;
      lds_dma(src.phik8, stage + L::POFF + 16 * NT * P + wofs, row * 128 + 16 * fp8_chunk(row, pc), j * (kBlock * D));
    });
    static_for<64 * 256 / (16 * NT)>([&](auto P) {
      const int qd = tid + NT * P, row = qd >> 4, pc = qd & 15;
      const int tok = min(kBlock * j + row, A.N - 1);
      lds_dma(src.vrows, stage + L::VOFF + 16 * NT * P + wofs, tok * (2 * D) + 16 * (pc ^ (row & 15)), 0);
    });
  } else {
    dma_tile<FP8, NT, PV8, false>(A, src, j, tid, stage);
  }
}

// The 32 KB bf16 image of H^T, stored in memory already in its LDS layout, into `dst`.
template <int NT>
__device__ __forceinline__ void dma_himage(const TileSrc& src, int tid, uint8_t* dst) {
  const int wofs = 1024 * __builtin_amdgcn_readfirstlane(tid >> 6);
  static_for<2048 / NT>([&](auto P) { lds_dma(src.hbf, dst + 16 * NT * P + wofs, 16 * (tid + NT * P), 0); });
}

constexpr int kLutReg = 64;   // LUT rows up to this long live in one register (lane x holds entry x)
// LDS operand reads are issued this many matrix-core steps ahead of their use
constexpr int kSReadAhead = 1;   // key-tile rows (S and phi products)
constexpr int kVReadAhead = 3;   // V^T rows (P.V products)

// Entry x of this query block's LUT row: read across lanes from the register copy, or from
// memory when the row is longer than a wave.
template <bool LUT_REG>
__device__ __forceinline__ int lut_entry(int lutv, const int32_t* lutG, int x) {
  if constexpr (LUT_REG) return __builtin_amdgcn_readlane(lutv, x);
  else return __builtin_amdgcn_readfirstlane(lutG[x]);
}

// Per-lane state of the routed-block loop: QT queries per lane (one per 16-query tile).
template <int QT>
struct FwdState {
  f32x4 acc[QT][8];      // O_s^T: sum_s p_s V_s, features 16dt + 4g + rr
  f32x4 accl[QT][8];     // sum over routed keys of (phi(q).phi(k_s)) V_s, same layout
  float m_run[QT];       // running max (log2 units)
  float l_run[QT];       // low-bit P.V: this lane's partial sum of p
  f32x4 lsum[QT];        // bf16 P.V: the sum of the bf16 P over the routed keys (every element
                         // holds the sum for this lane's query), from products with a ones operand
};

// Operands of this lane's queries that stay in registers for the whole loop.
template <int QT>
struct QueryOps {
  i32x8 q8[QT];          // FP8: e4m3 codes of features 32g..32g+31 (B of S^T = K Q^T)
  bf16x8 qb[QT][4];      // native: bf16 features 32s + 8g + e
  i32x8 phq8[QT];        // e4m3 codes of 448 phi(q), features 32s + 8g + e in (s, e) order
  bf16x8 phb[QT][4];     // phi(q) in bf16, same features (B of O_l^T = H^T phi(q)^T)
};

// One routed block, the r-th LUT entry, whose tile is in LDS stage r % 2 and whose K scale is
// ksc.  The copy of the next tile (or, after the last, of the epilogue's H^T image) into the
// other stage runs meanwhile.  mask: the block may be partial (only the last LUT entry can
// be: LUT rows are ascending and only block T-1 is partial).
template <bool FP8, bool LUT_REG, int QT, int STG, bool PV8>
__device__ __forceinline__ void fwd_iteration(const FwdArgs& A, FwdState<QT>& st, uint8_t* smem0, uint8_t* smem1, int lutv,
                                              float& ksc, const int32_t* lutG, int r,
                                              int topk, int bh, int l16, int g, int tid, const QueryOps<QT>& qo,
                                              float cq, bool mask, const TileSrc& src, float& zacc) {
  constexpr int NT = 256 / QT;
  using L = FwdLds<FP8, NT, PV8>;
  constexpr int D = 128;
  // the two stages are separate LDS objects and the stage roles are fixed per instantiation,
  // so the compiler can see that this block's reads never touch the copy in flight
  const uint8_t* stage = STG == 0 ? smem0 : smem1;

  // ---- first, start the copy of the next tile into the other stage, whose previous tile
  // (block r-1) was consumed before the last barrier; it lands while this block is processed
  uint8_t* next = STG == 0 ? smem1 : smem0;
  float ksc_next = 1.f;
  float znext = 0.f;   // z_j of the next block: a load that lands with its tile copy
  if (r + 1 < topk) {
    const int jn = lut_entry<LUT_REG>(lutv, lutG, r + 1);
    if constexpr (FP8) ksc_next = A.k_scale[(size_t)bh * A.T + jn];
    if (tid < D) znext = A.zblk[((size_t)bh * A.T + jn) * D + tid];
    dma_tile<FP8, NT, PV8>(A, src, jn, tid, next);
  } else {
    dma_himage<NT>(src, tid, next);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- S^T = K_j Q^T and Ph^T = phi(K_j) phi(Q)^T: keys 16mt + 4g + rr x queries l16 of each
  // query tile.  Operand reads run one key tile ahead of the matrix-core products; the
  // scheduling fences keep the compiler from hoisting every read, which would hold all
  // operands of the block in registers at once.
  f32x4 S[QT][4], Ph[QT][4];
  if constexpr (FP8) {
    i32x8 kr[4], pr[4];
    static_for<kSReadAhead>([&](auto mt) {
      kr[mt] = lds_fp8_row(stage, 16 * mt + l16, g);
      pr[mt] = lds_fp8_row(stage + L::POFF, 16 * mt + l16, g);
    });
    static_for<4>([&](auto mt) {
      if constexpr (mt + kSReadAhead < 4) {
        kr[mt + kSReadAhead] = lds_fp8_row(stage, 16 * (mt + kSReadAhead) + l16, g);
        pr[mt + kSReadAhead] = lds_fp8_row(stage + L::POFF, 16 * (mt + kSReadAhead) + l16, g);
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        S[qt][mt] = mfma_fp8(kr[mt], qo.q8[qt], f32x4{0.f, 0.f, 0.f, 0.f});
        Ph[qt][mt] = mfma_fp8(pr[mt], qo.phq8[qt], f32x4{0.f, 0.f, 0.f, 0.f});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 16 * mt + l16;
      const uint8_t* krow = stage + row * L::KROW;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) S[qt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 16 * ((4 * s + g) ^ (row & 15)));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) S[qt][mt] = mfma_bf16(__builtin_bit_cast(bf16x8, a), qo.qb[qt][s], S[qt][mt]);
      }
      const i32x8 pa = lds_fp8_row(stage + L::POFF, row, g);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) Ph[qt][mt] = mfma_fp8(pa, qo.phq8[qt], f32x4{0.f, 0.f, 0.f, 0.f});
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float cj = cq;
  if constexpr (FP8) cj = cq * ksc;
  if (mask) {   // phi codes of keys past N are zero already; only the scores need it
    const int nvalid = A.N - kBlock * (A.T - 1);   // only block T-1 can be partial
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (16 * mt + 4 * g + rr >= nvalid) S[qt][mt][rr] = -INFINITY;
  }

  // ---- online softmax, one query per lane and tile.  The running max is only raised when
  // the block max exceeds it by more than 8 (log2 units), so p <= 256; the rescale is skipped
  // by the whole wave when no lane needs it.  With low-bit P.V the running max is raised to an
  // integer (the ceiling of the block max), so every rescale and P scale is a power of two.
  float mx[QT];
  bool raise_any = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // chained three-input maxima over the 16 scores, from -inf (a first two-input max made the
    // compiler quiet both inputs first)
    float m = -INFINITY;
    static_for<8>([&](auto u) {
      constexpr int a = 2 * u, b = 1 + 2 * u;
      m = fmaxf(fmaxf(m, S[qt][a / 4][a % 4]), S[qt][b / 4][b % 4]);
    });
    mx[qt] = rows4_max(m) * cj;
    raise_any = raise_any || (mx[qt] > st.m_run[qt] + 8.f);
  }
  if (__builtin_amdgcn_ballot_w64(raise_any) != 0) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mnew = mx[qt] > st.m_run[qt] + 8.f ? (PV8 ? ceilf(mx[qt]) : mx[qt]) : st.m_run[qt];
      const float f = __builtin_amdgcn_exp2f(st.m_run[qt] - mnew);
      st.l_run[qt] *= f;
      st.lsum[qt] *= f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) st.acc[qt][dt] *= f;
      st.m_run[qt] = mnew;
    }
  }

  if constexpr (PV8) {
    // ---- low-bit P.V (SLA2 page, section 5).  Per query, this block's P is coded as
    // e4m3(2^(x - cb + 8)) with cb = ceil(block max), values up to 256; the normaliser takes
    // the unquantised values.  A (the phi products) is coded with the fixed scale 2^-10.  Each
    // lane's 16 keys fill 16 of the 32 k-positions of its lane group in a 16x16x128 e4m3
    // product (the other 16 are zero), matching the V^T tile's byte order; the matrix cores
    // apply 2^(cb - 8 - m_run) to P and the channel's 2^e to V.
    i32x8 p8[QT], a8[QT];
    int pexp[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float off = ceilf(mx[qt]) - 8.f;
      float psum = 0.f;
      uint32_t pw[4], aw[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float pv[4], av[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pv[rr] = __builtin_amdgcn_exp2f(fmaf(S[qt][mt][rr], cj, -off));
          av[rr] = clamp_fp8(Ph[qt][mt][rr] * 0x1p-10f);
          psum += pv[rr];
        }
        pw[mt] = pack_fp8x4(pv[0], pv[1], pv[2], pv[3]);
        aw[mt] = pack_fp8x4(av[0], av[1], av[2], av[3]);
      }
      p8[qt] = i32x8{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], 0, 0, 0, 0};
      a8[qt] = i32x8{(int)aw[0], (int)aw[1], (int)aw[2], (int)aw[3], 0, 0, 0, 0};
      const int rel = (int)(off - st.m_run[qt]);   // <= 0: m_run >= ceil(block max) - 8
      st.l_run[qt] += __builtin_amdgcn_ldexpf(psum, rel);
      pexp[qt] = rel + 127 > 0 ? rel + 127 : 0;    // E8M0 byte (2^-127 for negligible blocks)
    }
    // O_s^T += V^T P^T and O_corr^T += V^T A^T over the eight feature tiles; the scale byte of
    // channel 16dt + l16 is byte dt of this lane's 8 exponent bytes
    const u32x2 ve = *reinterpret_cast<const u32x2*>(stage + L::VEOFF + 8 * l16);
    auto vread = [&](int dt) {
      const int row = 16 * dt + l16;
      const u32x4 a = *reinterpret_cast<const u32x4*>(stage + L::VOFF + row * 64 + 16 * (g ^ ((row >> 2) & 3)));
      return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    };
    i32x8 vq[8];
    static_for<kVReadAhead>([&](auto dt) { vq[dt] = vread(dt); });
    static_for<8>([&](auto dt) {
      if constexpr (dt + kVReadAhead < 8) vq[dt + kVReadAhead] = vread(dt + kVReadAhead);
      const int vs = dt < 4 ? (int)ve.x : (int)ve.y;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        st.acc[qt][dt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vq[dt], p8[qt], st.acc[qt][dt], 0, 0,
                                                                          dt & 3, vs, 0, pexp[qt]);
        st.accl[qt][dt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vq[dt], a8[qt], st.accl[qt][dt], 0, 0,
                                                                           dt & 3, vs, 0, 127 + 10);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  } else {
    // P (probabilities) and A (448^2 phi(q).phi(k), the raw product of the codes) of key half s,
    // keys 32s + 16h + 4g + rr, as the bf16 B operands of the products below
    bf16x8 pop[QT][2], aop[QT][2];
    auto make_ops = [&](int qt, int s) {
      float pv[8], av[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pv[4 * h + rr] = __builtin_amdgcn_exp2f(fmaf(S[qt][2 * s + h][rr], cj, -st.m_run[qt]));
          av[4 * h + rr] = Ph[qt][2 * s + h][rr];
        }
      const uint32_t pw[4] = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                              pack_bf16x2(pv[6], pv[7])};
      const uint32_t aw[4] = {pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]), pack_bf16x2(av[4], av[5]),
                              pack_bf16x2(av[6], av[7])};
      pop[qt][s] = __builtin_bit_cast(bf16x8, pw);
      aop[qt][s] = __builtin_bit_cast(bf16x8, aw);
    };

#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      make_ops(qt, 0);
      make_ops(qt, 1);
    }

    // ---- O_s^T += V^T P^T and O_corr^T += V^T Ph^T, sharing each V^T operand read between the
    // query tiles and the two products; reads run one feature tile ahead of the products
    auto vread = [&](int dt, int s) {
      const int row = 16 * dt + l16;
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stage + L::VOFF + row * 128 +
                                                                       16 * ((4 * s + g) ^ (row & 7))));
    };
    // Steps k = 0..15 take key half s = k / 8 of feature tile dt = k % 8, so the two products
    // that accumulate into the same registers are eight steps apart.
    bf16x8 vq[16];
    const bf16x8 kOnes = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    static_for<kVReadAhead>([&](auto k) { vq[k] = vread(k % 8, k / 8); });
    static_for<16>([&](auto k) {
      if constexpr (k + kVReadAhead < 16) vq[k + kVReadAhead] = vread((k + kVReadAhead) % 8, (k + kVReadAhead) / 8);
      constexpr int dt = k % 8, sh = k / 8;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        st.acc[qt][dt] = mfma_bf16(vq[k], pop[qt][sh], st.acc[qt][dt]);
        st.accl[qt][dt] = mfma_bf16(vq[k], aop[qt][sh], st.accl[qt][dt]);
        // the row sum of P over key half sh: a ones A operand sums the 32 keys of the half,
        // those of all four lane groups, on the matrix cores instead of the VALU
        if constexpr (dt == 0) st.lsum[qt] = mfma_bf16(kOnes, pop[qt][sh], st.lsum[qt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  wait_dma();
  lds_barrier();
  ksc = ksc_next;
  if (r + 1 < topk) zacc += znext;   // Z_R(i) in LUT order
}

// One unrouted block for the direct form of the linear branch (a large share of the blocks
// routed): accl^T += V^T A^T with A = 448^2 phi(q).phi(K~_s) over its keys, the products of the
// routed part above, in bf16 (V^T tiles, or in the low-bit P.V mode the bf16 V rows through
// transposing reads).  Its tile is in LDS stage STG; the copy of the next unrouted block
// (jn >= 0) into the other stage starts first.
template <bool FP8, int QT, bool PV8, int STG>
__device__ __forceinline__ void lin_iteration(const FwdArgs& A, FwdState<QT>& st, uint8_t* smem0, uint8_t* smem1,
                                              int jn, int l16, int g, int tid, const QueryOps<QT>& qo,
                                              const TileSrc& src) {
  constexpr int NT = 256 / QT;
  using L = FwdLds<FP8, NT, PV8>;
  const uint8_t* stage = STG == 0 ? smem0 : smem1;
  uint8_t* next = STG == 0 ? smem1 : smem0;
  if (jn >= 0) dma_lin<FP8, NT, PV8>(A, src, jn, tid, next);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 Ph[QT][4];
  static_for<4>([&](auto mt) {
    const i32x8 pr = lds_fp8_row(stage + L::POFF, 16 * mt + l16, g);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) Ph[qt][mt] = mfma_fp8(pr, qo.phq8[qt], f32x4{0.f, 0.f, 0.f, 0.f});
  });
  // A of key half s (keys 32s + 16h + 4g + rr) as the bf16 B operand, as for P above
  bf16x8 aop[QT][2];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      const uint32_t aw[4] = {pack_bf16x2(Ph[qt][2 * sh][0], Ph[qt][2 * sh][1]),
                              pack_bf16x2(Ph[qt][2 * sh][2], Ph[qt][2 * sh][3]),
                              pack_bf16x2(Ph[qt][2 * sh + 1][0], Ph[qt][2 * sh + 1][1]),
                              pack_bf16x2(Ph[qt][2 * sh + 1][2], Ph[qt][2 * sh + 1][3])};
      aop[qt][sh] = __builtin_bit_cast(bf16x8, aw);
    }
  static_for<16>([&](auto k) {
    constexpr int dt = k % 8, sh = k / 8;
    bf16x8 v;
    if constexpr (PV8) {   // V rows: keys 32sh + 4g + rr and 32sh + 16 + 4g + rr of feature 16dt + l16
      const u32x2 a = lds_read_tr16_sw256(stage + L::VOFF, 32 * sh + 4 * g, 16 * dt, l16);
      const u32x2 b = lds_read_tr16_sw256(stage + L::VOFF, 32 * sh + 16 + 4 * g, 16 * dt, l16);
      v = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
    } else {
      const int row = 16 * dt + l16;
      v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stage + L::VOFF + row * 128 +
                                                                     16 * ((4 * sh + g) ^ (row & 7))));
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.accl[qt][dt] = mfma_bf16(v, aop[qt][sh], st.accl[qt][dt]);
  });
  wait_dma();
  lds_barrier();
}

// phi(q) = softmax over the 128 features of query row q (bf16 input): this lane's features
// 32s + 8g + e (s < 4, e < 8), f[s][e].
__device__ __forceinline__ void phi_q_values(const uint16_t* qrow, int g, float (&f)[4][8]) {
  u32x4 uu[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) uu[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4 u = uu[s];
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[s][2 * e] = bf16_lo(uw[e]);
      f[s][2 * e + 1] = bf16_hi(uw[e]);
    }
  }
  float mx = f[0][0];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, f[s][e]);
  mx = rows4_max(mx);
  float sm = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[s][e] = __builtin_amdgcn_exp2f((f[s][e] - mx) * kLog2e);
      sm += f[s][e];
    }
  const float rs = 1.f / rows4_sum(sm);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) f[s][e] *= rs;
}

// e4m3 codes of 448 phi(q) in (s, e) order: the B operand of Ph^T = phi(K) phi(q)^T, whose
// phi(K) codes are stored with the same feature permutation.
__device__ __forceinline__ i32x8 phi_q_codes(const float (&f)[4][8]) {
  uint32_t wds[8];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    wds[2 * s] = pack_fp8x4(clamp_fp8(f[s][0] * kPhiCodeScale), clamp_fp8(f[s][1] * kPhiCodeScale),
                            clamp_fp8(f[s][2] * kPhiCodeScale), clamp_fp8(f[s][3] * kPhiCodeScale));
    wds[2 * s + 1] = pack_fp8x4(clamp_fp8(f[s][4] * kPhiCodeScale), clamp_fp8(f[s][5] * kPhiCodeScale),
                                clamp_fp8(f[s][6] * kPhiCodeScale), clamp_fp8(f[s][7] * kPhiCodeScale));
  }
  return i32x8{(int)wds[0], (int)wds[1], (int)wds[2], (int)wds[3], (int)wds[4], (int)wds[5], (int)wds[6], (int)wds[7]};
}

// Epilogue of the fused forward for this wave's queries: O_s = acc / l, the linear branch
// O_l = (phi(q) H_tot - routed part) / (phi(q).(Z_tot - Z_R) + eps) (or the unrouted part itself
// in the direct form), O = alpha O_s + (1 - alpha) O_l, and the optional lse and backward stores.
// alphaS holds alpha of the head and zdS = Z_tot - Z_R(i), both per feature, in LDS.
// The bf16 LDS image of H^T has rows 0..63 at Hlo and rows 64..127 at Hhi (256-byte rows, chunk
// k of row r at chunk k ^ (r % 16)).
template <bool FP8, int QT>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& A, const FwdState<QT>& st, const QueryOps<QT>& qo,
                                             const uint8_t* Hlo, const uint8_t* Hhi, bool direct,
                                             const float* alphaS, const float* zdS, int bh, const int (&qrow)[QT],
                                             const bool (&qok)[QT], int l16, int g, int topk) {
  constexpr int D = 128;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l_tot = rows4_sum(st.l_run[qt]) + st.lsum[qt][0];   // one of the two is zero
    constexpr float kCodes2 = 1.f / (kPhiCodeScale * kPhiCodeScale);   // undo the code scales
    const float inv_l = 1.f / l_tot;
    // denominator over the unrouted blocks: phi(q).(Z_tot - Z_R), with the bf16 phi(q)
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 bw = __builtin_bit_cast(u32x4, qo.phb[qt][s]);
      const uint32_t ww[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 32 * s + 8 * g + 2 * e;
        den = fmaf(bf16_lo(ww[e]), zdS[a], den);
        den = fmaf(bf16_hi(ww[e]), zdS[a + 1], den);
      }
    }
    // with every block routed the linear branch is an empty sum, 0 (the complement form would
    // leave only rounding, amplified by 1/eps)
    const float inv_den = topk < A.T ? 1.f / (rows4_sum(den) + A.eps) : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      // numerator over the unrouted blocks: phi(q) H_tot minus the routed part, or (direct)
      // the unrouted part itself
      f32x4 ol = f32x4{0.f, 0.f, 0.f, 0.f};
      float lsign = -kCodes2;
      if (!direct) {
        const int hr = 16 * dt + l16;
        const uint8_t* hrow = (dt < 4 ? Hlo : Hhi) + (hr & 63) * 256;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(hrow + 16 * ((4 * s + g) ^ (hr & 15)));
          ol = mfma_bf16(__builtin_bit_cast(bf16x8, a), qo.phb[qt][s], ol);
        }
      } else {
        lsign = kCodes2;
      }
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(alphaS + 16 * dt + 4 * g);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
      float ov[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        ov[rr] = av[rr] * (st.acc[qt][dt][rr] * inv_l) +
                 (1.f - av[rr]) * (fmaf(lsign, st.accl[qt][dt][rr], ol[rr]) * inv_den);
      if (qok[qt]) {
        u32x2 sv;
        sv.x = pack_bf16x2(ov[0], ov[1]);
        sv.y = pack_bf16x2(ov[2], ov[3]);
        const size_t e0 = ((size_t)bh * A.N + qrow[qt]) * D + 16 * dt + 4 * g;
        *reinterpret_cast<u32x2*>(A.o + e0) = sv;
        if (A.os != nullptr) {   // the two branches, for the backward pass
          float sv4[4], lv4[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            sv4[rr] = st.acc[qt][dt][rr] * inv_l;
            lv4[rr] = fmaf(lsign, st.accl[qt][dt][rr], ol[rr]) * inv_den;
          }
          u32x2 s2, l2;
          s2.x = pack_bf16x2(sv4[0], sv4[1]);
          s2.y = pack_bf16x2(sv4[2], sv4[3]);
          l2.x = pack_bf16x2(lv4[0], lv4[1]);
          l2.y = pack_bf16x2(lv4[2], lv4[3]);
          *reinterpret_cast<u32x2*>(A.os + e0) = s2;
          *reinterpret_cast<u32x2*>(A.ol + e0) = l2;
        }
      }
    }
    if (A.os != nullptr && g == 0 && qok[qt]) A.inv_den[(size_t)bh * A.T * kBlock + qrow[qt]] = inv_den;
    if (A.lse != nullptr) {
      // native mode scored the raw keys: log-sum-exp over K~ = K - mu is lower by q.mu/sqrt(d)
      float shift = 0.f;
      if constexpr (!FP8) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 wv = __builtin_bit_cast(u32x4, qo.qb[qt][s]);
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
      if (g == 0 && qok[qt]) A.lse[(size_t)bh * A.N + qrow[qt]] = (st.m_run[qt] + log2f(l_tot)) * kLn2 - shift;
    }
  }
}

// One workgroup of 4/QT waves per (head, query block).  Wave w owns queries
// 16 QT w + 16 qt + (0..15), qt < QT, and computes S^T = K_j Q^T so that each lane holds one
// query (l % 16) of each tile and 16 of the block's keys (16mt + 4(l/16) + rr): the softmax
// state is per lane, and P feeds the P.V product as the B operand of O^T = V^T P^T without a
// transpose.  With QT = 2 every key-tile and V^T operand read from LDS serves two query tiles.
// The linear branch needs, for the unrouted blocks, phi(q) H_i and phi(q).Z_i with
// H_i = h_sum - sum over routed j of h_j.  The routed part phi(q) h_j = (phi(q) phi(K_j)^T) V_j
// is evaluated by re-association over the same routed keys and V^T tiles as the sparse
// branch, with phi(K~) and phi(q) as e4m3 codes (phi(q) scaled per query).
// Pipeline per routed block r: start copying the tile of block r+1 into the other LDS stage,
// compute on the LDS tile of block r, wait for the copy, barrier.
template <bool FP8, bool LUT_REG, int QT, bool PV8 = false>
__global__ __launch_bounds__(256 / QT, 2) void fwd_mfma_kernel(FwdArgs A) {
  constexpr int NT = 256 / QT;
  using L = FwdLds<FP8, NT, PV8>;
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[L::STAGE];   // stage of even LUT entries
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[L::STAGE];   // stage of odd LUT entries
  // alpha of the head and Z_tot - Z_R(i), per feature, for the epilogue.  When a stage is larger
  // than the H^T image (native Q.K^T: 40 KB stages), they go to the spare end of the epilogue's
  // stage after the loop, so that the workgroup takes exactly 80 KB of LDS and two fit a CU's
  // 160 KB; otherwise they have arrays of their own, written before the loop.
  constexpr bool kSpare = L::STAGE >= 128 * 256 + 2 * D * (int)sizeof(float);
  float* alphaS;
  float* zdS;
  if constexpr (!kSpare) {
    __shared__ float alphaArr[D], zdArr[D];
    alphaS = alphaArr;
    zdS = zdArr;
  }

  const int lid = xcd_remap(blockIdx.x, A.nblocks);
  // uniform indices in scalar registers, so per-block scalars load through the scalar cache
  const int bh = __builtin_amdgcn_readfirstlane(lid / A.T), i = __builtin_amdgcn_readfirstlane(lid % A.T);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int hidx = bh % A.H;
  int qrow[QT];   // this lane's query tokens
  int qsrc[QT];   // the token its operands load from: rows past N read row N-1 (never stored)
  bool qok[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    qrow[qt] = kBlock * i + 16 * QT * w + 16 * qt + l16;
    qok[qt] = qrow[qt] < A.N;
    qsrc[qt] = min(qrow[qt], A.N - 1);
  }
  const int32_t* lutG = A.lut + ((size_t)bh * A.T + i) * A.topk;
  const int topk = A.topk;

  // The LUT row into a register (lane x holds entry x) and, straight from memory, its first
  // entry, so that the first tile load starts at once; the query operands load meanwhile.
  const int lutv = (LUT_REG && lane < topk) ? lutG[lane] : 0;
  static_assert(NT >= D, "one thread per feature for alpha and Z_R");
  const float alv = tid < D ? A.alpha[(size_t)hidx * D + tid] : 0.f;
  const TileSrc src = tile_src(A, bh);
  const int j0 = __builtin_amdgcn_readfirstlane(lutG[0]);
  float ksc = FP8 ? A.k_scale[(size_t)bh * A.T + j0] : 1.f;
  // Z_R(i) = sum of z_j over the routed blocks, added in LUT order by threads tid < D (feature
  // tid) as the loop walks the row: each z_j loads with its block's tile copy
  float zacc = tid < D ? A.zblk[((size_t)bh * A.T + j0) * D + tid] : 0.f;
  const float zsum = tid < D ? A.z_sum[(size_t)bh * D + tid] : 0.f;
  dma_tile<FP8, NT, PV8>(A, src, j0, tid, smem0);

  QueryOps<QT> qo;
  float cq = kLog2e / sqrtf((float)D);
  if constexpr (FP8) cq *= A.q_scale[(size_t)bh * A.T + i];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if constexpr (FP8) {
      const uint8_t* src8 = A.q8 + (((size_t)bh * A.T * kBlock) + qrow[qt]) * D + 32 * g;
      const u32x4 a = *reinterpret_cast<const u32x4*>(src8);
      const u32x4 b = *reinterpret_cast<const u32x4*>(src8 + 16);
      qo.q8[qt] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(A.q + ((size_t)bh * A.N + qsrc[qt]) * D + 32 * s + 8 * g);
        qo.qb[qt][s] = __builtin_bit_cast(bf16x8, a);
      }
    }
    float f[4][8];
    phi_q_values(A.q + ((size_t)bh * A.N + qsrc[qt]) * D, g, f);
    qo.phq8[qt] = phi_q_codes(f);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t bw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) bw[e] = pack_bf16x2(f[s][2 * e], f[s][2 * e + 1]);
      qo.phb[qt][s] = __builtin_bit_cast(bf16x8, bw);
    }
  }
  if constexpr (!kSpare) {
    if (tid < D) alphaS[tid] = alv;   // read in the epilogue, after several barriers
  }
  // the last routed block is partial iff it is block T-1 and N is not a multiple of 64
  const bool last_partial = (lut_entry<LUT_REG>(lutv, lutG, topk - 1) == A.T - 1) && (A.N % kBlock != 0);

  FwdState<QT> st;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      st.acc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.accl[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    st.m_run[qt] = -INFINITY;
    st.l_run[qt] = 0.f;
    st.lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The first tile and every query-operand load complete here, before the loop: a wait for a
  // first use inside the loop could not tell them from the copies in flight there.
  wait_dma();
  lds_barrier();

  for (int r = 0; r < topk; r += 2) {
    fwd_iteration<FP8, LUT_REG, QT, 0, PV8>(A, st, smem0, smem1, lutv, ksc, lutG, r, topk, bh, l16, g, tid, qo, cq,
                                       last_partial && r == topk - 1, src, zacc);
    if (r + 1 < topk)
      fwd_iteration<FP8, LUT_REG, QT, 1, PV8>(A, st, smem0, smem1, lutv, ksc, lutG, r + 1, topk, bh, l16, g, tid, qo,
                                         cq, last_partial && r + 1 == topk - 1, src, zacc);
  }

  // With more than half of the blocks routed, the complement H_tot - (routed part) would be a
  // small difference of two large terms, amplifying the rounding of the routed part; the
  // unrouted part is then summed directly over the unrouted blocks instead (the same products
  // as the routed part above), and H_tot is not used.
  // (the low-bit P.V mode switches at a third: its routed-part products take e4m3 V, whose
  // rounding the complement amplifies sooner; its direct loop reads bf16 V rows)
  const bool direct = (PV8 ? 3 * topk > A.T : 2 * topk > A.T) && topk < A.T;
  if (direct) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) st.accl[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the unrouted blocks, ascending: a bitmap of the LUT row (in stage 1's key region, which
    // no copy below touches), then a ballot compaction into a list (stage 0's key region)
    static_assert(4096 * 2 <= L::KTILE, "the list of unrouted blocks fits in a key region");
    uint32_t* bits = reinterpret_cast<uint32_t*>(smem1);   // 128 words: T <= 4096
    int* wcnt = reinterpret_cast<int*>(smem1 + 512);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(smem0);
    if (tid < 128) bits[tid] = 0u;
    lds_barrier();
    for (int x = tid; x < topk; x += NT) {
      const int j = lutG[x];
      atomicOr(bits + (j >> 5), 1u << (j & 31));
    }
    lds_barrier();
    int nun = 0;
    for (int j0 = 0; j0 < A.T; j0 += NT) {
      const int j = j0 + tid;
      const bool un = j < A.T && ((bits[j >> 5] >> (j & 31)) & 1u) == 0u;
      const uint64_t b = __builtin_amdgcn_ballot_w64(un);
      if (lane == 0) wcnt[w] = __popcll(b);
      lds_barrier();
      int off = nun;
      for (int ww = 0; ww < w; ++ww) off += wcnt[ww];
      if (un) ulist[off + __popcll(b & ((1ull << lane) - 1ull))] = (uint16_t)j;
      for (int ww = 0; ww < NT / 64; ++ww) nun += wcnt[ww];
      lds_barrier();
    }
    // nun = T - topk >= 1; every copy below stays in the phi and V^T regions of the stages
    int u = __builtin_amdgcn_readfirstlane((int)ulist[0]);
    dma_lin<FP8, NT, PV8>(A, src, u, tid, smem1);
    wait_dma();
    lds_barrier();
    for (int n = 0; n < nun; n += 2) {
      const int u1 = n + 1 < nun ? __builtin_amdgcn_readfirstlane((int)ulist[n + 1]) : -1;
      lin_iteration<FP8, QT, PV8, 1>(A, st, smem0, smem1, u1, l16, g, tid, qo, src);
      if (n + 1 < nun) {
        const int u2 = n + 2 < nun ? __builtin_amdgcn_readfirstlane((int)ulist[n + 2]) : -1;
        lin_iteration<FP8, QT, PV8, 0>(A, st, smem0, smem1, u2, l16, g, tid, qo, src);
      }
    }
  }

  // ---------------- epilogue ----------------
  // H^T (bf16 image copied during the last iteration) is in the stage after the last tile's
  const uint8_t* Hs = (topk & 1) ? smem1 : smem0;
  // Z_tot - Z_R(i) per feature for the denominator; Z_R(i) also for the backward pass
  if (tid < D && A.os != nullptr) A.zrout[((size_t)bh * A.T + i) * D + tid] = zacc;
  if constexpr (kSpare) {
    // past the H^T image: that region last held a tile consumed before the last barrier, and
    // no copy is in flight
    alphaS = reinterpret_cast<float*>((Hs == smem1 ? smem1 : smem0) + 128 * 256);
    zdS = alphaS + D;
    if (tid < D) alphaS[tid] = alv;
  }
  if (tid < D) zdS[tid] = zsum - zacc;
  lds_barrier();
  fwd_epilogue<FP8, QT>(A, st, qo, Hs, Hs + 64 * 256, direct, alphaS, zdS, bh, qrow, qok, l16, g, topk);
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
    // with every block routed the linear branch is an empty sum, 0; the complement form would
    // leave only rounding, amplified by 1/eps
    const float os = acc[x] / l_tot, olin = topk < T ? num / den : 0.f;
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

hipError_t launch_fwd(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const BwdWorkspace* bw,
                      hipStream_t s) {
  if (g.bf16) {
    FwdArgs A;
    A.q = (const uint16_t*)t.q;
    A.k = (const uint16_t*)t.k;
    A.q8 = t.q8;
    A.k8 = t.k8;
    A.q_scale = t.q_scale;
    A.k_scale = t.k_scale;
    A.vt = ws.vt;
    A.vexp = g.pv8 ? ws.vexp : nullptr;
    A.v = (const uint16_t*)t.v;
    A.phik8 = ws.phik8;
    A.zblk = ws.zblk;
    A.zrout = ws.zrout;
    A.lut = t.lut;
    A.hbf = ws.hbf;
    A.z_sum = t.z_sum;
    A.alpha = t.alpha;
    A.k_mean = t.k_mean;
    A.o = (uint16_t*)t.o;
    A.lse = t.lse;
    // with the backward workspace (bf16, FP8 Q.K^T, d = 128) the forward keeps O_s, O_l, 1/den
    A.os = bw != nullptr ? bw->os : nullptr;
    A.ol = bw != nullptr ? bw->ol : nullptr;
    A.inv_den = bw != nullptr ? bw->inv_den : nullptr;
    A.N = g.N;
    A.T = g.T;
    A.H = g.H;
    A.topk = g.topk;
    A.nblocks = g.BH * g.T;
    A.eps = g.eps;
    const bool lut_reg = g.topk <= kLutReg;
    // One query tile per wave, four waves per workgroup (two workgroups per CU in FP8 mode).
    // Two tiles per wave (QT = 2: every LDS operand read serving both) measured 30% slower at
    // C2: half the waves per CU leave too little to overlap the copies and the barriers.
    if (g.pv8) {
      if (lut_reg) hipLaunchKernelGGL((fwd_mfma_kernel<true, true, 1, true>), dim3(A.nblocks), dim3(256), 0, s, A);
      else hipLaunchKernelGGL((fwd_mfma_kernel<true, false, 1, true>), dim3(A.nblocks), dim3(256), 0, s, A);
    } else if (g.fp8) {
      if (lut_reg) hipLaunchKernelGGL((fwd_mfma_kernel<true, true, 1>), dim3(A.nblocks), dim3(256), 0, s, A);
      else hipLaunchKernelGGL((fwd_mfma_kernel<true, false, 1>), dim3(A.nblocks), dim3(256), 0, s, A);
    } else {
      if (lut_reg) hipLaunchKernelGGL((fwd_mfma_kernel<false, true, 1>), dim3(A.nblocks), dim3(256), 0, s, A);
      else hipLaunchKernelGGL((fwd_mfma_kernel<false, false, 1>), dim3(A.nblocks), dim3(256), 0, s, A);
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

}  // namespace sla2
