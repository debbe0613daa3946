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
// The forward run before it stores O_s, O_l and 1/den per query (den = phi(q).Z_i + eps).
// With dO_s = alpha dO and dO_l = (1 - alpha) dO:
//   D_q = rowsum(dO_s * O_s), dnum = dO_l / den, dden = -(dO_l . O_l) / den,
//   dalpha = sum over tokens of dO * (O_s - O_l);
// sparse branch, P recomputed from lse over each routed pair:
//   dP = dO_s V^T, dS = P (dP - D_q), dQ' = dS K' / sqrt(d), dK' = dS^T Q' / sqrt(d),
//   dV = P^T dO_s;
// linear branch, O_l = phi(q) H_i / den with H_i, Z_i over the unrouted blocks:
//   dphi(q) = dnum H_i^T + dden Z_i, dH_i = phi(q)^T dnum, dZ_i = dden^T phi(q),
//   dh_j = sum of dH_i over the query blocks i that do not route to j (dz_j likewise),
//   dphi(k) = V dh_j^T + dz_j, dV += phi(k) dh_j, then the softmax backward of phi.
// Neither H_i nor dH_i is formed per pair.  Query side: H_i = H_tot - sum over the routed j of
// phi(K_j)^T V_j, so dnum H_i^T = dnum H_tot^T - sum_j (dnum V_j^T) phi(K_j), evaluated on the
// routed key tiles the sparse branch loads anyway.  Key side: with dH_i = (phi(q_i) / den)^T
// dO_i diag(1 - alpha), dh_j = (G_tot - sum over the query blocks i routing to j of
// (phi(q_i) / den)^T dO_i) diag(1 - alpha), one 128 x 128 product per routing pair, whose dO_i^T
// operand is the tile the sparse branch's dV product reads.
//
// Kernels: bwd_prep_kernel (per-token terms and the transposed operand tiles), the column sums
// G_tot and dZ_tot, bwd_query_kernel (dQ), bwd_key_kernel (dK~ with its column sums per key
// block, dV), then the key-smoothing mean, dK and dalpha.  Both main kernels copy each pair's tiles into LDS with direct-to-LDS loads
// while the previous pair is processed (two stages), and run the products on the bf16
// 16x16x32 matrix cores (the scores on the e4m3 16x16x128 ones, as the forward computed them).
#include <math.h>

#include "sla2_device.hpp"
#include "sla2_internal.hpp"
#include "sla2_lds.hpp"

namespace sla2 {

namespace {

constexpr int kD = 128;
constexpr int kNT = 256;
constexpr int kTTile = kD * kBlock * 2;   // bytes of one transposed bf16 tile: 128 rows x 64
constexpr int kQReadAhead = 1;            // feature tiles whose LDS operands are read ahead (query side)
constexpr int kKReadAhead = 2;            // the same on the key side

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
};

// rows x RB bytes from global rows of stride ld bytes
template <int RB>
__device__ __forceinline__ void stage(LTile<RB> dst, const uint8_t* src, size_t ld, int rows, int tid) {
  constexpr int NC = RB / 16;
  for (int x = tid; x < rows * NC; x += kNT) {
    const int r = x / NC, c = x % NC;
    *reinterpret_cast<u32x4*>(dst.chunk(r, c)) = *reinterpret_cast<const u32x4*>(src + (size_t)r * ld + 16 * c);
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

// 16-byte chunk (4s + g) of row `row` of a staged 128-byte-row tile (64 bf16 per row): the
// operand holding elements 32s + 8g .. 32s + 8g + 7
__device__ __forceinline__ bf16x8 op128(const uint8_t* base, int row, int s, int g) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + row * 128 + 16 * ((4 * s + g) ^ (row & 7))));
}
// the same for a staged 256-byte-row tile (128 bf16 per row)
__device__ __forceinline__ bf16x8 op256(const uint8_t* base, int row, int s, int g) {
  return __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const u32x4*>(base + row * 256 + 16 * ((4 * s + g) ^ (row & 15))));
}

// Column of token x of a 64-block in the transposed tiles (the forward's V^T order): within
// each 32-half, tokens 4gg + e sit at 8gg + e and tokens 16 + 4gg + e at 8gg + 4 + e.  A 16 x 16
// product's output (token rows 4g + r of two adjacent 16-row tiles) then packs, without a
// transpose, into the B operand whose k-index is this column.
__device__ __forceinline__ int vt_pos(int x) {
  const int s = x >> 5, rem = x & 31, h = rem >> 4, gg = (rem & 15) >> 2, e = rem & 3;
  return 32 * s + 8 * gg + 4 * h + e;
}

// The operand with rows c = c0 + l%16 of dO^T and the k-run of query half s in the packed order
// (queries 32s + 4g + 0..3, then 32s + 16 + 4g + 0..3), read from the staged dO rows (256-byte
// rows, swizzled) with transposing reads: the A operand of dV^T = dO^T P and, identically laid
// out, the B operand of the dh_j correction (phi(q)/den)^T dO.
__device__ __forceinline__ bf16x8 dot_op(const uint8_t* dorows, int s, int c0, int l16, int g) {
  const u32x2 a = lds_read_tr16_sw256(dorows, 32 * s + 4 * g, c0, l16);
  const u32x2 b = lds_read_tr16_sw256(dorows, 32 * s + 16 + 4 * g, c0, l16);
  return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// 8 bf16 values as the B operand: v[4h + rr] from output tile 2s + h, row 4g + rr
__device__ __forceinline__ bf16x8 pack8(const float (&v)[8]) {
  const uint32_t w[4] = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7])};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

struct BwdArgs {
  const uint16_t* q;       // bf16 [BH, N, D]
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* alpha;      // [H, D]
  const float* k_mean;     // [BH, D]
  const uint8_t* q8;       // [BH, 64T, D] (pad rows code 0)
  const uint8_t* k8;
  const float* q_scale;    // [BH, T]
  const float* k_scale;
  const float* lse;        // [BH, N]
  const int32_t* lut;      // [BH, T, topk]
  const uint8_t* mask;     // [BH, T, T]
  const float* h_sum;      // [BH, D, D], h_sum[c][a]
  const float* z_sum;      // [BH, D]
  const float* zrout;      // forward workspace: [BH, T, D] Z_R(i)
  // stored by the forward
  const uint16_t* os;      // [BH, N, D] O_s (bf16)
  const uint16_t* ol;      // [BH, N, D] O_l (bf16)
  const float* inv_den;    // [BH, 64T] 1 / den (0 when every block is routed)
  // backward workspace
  uint16_t* q8t;           // [BH, T, D, 64] e4m3 values of Q8 (unscaled) transposed, vt_pos
  uint16_t* phqdt;         // [BH, T, D, 64] (phi(q) / den)^T, vt_pos
  uint16_t* k8t;           // [BH, T, D, 64] e4m3 values of K8 transposed, vt_pos
  uint16_t* phkt;          // [BH, T, D, 64] phi(K~)^T, vt_pos (pad tokens 0)
  uint16_t* htimg;         // [BH, D, D] bf16 H_tot rows a (h_sum transposed), LDS image
  float* qrec;             // [BH, T, 256] per query block: -lse log2(e) [64], D_q[64], zeros
  float* dden;             // [BH, 64T]
  int32_t* inv;            // [BH, T, T] query blocks routing to key block j, ascending
  int32_t* inv_cnt;        // [BH, T]
  float* dZ;               // [BH, T, D]
  float* gpart;            // [BH, PG, D, D] partials of G_tot
  float* zpart;            // [BH, PG, D]
  float* g_tot;            // [BH, D, D] G_tot[a][c] = sum over tokens of phi(q)[a] / den * dO[c]
  float* dZ_tot;           // [BH, D]
  float* dalpha_part;      // [BH, T, D]
  float* dkt;              // [BH, 64T, D] dK~ (fp32)
  float* colsum_part;      // [BH, T, D] column sums of dK~ over each key block
  float* dk_mean;          // [BH, D]
  // outputs
  uint16_t* dq;            // bf16 [BH, N, D]
  uint16_t* dk;
  uint16_t* dv;
  float* dalpha;           // [H, D]
  int B, H, N, T, topk, pg, nblocks;
  int smooth_k;
};

// ---------------------------------------------------------------------------------------
// Per (head, 64-token block b), four threads per token (32 features each).  As a query block:
// D_q, dden, the dalpha and dZ_i column sums, and the transposed tiles (phi(q)/den)^T and
// Q8^T.  As a key block: K8^T and phi(K~)^T.  Block 0 also writes the bf16
// image of H_tot with rows a.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs A) {
  __shared__ uint16_t tr[kD * kBlock];        // [feature][vt_pos(token)]
  __shared__ float red[kBlock][kD + 4];       // per-token values of one column sum
  const int b = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, hidx = bh % A.H;
  const int x = tid >> 2, c0 = 32 * (tid & 3);
  const int tok = kBlock * b + x;
  const bool ok = tok < A.N;
  const int px = vt_pos(x);
  const size_t trow = (size_t)bh * A.N + (ok ? tok : 0);       // row of the [BH, N, D] tensors
  const size_t prow = (size_t)bh * A.T * kBlock + tok;          // row of the padded [BH, 64T, D] ones
  const size_t tile = ((size_t)bh * A.T + b) * kD * kBlock;     // block b's transposed tiles
  auto flush = [&](uint16_t* dst) {
    __syncthreads();
    for (int e = tid; e < kD * kBlock / 8; e += kNT)
      reinterpret_cast<u32x4*>(dst + tile)[e] = reinterpret_cast<const u32x4*>(tr)[e];
    __syncthreads();
  };
  auto colsum = [&](float* dst) {   // dst[c] = sum over the 64 tokens of red[.][c]
    __syncthreads();
    if (tid < kD) {
      float s = 0.f;
      for (int t = 0; t < kBlock; ++t) s += red[t][tid];
      dst[tid] = s;
    }
    __syncthreads();
  };
  auto load32 = [&](const uint16_t* src, float (&f)[32]) {   // features c0.. of row trow (0 past N)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 wv = ok ? *reinterpret_cast<const u32x4*>(src + trow * kD + c0 + 8 * u) : u32x4{0, 0, 0, 0};
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[8 * u + 2 * e] = bf16_lo(ww[e]);
        f[8 * u + 2 * e + 1] = bf16_hi(ww[e]);
      }
    }
  };
  // softmax over the 128 features of a row held by the four threads of a token
  auto softmax32 = [&](float (&f)[32]) {
    float mx = f[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, f[e]);
    mx = fmaxf(mx, dpp<0xB1>(mx));
    mx = fmaxf(mx, dpp<0x4E>(mx));
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      f[e] = __expf(f[e] - mx);
      s += f[e];
    }
    s += dpp<0xB1>(s);
    s += dpp<0x4E>(s);
    const float is = 1.f / s;
#pragma unroll
    for (int e = 0; e < 32; ++e) f[e] *= is;
  };

  float dO[32], al[32];
  load32(A.dout, dO);
#pragma unroll
  for (int e = 0; e < 32; ++e) al[e] = A.alpha[(size_t)hidx * kD + c0 + e];
  const float inv_den = ok ? A.inv_den[prow] : 0.f;   // pad rows are never written by the forward
  float dq = 0.f, dd = 0.f;
  {
    float os[32], ol[32];
    load32(A.os, os);
    load32(A.ol, ol);
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      dq = fmaf(al[e] * dO[e], os[e], dq);
      dd = fmaf((1.f - al[e]) * dO[e], ol[e], dd);
      red[x][c0 + e] = dO[e] * (os[e] - ol[e]);
    }
  }
  dq += dpp<0xB1>(dq);
  dq += dpp<0x4E>(dq);
  dd += dpp<0xB1>(dd);
  dd += dpp<0x4E>(dd);
  const float dden = -dd * inv_den;
  colsum(A.dalpha_part + ((size_t)bh * A.T + b) * kD);

  // phi(q) / den and the column sums dZ_i = sum_q dden phi(q)
  {
    float f[32];
    load32(A.q, f);
    softmax32(f);
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float ph = ok ? f[e] : 0.f;
      tr[(c0 + e) * kBlock + px] = f32_to_bf16(ph * inv_den);
      red[x][c0 + e] = dden * ph;
    }
  }
  flush(A.phqdt);
  colsum(A.dZ + ((size_t)bh * A.T + b) * kD);

  // e4m3 values of the Q and K~ codes (exact in bf16), transposed
  for (int which = 0; which < 2; ++which) {
    const uint32_t* codes = reinterpret_cast<const uint32_t*>((which == 0 ? A.q8 : A.k8) + prow * kD + c0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {   // four codes per word
      const f32x4 v = e4m3_decode4(codes[q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) tr[(c0 + 4 * q + e) * kBlock + px] = f32_to_bf16(v[e]);
    }
    flush(which == 0 ? A.q8t : A.k8t);
  }

  // phi(K~)^T (pad tokens 0)
  {
    float f[32];
    load32(A.k, f);
#pragma unroll
    for (int e = 0; e < 32; ++e) f[e] -= A.k_mean[(size_t)bh * kD + c0 + e];
    softmax32(f);
#pragma unroll
    for (int e = 0; e < 32; ++e) tr[(c0 + e) * kBlock + px] = f32_to_bf16(ok ? f[e] : 0.f);
  }
  flush(A.phkt);

  // per-query record of the key side, and dden
  float* rec = A.qrec + ((size_t)bh * A.T + b) * kRec;
  if ((tid & 3) == 0) {
    rec[x] = ok ? -A.lse[trow] * kLog2e : -INFINITY;   // -lse log2(e); pad queries: P = 2^-inf = 0
    rec[kBlock + x] = dq;   // 0 past N (dO is 0 there)
    A.dden[prow] = dden;
  }
  if (tid >= 2 * kBlock) rec[tid] = 0.f;

  // H_tot with rows a: image[a] chunk k at k ^ (a % 16)
  if (b == 0) {
    const float* hs = A.h_sum + (size_t)bh * kD * kD;
    uint16_t* img = A.htimg + (size_t)bh * kD * kD;
    for (int e = tid; e < kD * kD; e += kNT) {
      const int c = e / kD, a = e % kD;
      img[a * kD + 8 * ((c >> 3) ^ (a & 15)) + (c & 7)] = f32_to_bf16(hs[e]);
    }
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

// Partials of G_tot[a][c] = sum over tokens of (phi(q)/den)[a] dO[c] over kGChunk query blocks,
// and of dZ_tot.  Wave w: rows a = 32w..32w+31.
__global__ __launch_bounds__(256) void bwd_gtot_kernel(BwdArgs A) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[2 * kTTile];
  const LTile<128> PT{sm};
  const LTile<256> DO{sm + kTTile};   // dO rows of the block (rows past N: row N-1, times phi 0)
  const int p = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  f32x4 acc[2][8];
#pragma unroll
  for (int at = 0; at < 2; ++at)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[at][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int b0 = p * kGChunk, b1 = min(A.T, b0 + kGChunk);
  for (int b = b0; b < b1; ++b) {
    __syncthreads();
    const size_t tile = ((size_t)bh * A.T + b) * kD * kBlock;
    stage<128>(PT, reinterpret_cast<const uint8_t*>(A.phqdt + tile), 128, kD, tid);
    for (int x = tid; x < kBlock * 16; x += kNT) {
      const int r = x >> 4, c = x & 15, tok = min(kBlock * b + r, A.N - 1);
      *reinterpret_cast<u32x4*>(DO.chunk(r, c)) =
          *reinterpret_cast<const u32x4*>(A.dout + ((size_t)bh * A.N + tok) * kD + 8 * c);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 fa0 = PT.op(32 * w + l16, 32 * s + 8 * g), fa1 = PT.op(32 * w + 16 + l16, 32 * s + 8 * g);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const bf16x8 fo = dot_op(DO.p, s, 16 * ct, l16, g);
        acc[0][ct] = mfma_bf16(fa0, fo, acc[0][ct]);
        acc[1][ct] = mfma_bf16(fa1, fo, acc[1][ct]);
      }
    }
  }
  float* out = A.gpart + ((size_t)bh * A.pg + p) * kD * kD;
#pragma unroll
  for (int at = 0; at < 2; ++at)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(32 * w + 16 * at + 4 * g + r) * kD + 16 * ct + l16] = acc[at][ct][r];
  if (tid < kD) {
    float z = 0.f;
    for (int b = b0; b < b1; ++b) z += A.dZ[((size_t)bh * A.T + b) * kD + tid];
    A.zpart[((size_t)bh * A.pg + p) * kD + tid] = z;
  }
}

// Entry x of a list held in a register (lane x holds entry x) when it has at most 64 entries,
// else read from memory.
__device__ __forceinline__ int list_entry(bool in_reg, int regv, const int32_t* mem, int x) {
  return in_reg ? __builtin_amdgcn_readlane(regv, x) : __builtin_amdgcn_readfirstlane(mem[x]);
}

// ---------------------------------------------------------------------------------------
// Query side.  One workgroup of eight waves per (head, query block i), in two roles over the
// same staged key tiles; wave w owns queries 16(w % 4)..+15, one per lane column (l % 16).
// Products are computed transposed so that each lane holds one query and the pair's keys
// 16mt + 4g + r, and their results pack straight into B operands (keys at vt_pos, the order of
// the transposed tiles):
//   sparse waves (w < 4): S^T = K8 Q8^T, dP^T = V dO_s^T, dS^T, then dQ'^T += K8^T dS^T;
//   linear waves (w >= 4): U^T = V dnum^T, then C^T += phi(K)^T U^T.
// ---------------------------------------------------------------------------------------
constexpr int kNT2 = 512;   // threads of the two-role kernels

namespace qlds {
constexpr int K8 = 0;                 // e4m3 rows of key block j       64 x 128 B
constexpr int V = K8 + 8192;          // V rows                          64 x 256 B
constexpr int KT = V + 16384;         // K8 values^T                     128 x 128 B
constexpr int PT = KT + 16384;        // phi(K~)^T                       128 x 128 B
constexpr int STAGE = PT + 16384;
static_assert(STAGE >= 2 * kD * kD, "the H_tot image fits in a stage");
static_assert(STAGE >= 4 * kBlock * kD, "the linear part of dQ (fp32) fits in a stage");
}  // namespace qlds

struct QSrc {
  __amdgpu_buffer_rsrc_t k8, v, kt, pt, him;
};

// key block j's tiles into a stage: 7 16-byte copies per thread
__device__ __forceinline__ void q_dma(const QSrc& s, int j, int N, int tid, uint8_t* st) {
  const int wofs = 1024 * __builtin_amdgcn_readfirstlane(tid >> 6);
  {
    const int row = tid >> 3, pc = tid & 7;
    lds_dma(s.k8, st + qlds::K8 + wofs, row * 128 + 16 * fp8_chunk(row, pc), j * 8192);
  }
  static_for<2>([&](auto P) {
    const int qd = tid + kNT2 * P, row = qd >> 4, pc = qd & 15;
    const int tok = min(kBlock * j + row, N - 1);   // rows past N: a finite row, masked later
    lds_dma(s.v, st + qlds::V + 8192 * P + wofs, tok * 256 + 16 * (pc ^ (row & 15)), 0);
  });
  static_for<2>([&](auto P) {
    const int qd = tid + kNT2 * P, row = qd >> 3, pc = qd & 7;
    const int vo = row * 128 + 16 * (pc ^ (row & 7));
    lds_dma(s.kt, st + qlds::KT + 8192 * P + wofs, vo, j * kTTile);
    lds_dma(s.pt, st + qlds::PT + 8192 * P + wofs, vo, j * kTTile);
  });
}

// the 32 KB image of H_tot (rows a) into a stage
__device__ __forceinline__ void q_dma_himage(const QSrc& s, int tid, uint8_t* st) {
  const int wofs = 1024 * __builtin_amdgcn_readfirstlane(tid >> 6);
  static_for<4>([&](auto P) { lds_dma(s.him, st + 8192 * P + wofs, 16 * (tid + kNT2 * P), 0); });
}

struct QOps {
  i32x8 q8;       // sparse waves: e4m3 codes of features 32g..32g+31
  bf16x8 b[4];    // features 32s + 8g + e: alpha dO (sparse waves) or dnum (linear waves)
  float lse_l;    // sparse waves: lse * log2(e)
  float dq_l;     // sparse waves: D_q
};

// One routed pair: key block j = LUT entry r in stage STG, K scale ksc.  The next block's tiles
// (after the last, the H_tot image) are copied into the other stage meanwhile.  acc: dQ'^T
// (sparse waves, scales folded in) or C^T (linear waves), features 16ct + 4g + r.
template <int STG>
__device__ __forceinline__ void q_iteration(const BwdArgs& A, f32x4 (&acc)[8], uint8_t* smem0, uint8_t* smem1,
                                            const QSrc& src, bool lut_reg, int lutv, const int32_t* lutG,
                                            int r, int topk, int bh, float sq, float& ksc, const QOps& qo,
                                            bool sparse, int nvalid, int l16, int g, int tid) {
  const uint8_t* stg = STG == 0 ? smem0 : smem1;
  uint8_t* next = STG == 0 ? smem1 : smem0;
  float ksc_next = 1.f;
  if (r + 1 < topk) {
    const int jn = list_entry(lut_reg, lutv, lutG, r + 1);
    ksc_next = A.k_scale[(size_t)bh * A.T + jn];
    q_dma(src, jn, A.N, tid, next);
  } else {
    q_dma_himage(src, tid, next);
  }
  __builtin_amdgcn_sched_barrier(0);

  if (sparse) {
    const float inv_sqrt_d = 0.08838834764831845f;   // 1 / sqrt(128)
    // P^T and dS^T (times k_scale / sqrt(d), the factor of dQ' = dS K' / sqrt(d)) of key half s
    // (tiles 2s, 2s+1) as B operands
    const float cj = kLog2e * inv_sqrt_d * sq * ksc, fs = ksc * inv_sqrt_d;
    // only fs P is needed here, so fs (> 0) enters the exponent: 2^(x - lse + log2 fs)
    const float nl = __builtin_amdgcn_logf(fs) - qo.lse_l;
    f32x4 S[4], dP[4];
    bf16x8 dso_[2];
    auto half_ops = [&](int s) {
      float dv8[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int mt = 2 * s + h;
          const float pf = __builtin_amdgcn_exp2f(fmaf(S[mt][rr], cj, nl));   // fs P
          dv8[4 * h + rr] = pf * (dP[mt][rr] - qo.dq_l);
        }
      if (nvalid < kBlock) {   // the partial last block only: keys past N
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (16 * (2 * s + h) + 4 * g + rr >= nvalid) dv8[4 * h + rr] = 0.f;
      }
      dso_[s] = pack8(dv8);
    };
    // operand reads run one key tile ahead of the products that use them
    i32x8 kr[4];
    bf16x8 va[4][4];
    auto read_keys = [&](auto mt) {
      kr[mt] = lds_fp8_row(stg + qlds::K8, 16 * mt + l16, g);
#pragma unroll
      for (int s = 0; s < 4; ++s) va[mt][s] = op256(stg + qlds::V, 16 * mt + l16, s, g);
    };
    read_keys(std::integral_constant<int, 0>{});
    static_for<4>([&](auto mt) {
      if constexpr (mt + 1 < 4) read_keys(std::integral_constant<int, mt + 1>{});
      S[mt] = mfma_fp8(kr[mt], qo.q8, f32x4{0.f, 0.f, 0.f, 0.f});
      dP[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) dP[mt] = mfma_bf16(va[mt][s], qo.b[s], dP[mt]);
      if constexpr (mt == 2) half_ops(0);   // while tile 2's products run
      __builtin_amdgcn_sched_barrier(0);
    });
    half_ops(1);
    bf16x8 ka[8][2];
    auto read_feat = [&](auto ct) {
#pragma unroll
      for (int s = 0; s < 2; ++s) ka[ct][s] = op128(stg + qlds::KT, 16 * ct + l16, s, g);
    };
    static_for<kQReadAhead>([&](auto ct) { read_feat(ct); });
    static_for<8>([&](auto ct) {
      if constexpr (ct + kQReadAhead < 8) read_feat(std::integral_constant<int, ct + kQReadAhead>{});
#pragma unroll
      for (int s = 0; s < 2; ++s) acc[ct] = mfma_bf16(ka[ct][s], dso_[s], acc[ct]);
      __builtin_amdgcn_sched_barrier(0);
    });
  } else {
    // U^T = V dnum^T, packed as the B operand of C^T += phi(K)^T U^T
    f32x4 U[4];
    bf16x8 va[4][4];
    auto read_keys = [&](auto mt) {
#pragma unroll
      for (int s = 0; s < 4; ++s) va[mt][s] = op256(stg + qlds::V, 16 * mt + l16, s, g);
    };
    read_keys(std::integral_constant<int, 0>{});
    static_for<4>([&](auto mt) {
      if constexpr (mt + 1 < 4) read_keys(std::integral_constant<int, mt + 1>{});
      U[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) U[mt] = mfma_bf16(va[mt][s], qo.b[s], U[mt]);
      __builtin_amdgcn_sched_barrier(0);
    });
    bf16x8 uo[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float uv8[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) uv8[4 * h + rr] = U[2 * s + h][rr];
      uo[s] = pack8(uv8);
    }
    bf16x8 pa[8][2];
    auto read_feat = [&](auto ct) {
#pragma unroll
      for (int s = 0; s < 2; ++s) pa[ct][s] = op128(stg + qlds::PT, 16 * ct + l16, s, g);
    };
    static_for<kQReadAhead>([&](auto ct) { read_feat(ct); });
    static_for<8>([&](auto ct) {
      if constexpr (ct + kQReadAhead < 8) read_feat(std::integral_constant<int, ct + kQReadAhead>{});
#pragma unroll
      for (int s = 0; s < 2; ++s) acc[ct] = mfma_bf16(pa[ct][s], uo[s], acc[ct]);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  wait_dma();
  lds_barrier();
  ksc = ksc_next;
}

__global__ __launch_bounds__(512, 1) void bwd_query_kernel(BwdArgs A) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[qlds::STAGE];   // stage of even LUT entries
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[qlds::STAGE];   // stage of odd LUT entries
  __shared__ float zS[kD];                                                // Z_i
  const int lid = xcd_remap(blockIdx.x, A.nblocks);
  const int bh = __builtin_amdgcn_readfirstlane(lid / A.T), i = __builtin_amdgcn_readfirstlane(lid % A.T);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4, wq = w & 3;
  const bool sparse = w < 4;
  const int hidx = bh % A.H, T = A.T, N = A.N, topk = A.topk;
  const int qq = kBlock * i + 16 * wq + l16;   // this lane's query
  const bool qok = qq < N;
  const int32_t* lutG = A.lut + ((size_t)bh * T + i) * topk;
  const bool lut_reg = topk <= 64;
  const int lutv = (lut_reg && lane < topk) ? lutG[lane] : 0;

  QSrc src;
  src.k8 = rsrc(A.k8 + (size_t)bh * T * kBlock * kD, (size_t)T * kBlock * kD);
  src.v = rsrc(A.v + (size_t)bh * N * kD, (size_t)N * kD * 2);
  src.kt = rsrc(A.k8t + (size_t)bh * T * kD * kBlock, (size_t)T * kTTile);
  src.pt = rsrc(A.phkt + (size_t)bh * T * kD * kBlock, (size_t)T * kTTile);
  src.him = rsrc(A.htimg + (size_t)bh * kD * kD, (size_t)kD * kD * 2);
  const int j0 = __builtin_amdgcn_readfirstlane(lutG[0]);
  float ksc = A.k_scale[(size_t)bh * T + j0];
  q_dma(src, j0, N, tid, smem0);

  QOps qo;
  qo.q8 = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  qo.lse_l = 0.f;
  qo.dq_l = 0.f;
  const float invd = qok ? A.inv_den[(size_t)bh * T * kBlock + qq] : 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = 32 * s + 8 * g;
    const u32x4 raw = qok ? *reinterpret_cast<const u32x4*>(A.dout + ((size_t)bh * N + qq) * kD + c) : u32x4{0, 0, 0, 0};
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(A.alpha + (size_t)hidx * kD + c);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(A.alpha + (size_t)hidx * kD + c + 4);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    float b8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = (e & 1) ? bf16_hi(rw[e >> 1]) : bf16_lo(rw[e >> 1]);
      b8[e] = sparse ? av[e] * d : (1.f - av[e]) * d * invd;   // alpha dO or dnum
    }
    qo.b[s] = pack8(b8);
  }
  if (sparse) {
    const uint8_t* s8 = A.q8 + ((size_t)bh * T * kBlock + qq) * kD + 32 * g;   // pad rows: code 0
    const u32x4 a = *reinterpret_cast<const u32x4*>(s8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(s8 + 16);
    qo.q8 = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    qo.lse_l = qok ? A.lse[(size_t)bh * N + qq] * kLog2e : 0.f;
    qo.dq_l = A.qrec[((size_t)bh * T + i) * kRec + kBlock + 16 * wq + l16];
  }
  const float dden_l = A.dden[(size_t)bh * T * kBlock + qq];
  const float sq = A.q_scale[(size_t)bh * T + i];
  if (tid < kD) zS[tid] = A.z_sum[(size_t)bh * kD + tid] - A.zrout[((size_t)bh * T + i) * kD + tid];
  // only block T-1 can be partial, and only as the last LUT entry (rows are ascending)
  const int nlast = N - kBlock * (T - 1);
  const bool last_partial = list_entry(lut_reg, lutv, lutG, topk - 1) == T - 1 && nlast < kBlock;

  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_dma();
  lds_barrier();

  // pairs of LUT entries, then the odd last one: the loop body has no branch on the count, so
  // its registers need no reshuffling at a join
  int r = 0;
  for (; r + 1 < topk; r += 2) {
    q_iteration<0>(A, acc, smem0, smem1, src, lut_reg, lutv, lutG, r, topk, bh, sq, ksc, qo, sparse, kBlock, l16, g,
                   tid);
    q_iteration<1>(A, acc, smem0, smem1, src, lut_reg, lutv, lutG, r + 1, topk, bh, sq, ksc, qo, sparse,
                   (last_partial && r + 1 == topk - 1) ? nlast : kBlock, l16, g, tid);
  }
  if (r < topk)
    q_iteration<0>(A, acc, smem0, smem1, src, lut_reg, lutv, lutG, r, topk, bh, sq, ksc, qo, sparse,
                   last_partial ? nlast : kBlock, l16, g, tid);

  // ---------------- epilogue: the H_tot image is in the stage after the last tile's; the
  // other stage carries the linear part of dQ from the linear waves to the sparse waves
  const uint8_t* Hs = (topk & 1) ? smem1 : smem0;
  float* X = reinterpret_cast<float*>((topk & 1) ? smem0 : smem1);
  if (!sparse) {
    // phi(q) at features a = 16at + 4g + r (the layout of the accumulators)
    float ph[8][4];
    {
      const uint16_t* qr = A.q + ((size_t)bh * N + min(qq, N - 1)) * kD + 4 * g;
      float mx = -INFINITY;
#pragma unroll
      for (int at = 0; at < 8; ++at) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(qr + 16 * at);
        ph[at][0] = bf16_lo(wv.x);
        ph[at][1] = bf16_hi(wv.x);
        ph[at][2] = bf16_lo(wv.y);
        ph[at][3] = bf16_hi(wv.y);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, ph[at][rr]);
      }
      mx = rows4_max(mx);
      float sm = 0.f;
#pragma unroll
      for (int at = 0; at < 8; ++at)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          ph[at][rr] = __expf(ph[at][rr] - mx);
          sm += ph[at][rr];
        }
      const float is = 1.f / rows4_sum(sm);
#pragma unroll
      for (int at = 0; at < 8; ++at)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ph[at][rr] *= is;
    }
    // dphi(q)^T = H_tot dnum^T - C^T + Z_i dden, then the softmax backward
    float dphi[8][4], dotp = 0.f;
#pragma unroll
    for (int at = 0; at < 8; ++at) {
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) t = mfma_bf16(op256(Hs, 16 * at + l16, s, g), qo.b[s], t);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        dphi[at][rr] = t[rr] - acc[at][rr] + zS[16 * at + 4 * g + rr] * dden_l;
        dotp = fmaf(ph[at][rr], dphi[at][rr], dotp);
      }
    }
    dotp = rows4_sum(dotp);
#pragma unroll
    for (int at = 0; at < 8; ++at)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) X[((wq * 8 + at) * 4 + rr) * 64 + lane] = ph[at][rr] * (dphi[at][rr] - dotp);
  }
  __syncthreads();
  if (sparse && qok) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      float o[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) o[rr] = acc[ct][rr] + X[((wq * 8 + ct) * 4 + rr) * 64 + lane];
      u32x2 sv;
      sv.x = pack_bf16x2(o[0], o[1]);
      sv.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<u32x2*>(A.dq + ((size_t)bh * N + qq) * kD + 16 * ct + 4 * g) = sv;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Key side.  One workgroup of eight waves per (head, key block j), in two roles over the same
// staged query tiles.  Per routing query block i:
//   sparse waves (w < 4, keys 16w..16w+15, one per lane column): S = Q8 K8^T, dP = dO (alpha
//     V)^T, then dV^T += dO^T P and dK'^T += Q8^T dS (queries in the packed vt_pos order);
//   correction waves (w >= 4): C[a][c] += (phi(q)/den)^T dO over rows a = 32(w - 4)..+31.
// dO is staged once, as rows copied from the input; the dO^T operands come from the same tile
// through transposing reads.
// ---------------------------------------------------------------------------------------
namespace klds {
constexpr int Q8 = 0;                 // e4m3 rows of query block i      64 x 128 B
constexpr int DO = Q8 + 8192;         // dO rows (the input)              64 x 256 B
constexpr int QT = DO + 16384;        // Q8 values^T                      128 x 128 B
constexpr int PT = QT + 16384;        // (phi(q)/den)^T                   128 x 128 B
constexpr int REC = PT + 16384;       // lse[64], D_q[64], zeros          1 KB
constexpr int STAGE = REC + 1024;
static_assert(STAGE >= 2 * kD * kD, "a dh_j image fits in a stage");
}  // namespace klds

struct KSrc {
  __amdgpu_buffer_rsrc_t q8, dout, qt, pt, rec;
};

// query block i's tiles into a stage: 7 16-byte copies per thread (8 in wave 0)
__device__ __forceinline__ void k_dma(const KSrc& s, int i, int N, int tid, uint8_t* st) {
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wofs = 1024 * w;
  {
    const int row = tid >> 3, pc = tid & 7;
    lds_dma(s.q8, st + klds::Q8 + wofs, row * 128 + 16 * fp8_chunk(row, pc), i * 8192);
  }
  static_for<2>([&](auto P) {
    const int qd = tid + kNT2 * P, row = qd >> 4, pc = qd & 15;
    const int tok = min(kBlock * i + row, N - 1);   // rows past N: a finite row, masked by P
    lds_dma(s.dout, st + klds::DO + 8192 * P + wofs, tok * 256 + 16 * (pc ^ (row & 15)), 0);
  });
  static_for<2>([&](auto P) {
    const int qd = tid + kNT2 * P, row = qd >> 3, pc = qd & 7;
    const int vo = row * 128 + 16 * (pc ^ (row & 7));
    lds_dma(s.qt, st + klds::QT + 8192 * P + wofs, vo, i * kTTile);
    lds_dma(s.pt, st + klds::PT + 8192 * P + wofs, vo, i * kTTile);
  });
  if (w == 0) lds_dma(s.rec, st + klds::REC, 16 * (tid & 63), i * (kRec * 4));
}

struct KOps {
  i32x8 k8;          // sparse waves: e4m3 codes of features 32g..32g+31 of this lane's key
  bf16x8 v[4];       // sparse waves: alpha V of this lane's key, features 32s + 8g + e
};

// acc: sparse waves: [0..7] dV^T, [8..15] dK'^T (features 16ct + 4g + r of this lane's key);
// correction waves: C[a][c] at [8at + ct], a = 32(w - 4) + 16at + 4g + r, c = 16ct + l%16
template <int STG>
__device__ __forceinline__ void k_iteration(const BwdArgs& A, f32x4 (&acc)[16], float& dz, uint8_t* smem0,
                                            uint8_t* smem1, const KSrc& src, bool inv_reg, int invv,
                                            const int32_t* invG, int x, int cnt, int bh, float ksc, int& i,
                                            float& sq, const KOps& ko, bool sparse, bool kok, int wc, int l16,
                                            int g, int tid) {
  const uint8_t* stg = STG == 0 ? smem0 : smem1;
  uint8_t* next = STG == 0 ? smem1 : smem0;
  // dZ_i (correction waves, one feature per thread) is loaded before the copies are issued:
  // waiting for it then never waits for them
  const int zt = tid - 4 * 64;
  const float dzi = (!sparse && zt < kD) ? A.dZ[((size_t)bh * A.T + i) * kD + zt] : 0.f;
  __builtin_amdgcn_sched_barrier(0);
  int i_next = 0;
  float sq_next = 1.f;
  if (x + 1 < cnt) {
    i_next = list_entry(inv_reg, invv, invG, x + 1);
    sq_next = A.q_scale[(size_t)bh * A.T + i_next];
    k_dma(src, i_next, A.N, tid, next);
  }
  __builtin_amdgcn_sched_barrier(0);

  if (sparse) {
    const float inv_sqrt_d = 0.08838834764831845f;   // 1 / sqrt(128)
    // P and dS (times q_scale / sqrt(d), the factor of dK' = dS^T Q' / sqrt(d)) of query half s
    // (tiles 2s, 2s+1) as B operands, with the pair's -lse log2(e) and D_q at rows 16mt + 4g .. +3
    const float* rec = reinterpret_cast<const float*>(stg + klds::REC);
    const float cij = kLog2e * inv_sqrt_d * sq * ksc, fk = sq * inv_sqrt_d;
    // P is 0 for pad keys (their scores start from -inf in the product's accumulator) and pad
    // queries (their record holds -inf for -lse log2(e)), with no per-element test
    const float kbias = kok ? 0.f : -INFINITY;
    f32x4 S[4], dP[4], l4[2], d4[2];
    bf16x8 po[2], dso_[2];
    auto read_rec = [&](int s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        l4[h] = *reinterpret_cast<const f32x4*>(rec + 16 * (2 * s + h) + 4 * g);
        d4[h] = *reinterpret_cast<const f32x4*>(rec + kBlock + 16 * (2 * s + h) + 4 * g);
      }
    };
    auto half_ops = [&](int s) {
      float p8[8], d8[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int mt = 2 * s + h;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[mt][rr], cij, l4[h][rr]));
          p8[4 * h + rr] = p;
          d8[4 * h + rr] = p * (dP[mt][rr] - d4[h][rr]) * fk;
        }
      }
      po[s] = pack8(p8);
      dso_[s] = pack8(d8);
    };
    // operand reads run one query tile ahead of the products that use them
    i32x8 qr[4];
    bf16x8 da[4][4];
    auto read_queries = [&](auto mt) {
      qr[mt] = lds_fp8_row(stg + klds::Q8, 16 * mt + l16, g);
#pragma unroll
      for (int s = 0; s < 4; ++s) da[mt][s] = op256(stg + klds::DO, 16 * mt + l16, s, g);
    };
    read_rec(0);
    read_queries(std::integral_constant<int, 0>{});
    static_for<4>([&](auto mt) {
      if constexpr (mt + 1 < 4) read_queries(std::integral_constant<int, mt + 1>{});
      S[mt] = mfma_fp8(qr[mt], ko.k8, f32x4{kbias, kbias, kbias, kbias});
      dP[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) dP[mt] = mfma_bf16(da[mt][s], ko.v[s], dP[mt]);
      if constexpr (mt == 2) {   // the first half's operands, while tile 2's products run
        half_ops(0);
        read_rec(1);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    half_ops(1);
    bf16x8 fo[8][2], fq[8][2];
    auto read_feat = [&](auto ct) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        fo[ct][s] = dot_op(stg + klds::DO, s, 16 * ct, l16, g);
        fq[ct][s] = op128(stg + klds::QT, 16 * ct + l16, s, g);
      }
    };
    static_for<kKReadAhead>([&](auto ct) { read_feat(ct); });
    static_for<8>([&](auto ct) {
      if constexpr (ct + kKReadAhead < 8) read_feat(std::integral_constant<int, ct + kKReadAhead>{});
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        acc[ct] = mfma_bf16(fo[ct][s], po[s], acc[ct]);
        acc[8 + ct] = mfma_bf16(fq[ct][s], dso_[s], acc[8 + ct]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  } else {
    bf16x8 fa[2][2];
#pragma unroll
    for (int at = 0; at < 2; ++at)
#pragma unroll
      for (int s = 0; s < 2; ++s) fa[at][s] = op128(stg + klds::PT, 32 * wc + 16 * at + l16, s, g);
    bf16x8 fo[8][2];
    auto read_feat = [&](auto ct) {
#pragma unroll
      for (int s = 0; s < 2; ++s) fo[ct][s] = dot_op(stg + klds::DO, s, 16 * ct, l16, g);
    };
    static_for<kKReadAhead>([&](auto ct) { read_feat(ct); });
    static_for<8>([&](auto ct) {
      if constexpr (ct + kKReadAhead < 8) read_feat(std::integral_constant<int, ct + kKReadAhead>{});
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        acc[ct] = mfma_bf16(fa[0][s], fo[ct][s], acc[ct]);
        acc[8 + ct] = mfma_bf16(fa[1][s], fo[ct][s], acc[8 + ct]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  dz += dzi;
  wait_dma();
  lds_barrier();
  i = i_next;
  sq = sq_next;
}

__global__ __launch_bounds__(512, 1) void bwd_key_kernel(BwdArgs A) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[klds::STAGE];   // stage of even list entries
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[klds::STAGE];   // stage of odd list entries
  __shared__ float dzS[kD], alS[kD];
  const int lid = xcd_remap(blockIdx.x, A.nblocks);
  const int bh = __builtin_amdgcn_readfirstlane(lid / A.T), j = __builtin_amdgcn_readfirstlane(lid % A.T);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const bool sparse = w < 4;
  const int wc = w & 3;
  const int hidx = bh % A.H, T = A.T, N = A.N;
  const int kk = kBlock * j + 16 * wc + l16;   // sparse waves: this lane's key
  const bool kok = kk < N;
  const int cnt = __builtin_amdgcn_readfirstlane(A.inv_cnt[(size_t)bh * T + j]);
  const int32_t* invG = A.inv + ((size_t)bh * T + j) * T;
  const bool inv_reg = cnt <= 64;
  const int invv = (inv_reg && lane < cnt) ? invG[lane] : 0;

  KSrc src;
  src.q8 = rsrc(A.q8 + (size_t)bh * T * kBlock * kD, (size_t)T * kBlock * kD);
  src.dout = rsrc(A.dout + (size_t)bh * N * kD, (size_t)N * kD * 2);
  src.qt = rsrc(A.q8t + (size_t)bh * T * kD * kBlock, (size_t)T * kTTile);
  src.pt = rsrc(A.phqdt + (size_t)bh * T * kD * kBlock, (size_t)T * kTTile);
  src.rec = rsrc(A.qrec + (size_t)bh * T * kRec, (size_t)T * kRec * 4);
  int i = 0;
  float sq = 1.f;
  if (cnt > 0) {
    i = list_entry(inv_reg, invv, invG, 0);
    sq = A.q_scale[(size_t)bh * T + i];
    k_dma(src, i, N, tid, smem0);
  }

  KOps ko;
  ko.k8 = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 4; ++s) ko.v[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  if (sparse) {
    const uint8_t* s8 = A.k8 + ((size_t)bh * T * kBlock + kk) * kD + 32 * g;   // pad rows: code 0
    const u32x4 a = *reinterpret_cast<const u32x4*>(s8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(s8 + 16);
    ko.k8 = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 32 * s + 8 * g;
      const u32x4 raw = kok ? *reinterpret_cast<const u32x4*>(A.v + ((size_t)bh * N + kk) * kD + c) : u32x4{0, 0, 0, 0};
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(A.alpha + (size_t)hidx * kD + c);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(A.alpha + (size_t)hidx * kD + c + 4);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
      float v8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = av[e] * ((e & 1) ? bf16_hi(rw[e >> 1]) : bf16_lo(rw[e >> 1]));
      ko.v[s] = pack8(v8);   // dP = dO_s V^T = dO (alpha V)^T
    }
  }
  const float ksc = A.k_scale[(size_t)bh * T + j];
  if (tid < kD) alS[tid] = A.alpha[(size_t)hidx * kD + tid];

  f32x4 acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dz = 0.f;
  wait_dma();
  lds_barrier();

  // pairs of list entries, then the odd last one (a loop body without a branch on the count)
  int x = 0;
  for (; x + 1 < cnt; x += 2) {
    k_iteration<0>(A, acc, dz, smem0, smem1, src, inv_reg, invv, invG, x, cnt, bh, ksc, i, sq, ko, sparse, kok, wc,
                   l16, g, tid);
    k_iteration<1>(A, acc, dz, smem0, smem1, src, inv_reg, invv, invG, x + 1, cnt, bh, ksc, i, sq, ko, sparse, kok,
                   wc, l16, g, tid);
  }
  if (x < cnt)
    k_iteration<0>(A, acc, dz, smem0, smem1, src, inv_reg, invv, invG, x, cnt, bh, ksc, i, sq, ko, sparse, kok, wc,
                   l16, g, tid);

  // ---------------- epilogue
  // correction waves: dh_j = (G_tot - C) diag(1 - alpha) as bf16 images with rows a and rows c,
  // and dz_j
  const LTile<256> DH{smem0}, DHT{smem1};
  if (!sparse) {
    const int zt = tid - 4 * 64;
    if (zt < kD) dzS[zt] = A.dZ_tot[(size_t)bh * kD + zt] - dz;
    const float* gt = A.g_tot + (size_t)bh * kD * kD;
#pragma unroll
    for (int at = 0; at < 2; ++at)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int a = 32 * wc + 16 * at + 4 * g + rr, c = 16 * ct + l16;
          const uint16_t bv = f32_to_bf16((gt[a * kD + c] - acc[8 * at + ct][rr]) * (1.f - alS[c]));
          *DH.el16(a, c) = bv;
          *DHT.el16(c, a) = bv;
        }
  }
  __syncthreads();
  __shared__ float csum[4][kD];   // per sparse wave: column sums of dK~ over its 16 keys
  if (sparse) {
    // phi(k~) of this lane's key: as B operand (features 32s + 8g + e) and at the accumulator
    // features 16at + 4g + r
    bf16x8 pko[4];
    float pk[8][4];
    {
      const uint16_t* kr = A.k + ((size_t)bh * N + min(kk, N - 1)) * kD;
      const float* mu = A.k_mean + (size_t)bh * kD;
      float fb[4][8];
      float mx = -INFINITY;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * g);
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          fb[s][2 * e] = bf16_lo(ww[e]) - mu[32 * s + 8 * g + 2 * e];
          fb[s][2 * e + 1] = bf16_hi(ww[e]) - mu[32 * s + 8 * g + 2 * e + 1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fb[s][e]);
      }
      mx = rows4_max(mx);
      float sm = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          fb[s][e] = __expf(fb[s][e] - mx);
          sm += fb[s][e];
        }
      const float rsum = 1.f / rows4_sum(sm);
      const float is = kok ? rsum : 0.f;   // pad keys: phi(k) = 0
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) fb[s][e] *= is;
        pko[s] = pack8(fb[s]);
      }
#pragma unroll
      for (int at = 0; at < 8; ++at) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(kr + 16 * at + 4 * g);
        const float raw[4] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y)};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) pk[at][rr] = __expf(raw[rr] - mu[16 * at + 4 * g + rr] - mx) * is;
      }
    }
    // dphi(k)^T = dh_j V^T + dz_j (V of this lane's key, unscaled); dV^T = alpha dV_sparse^T +
    // dh_j^T phi(k)^T
    bf16x8 vk[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      vk[s] = __builtin_bit_cast(bf16x8, kok ? *reinterpret_cast<const u32x4*>(A.v + ((size_t)bh * N + kk) * kD + 32 * s + 8 * g)
                                             : u32x4{0, 0, 0, 0});
    float dphi[8][4], dotp = 0.f;
#pragma unroll
    for (int at = 0; at < 8; ++at) {
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) t = mfma_bf16(DH.op(16 * at + l16, 32 * s + 8 * g), vk[s], t);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        dphi[at][rr] = t[rr] + dzS[16 * at + 4 * g + rr];
        dotp = fmaf(pk[at][rr], dphi[at][rr], dotp);
      }
    }
    dotp = rows4_sum(dotp);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[ct][rr] *= alS[16 * ct + 4 * g + rr];
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[ct] = mfma_bf16(DHT.op(16 * ct + l16, 32 * s + 8 * g), pko[s], acc[ct]);
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      f32x4 o;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) o[rr] = kok ? acc[8 + ct][rr] + pk[ct][rr] * (dphi[ct][rr] - dotp) : 0.f;
      if (kok) {
        *reinterpret_cast<f32x4*>(A.dkt + ((size_t)bh * T * kBlock + kk) * kD + 16 * ct + 4 * g) = o;
        u32x2 sv;
        sv.x = pack_bf16x2(acc[ct][0], acc[ct][1]);
        sv.y = pack_bf16x2(acc[ct][2], acc[ct][3]);
        *reinterpret_cast<u32x2*>(A.dv + ((size_t)bh * N + kk) * kD + 16 * ct + 4 * g) = sv;
      }
      // sums over this wave's 16 keys (the lanes of a 16-lane row) for the key-smoothing mean
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float cs = row16_sum(o[rr]);
        if (l16 == 0) csum[wc][16 * ct + 4 * g + rr] = cs;
      }
    }
  }
  __syncthreads();
  if (tid < kD)
    A.colsum_part[((size_t)bh * T + j) * kD + tid] = (csum[0][tid] + csum[1][tid]) + (csum[2][tid] + csum[3][tid]);
}

// mean over the N tokens of dK~ (zero without key smoothing) from the key blocks' column sums:
// 8 partial sums per feature over interleaved blocks, combined in fixed order
__global__ __launch_bounds__(1024) void bwd_mean_kernel(BwdArgs A) {
  __shared__ float red[8][kD];
  const int bh = blockIdx.x, c = threadIdx.x & (kD - 1), u = threadIdx.x >> 7;
  float s = 0.f;
#pragma unroll 8
  for (int j = u; j < A.T; j += 8) s += A.colsum_part[((size_t)bh * A.T + j) * kD + c];
  red[u][c] = s;
  __syncthreads();
  if (u == 0) {
    float t = 0.f;
    for (int k = 0; k < 8; ++k) t += red[k][c];
    A.dk_mean[(size_t)bh * kD + c] = A.smooth_k ? t / (float)A.N : 0.f;
  }
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
#pragma unroll 8
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
  A.h_sum = t.h_sum;
  A.z_sum = t.z_sum;
  A.zrout = ws.zrout;
  A.os = bw.os;
  A.ol = bw.ol;
  A.inv_den = bw.inv_den;
  A.q8t = bw.q8t;
  A.phqdt = bw.phqdt;
  A.k8t = bw.k8t;
  A.phkt = bw.phkt;
  A.htimg = bw.htimg;
  A.qrec = bw.qrec;
  A.dden = bw.dden;
  A.inv = bw.inv;
  A.inv_cnt = bw.inv_cnt;
  A.dZ = bw.dZ;
  A.gpart = bw.gpart;
  A.zpart = bw.zpart;
  A.g_tot = bw.g_tot;
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
  A.pg = (g.T + kGChunk - 1) / kGChunk;
  A.nblocks = g.BH * g.T;
  A.smooth_k = g.smooth_k ? 1 : 0;
  const dim3 blocks(g.T, g.BH);
  hipLaunchKernelGGL(bwd_prep_kernel, blocks, dim3(256), 0, s, A);
  hipLaunchKernelGGL(bwd_invlut_kernel, blocks, dim3(64), 0, s, A);
  hipLaunchKernelGGL(bwd_gtot_kernel, dim3(A.pg, g.BH), dim3(256), 0, s, A);
  hipError_t e = launch_sum_parts(bw.gpart, bw.zpart, A.pg, g.D, g.BH, bw.g_tot, bw.dZ_tot, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_query_kernel, dim3(A.nblocks), dim3(kNT2), 0, s, A);
  hipLaunchKernelGGL(bwd_key_kernel, dim3(A.nblocks), dim3(kNT2), 0, s, A);
  hipLaunchKernelGGL(bwd_mean_kernel, dim3(g.BH), dim3(1024), 0, s, A);
  hipLaunchKernelGGL(bwd_dk_kernel, dim3((g.N * 16 + 255) / 256, g.BH), dim3(256), 0, s, A);
  hipLaunchKernelGGL(bwd_dalpha_kernel, dim3(g.H), dim3(1024), 0, s, A);
  return hipGetLastError();
}

}  // namespace sla2
