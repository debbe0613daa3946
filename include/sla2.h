/*
 * sla2.h - C ABI of the SLA2 sparse-linear attention forward pass on MI355X (gfx950).
 *
 * The method is the one described on the pages
 *   "SLA2: Sparse-Linear Attention with Learnable Routing and QAT" (AI summary page) and
 *   "SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable Sparse-Linear
 *    Attention" (detailed summary page).
 * Per (batch b, head h), with blocks of 64 consecutive tokens (T = ceil(N/64), the last
 * block may be partial):
 *   1. router (SLA2 page, section 4): mean-pool Q and the smoothed keys K~ = K - mean_N(K)
 *      over each block, project the pooled rows with d x d matrices W_q, W_k, score every
 *      (query block, key block) pair and keep the `topk` best key blocks of each query-block
 *      row (hard Top-k, section 7) as the sparse set; all other key blocks go to the linear
 *      branch.
 *   2. sparse branch (SLA2 page, sections 3 and 5): softmax attention of each query over the
 *      keys of its routed blocks only, online softmax, with Q.K^T optionally in FP8 e4m3
 *      (one absmax scale per 64-token block) and P.V in the input precision.
 *   3. linear branch (SLA page, sections 2-4): phi = softmax over the d features,
 *      h_j = phi(K~_j)^T V_j and z_j = column sums of phi(K~_j) per key block;
 *      O_l = phi(Q) H_i / (phi(Q) . Z_i + eps) with H_i, Z_i summed over the unrouted blocks.
 *   4. mix (SLA2 page, section 3): O = alpha * O_s + (1 - alpha) * O_l, alpha in [0,1]^d
 *      per head.
 *
 * Conventions for every entry point below:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronises.  Every call only enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the default stream) and returns.
 *   - Token tensors are [B, H, N, d] row-major and contiguous.  Element type: float32
 *     (SLA2_F32) or bf16 (SLA2_BF16, raw 16-bit patterns).
 *   - Arguments are checked on the host before anything is launched; on failure the call
 *     returns a negative sla2_status, launches nothing and sla2_last_error() describes it
 *     (thread-local).  A failed kernel launch returns SLA2_ERR_HIP.
 *   - Calls must be made in the order sla2_route -> sla2_linear_precompute ->
 *     sla2_attention_fwd with the same params and tensors; each reads what the previous
 *     wrote (k_mean, lut, q8/k8, h, z, h_sum, z_sum and the workspace).
 *   - Pointers a call does not use may be NULL; a NULL pointer it needs is rejected with
 *     SLA2_ERR_INVALID_ARG and a message naming the tensor.
 *   - Results are deterministic: every reduction has a fixed order.
 *   - Inputs must be finite.
 */
#ifndef SLA2_H
#define SLA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLA2_OK = 0,
  SLA2_ERR_INVALID_ARG = -1,  /* a size, mode or pointer is out of range; nothing launched  */
  SLA2_ERR_UNSUPPORTED = -2,  /* a valid combination this build does not implement          */
  SLA2_ERR_HIP = -3           /* the HIP runtime reported an error                          */
} sla2_status;

typedef enum { SLA2_F32 = 0, SLA2_BF16 = 1 } sla2_dtype;

/* Arithmetic of the sparse branch's Q.K^T (SLA2 page, section 5, low-bit attention). */
typedef enum {
  SLA2_QK_NATIVE = 0,   /* Q.K^T in the input precision                                    */
  SLA2_QK_FP8_E4M3 = 1, /* OCP e4m3 codes, one absmax/448 scale per 64-token block (bf16)  */
  /* Mode 1 plus the sparse branch's P.V in e4m3 (SLA2 page, section 5: P and V quantised, the
   * product dequantised).  V: one power-of-two scale per (64-token block, channel), the
   * smallest 2^e >= absmax/448 (e >= -127).  P: one power-of-two scale per (query, routed
   * block), 2^(ceil(M) - 8) with M the block's largest score in log2 units, so the largest
   * code lies in [128, 256].  The softmax normaliser sums the unquantised P.  The routed part
   * of the linear branch (see sla2_attention_fwd) uses the same e4m3 V with the phi products
   * as e4m3 codes of scale 2^10.  bf16, d = 128, forward only (the backward returns
   * SLA2_ERR_UNSUPPORTED). */
  SLA2_QK_PV_FP8_E4M3 = 2
} sla2_qk_mode;

typedef struct sla2_params {
  int32_t B, H, N, d;   /* batch, heads, tokens (>= 1), head dim (64 or 128)                 */
  int32_t block;        /* token block size b_q = b_kv; must be 64 (SLA page, section 2)     */
  int32_t topk;         /* routed key blocks per query-block row, 1 <= topk <= T             */
  int32_t smooth_k;     /* 1: subtract the per-(b,h) token mean from K (SLA2 page, sec. 6)   */
  int32_t dtype;        /* sla2_dtype of q, k, v, o, h, vt                                   */
  int32_t qk_mode;      /* sla2_qk_mode; modes 1 and 2 need dtype SLA2_BF16                  */
  float eps;            /* linear-branch denominator guard, 1e-5 (SLA page, section 4)       */
} sla2_params;

/* Byte sizes of every caller-owned buffer for given params (0 = buffer unused). */
typedef struct sla2_sizes {
  size_t q_pool, k_pool, k_mean, lut, mask;
  size_t q8, k8, q_scale, k_scale;
  size_t h, z, h_sum, z_sum;
  size_t o, lse;
  size_t workspace;
  size_t workspace_bwd;   /* scratch of sla2_attention_bwd (0 where the backward is unsupported) */
} sla2_sizes;

typedef struct sla2_tensors {
  /* ---- inputs ---- */
  const void *q, *k, *v;   /* [B,H,N,d] dtype                                                */
  const float *wq, *wk;    /* [d,d] row-major [in][out], shared by all heads; NULL = identity */
  const float *alpha;      /* [H,d], values in [0,1]                                          */
  /* ---- written by sla2_route ---- */
  float *q_pool;           /* [B,H,T,d] block means of Q                                     */
  float *k_pool;           /* [B,H,T,d] block means of K~ (= block means of K minus k_mean)   */
  float *k_mean;           /* [B,H,d] token mean of K (zeros when smooth_k = 0)              */
  int32_t *lut;            /* [B,H,T,topk] routed key blocks of each query block, ascending  */
  uint8_t *mask;           /* [B,H,T,T] compressed mask: 1 = sparse branch, 0 = linear       */
  uint8_t *q8;             /* FP8 mode: [B,H,T*64,d] e4m3 codes of Q / q_scale (pad rows 0)  */
  float *q_scale;          /* FP8 mode: [B,H,T] absmax/448 of each Q block (1 if all zero)   */
  /* ---- written by sla2_linear_precompute ---- */
  uint8_t *k8;             /* FP8 mode: [B,H,T*64,d] e4m3 codes of K~ / k_scale              */
  float *k_scale;          /* FP8 mode: [B,H,T]                                              */
  void *h;                 /* [B,H,T,d,d] dtype, TRANSPOSED: h[j][c][a] = sum over the valid
                              tokens t of block j of phi(K~_t)[a] * V_t[c].  Required for
                              SLA2_F32; optional (NULL = not written) for SLA2_BF16, whose
                              forward never reads it                                           */
  float *z;                /* [B,H,T,d] z[j][a] = sum_t phi(K~_t)[a]; same rule as h          */
  float *h_sum;            /* [B,H,d,d] sum of h over all blocks (same transposed layout)    */
  float *z_sum;            /* [B,H,d]                                                        */
  /* ---- written by sla2_attention_fwd ---- */
  void *o;                 /* [B,H,N,d] dtype                                                */
  float *lse;              /* [B,H,N] or NULL: natural log of the sum over the routed keys s of
                              exp(q_t . K~_s / sqrt(d)) (dequantised operands in FP8 mode)   */
  /* ---- scratch shared by the three calls ---- */
  void *workspace;         /* sla2_sizes.workspace bytes, 256-byte aligned                    */
  /* ---- scratch of the backward pass only ---- */
  void *workspace_bwd;     /* sla2_sizes.workspace_bwd bytes, 256-byte aligned                */
} sla2_tensors;

/* Host only, pure: fills *out with the byte size of every buffer for *p.
 * Returns SLA2_OK or SLA2_ERR_INVALID_ARG / SLA2_ERR_UNSUPPORTED for params the calls
 * below would reject. */
int sla2_buffer_sizes(const sla2_params *p, sla2_sizes *out);

/* Router (SLA2 page, section 4; SLA page, section 2 Q2 step 1) plus the FP8 quantisation
 * of Q (SLA2 page, section 5).  Reads q, k, wq, wk; writes q_pool, k_pool, k_mean, lut,
 * mask and, in FP8 mode, q8 and q_scale.  Block scores are
 * s_ij = (q_pool_i W_q).(k_pool_j W_k) / sqrt(d), computed in fp64; ties in the Top-k go to
 * the lower block index.  Needs T <= 4096. */
int sla2_route(const sla2_params *p, const sla2_tensors *t, void *stream);

/* sla2_route for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * sla2_route, except that the router's scratch (fp64 block sums, key-mean partials, the
 * projected pooled rows and the block scores: 32 * d + 8 * ceil(N/64) bytes per query block of
 * every head) comes from a 64 MiB device array the library holds on each GPU it runs on until
 * the process ends, not from t->workspace, which is not read and may be NULL.  Sizes needing
 * more return SLA2_ERR_UNSUPPORTED before anything is launched (the 12-head, 32760-token layer
 * at d = 128 needs 50 MB).  Allocates nothing; the first call
 * on a device looks up that device's copy of the array.  Every call on a GPU shares its copy,
 * so calls that overlap on one GPU (on other streams or threads) race; each call overwrites
 * everything of it that it reads, so nothing needs clearing between calls. */
int sla2_route_noalloc(const sla2_params *p, const sla2_tensors *t, void *stream);

/* SoftTop-k router for training (SLA2 page, section 4: training replaces the hard Top-k by
 * SoftTop-k, which keeps the row sum; section 6: a sigmoid with temperature tau and a per-row
 * offset lambda_i found by binary search so that each row sums to k_sel).  Runs everything
 * sla2_route does (same reads and writes, including the hard lut and mask the kernels use),
 * then, from the same fp64 scores:
 *   P_ij = softmax_j(s_ij) (the compressed attention of SLA page, section 2 Q2 step 1),
 *   soft_mask[b,h,i,j] = sigmoid((P_ij - lambda_i) / tau),  lambda[b,h,i] = lambda_i,
 * with lambda_i the root of sum_j sigmoid((P_ij - lambda)/tau) = k_sel in [min_j P_ij -
 * tau (ln T + 2), max_j P_ij + tau (ln T + 2)], the value a binary search over that bracket
 * converges to (fp64; each row then sums to k_sel up to rounding).  The search keeps the
 * bracket and steps to the Newton point of the row sum when it lies inside, else to the
 * midpoint, until a Newton step is below 2^-30 of lambda (at most 60 steps).  k_sel = T gives
 * soft_mask = 1 and lambda = -inf.
 * soft_mask: device float[B,H,T,T]; lambda: device float[B,H,T]; both caller-owned.
 * tau must be positive and finite (else SLA2_ERR_INVALID_ARG). */
int sla2_route_soft(const sla2_params *p, const sla2_tensors *t, float tau, float *soft_mask,
                    float *lambda, void *stream);

/* Linear-branch precompute (SLA page, sections 2-3: h_j = phi(K_j)^T V_j, z_j =
 * rowsum phi(K_j)^T) plus the FP8 quantisation of K~.  Reads k, v and k_mean (not the lut);
 * writes h_sum, z_sum, h and z (when given), and in FP8 mode k8, k_scale.  For SLA2_BF16 it
 * also stages into the workspace what the fused forward reads: V^T tiles, e4m3 codes of
 * 448 phi(K~), z_j of every block and a bf16 image of h_sum^T.  It needs only sla2_route's
 * k_mean (running it beside the router's Top-k on a second stream was measured and gave no
 * gain: both fill the CUs' LDS). */
int sla2_linear_precompute(const sla2_params *p, const sla2_tensors *t, void *stream);

/* Fused sparse + linear + mix forward (SLA2 page, sections 3 and 6: sparse attention over
 * the M = 1 blocks, linear-attention statistics over the M = 0 blocks, O = alpha * O_s +
 * (1 - alpha) * O_l).  Reads q, k (native mode), v, alpha, lut, q8/q_scale, k8/k_scale,
 * h_sum, z_sum, k_mean, the workspace and, for SLA2_F32, h and z; writes o and, if non-NULL,
 * lse.  The linear statistics of query block i are those of its unrouted blocks, formed as
 * the totals minus the routed part: H_i = h_sum - sum over routed j of h_j, Z_i likewise (with
 * more than half of the blocks routed, a third for SLA2_QK_PV_FP8_E4M3, SLA2_BF16 sums
 * phi(Q_i) H_i over the unrouted blocks directly instead, since that difference would be small
 * next to its terms).
 * SLA2_F32 gathers the routed h_j, z_j; SLA2_BF16 evaluates phi(q) times the routed part of
 * H by re-association, as the sum over the routed keys s of (phi(q).phi(K~_s)) V_s (SLA page,
 * section 4), with phi(q) and phi(K~) as e4m3 codes of 448 phi (both phi <= 1), and sums
 * the routed part of Z from the precompute's per-block z_j as it walks the LUT row.
 * SLA2_QK_PV_FP8_E4M3: the P.V products of both uses take e4m3 P (or phi-product codes) and
 * e4m3 V from the precompute, with their power-of-two scales applied by the matrix cores.
 * Training forward: when t->workspace_bwd is non-NULL (and the backward supports the params:
 * SLA2_BF16, SLA2_QK_FP8_E4M3, d = 128) the call also stores in it, per query, the sparse
 * output O_s, the linear output O_l (both bf16) and 1/(phi(q).Z_i + eps), and per query block
 * the routed part of Z (in the workspace), which the backward reads; a workspace_bwd that is
 * not 256-byte aligned is SLA2_ERR_INVALID_ARG. */
int sla2_attention_fwd(const sla2_params *p, const sla2_tensors *t, void *stream);

/* Backward pass (SLA2 page, appendix A: gradients of Q, K, V through phi(Q), phi(K) and the
 * per-query-block dH_i, dZ_i, each key block collecting them from the query blocks that do not
 * route to it; section 5: low-bit forward, 16-bit backward).  Gradients of sum(dout * o) with
 * the routing held fixed (no gradient reaches W_q, W_k or the pooling), the FP8 quantiser
 * passed straight through (dQ' -> dQ, dK' -> dK~), and key smoothing differentiated
 * (dK = dK~ - mean over tokens of dK~ when smooth_k).
 * Supported: dtype SLA2_BF16, qk_mode SLA2_QK_FP8_E4M3, d = 128 (else SLA2_ERR_UNSUPPORTED; the
 * pages' backward is 16-bit, so a low-bit P.V forward has none here).
 * Reads what the three forward calls wrote for the same params and inputs: q, k, v, alpha,
 * k_mean, lut, mask, q8, q_scale, k8, k_scale, h_sum, z_sum, lse (so the forward must have
 * been given lse), the workspace, and the O_s, O_l, 1/den and routed part of Z that a training
 * forward (one given this workspace_bwd) stored; h and z are not read.  Writes only workspace_bwd and the outputs.
 * The linear branch never forms H_i or dH_i per block: the query side re-associates the routed
 * part of dnum H_i^T over the routed key tiles, and each key block forms its dh_j as the total
 * minus one product per routing query block.
 *   dout:   device bf16 [B,H,N,d], the gradient of the loss with respect to o;
 *   dq, dk, dv: device bf16 [B,H,N,d];
 *   dalpha: device float [H,d], summed over the batch and the tokens.
 * The matrix products take bf16 (and, for the scores, e4m3) operands with fp32 accumulation. */
int sla2_attention_bwd(const sla2_params *p, const sla2_tensors *t, const void *dout,
                       void *dq, void *dk, void *dv, float *dalpha, void *stream);

/* Diagnostic: runs one wave (64 lanes) of one matrix-core instruction the kernels use,
 * so a test can pin the operand lane layouts the kernels assume.
 *   which = 0: v_mfma_f32_16x16x32_bf16, a/b = 64 lanes x 8 bf16 (16 bytes per lane)
 *   which = 1: v_mfma_f32_16x16x128_f8f6f4 with e4m3 operands, 64 lanes x 32 bytes
 *   which = 2: v_mfma_f64_16x16x4_f64, a/b = 64 lanes x 1 double
 *   which = 3: v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 operands as for 1, each followed by
 *              64 lanes x one 32-bit scale word (E8M0 exponent bytes); the instruction takes
 *              byte 2 of A's word and byte 0 of B's (2304 bytes per operand)
 *   which = 4: no matrix instruction: the kernels' e4m3 decode, lane l decoding the four code
 *              bytes of 32-bit word l of a (256 bytes) into d[4l..4l+3]; b is not read
 * a, b: device arrays of the lane-major operand registers; d: device array of the lane-major
 * accumulator registers of the result (C = 0): float[64*4] for which = 0, 1, 3 and 4,
 * double[64*4] for which = 2.  Returns SLA2_ERR_INVALID_ARG for other values of `which`. */
int sla2_selftest_mfma(int which, const void *a, const void *b, void *d, void *stream);

const char *sla2_status_string(int status);
const char *sla2_last_error(void);   /* message of the last failed call on this thread */

#ifdef __cplusplus
}
#endif
#endif /* SLA2_H */
