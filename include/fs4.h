/*
 * fs4.h — C ABI of libfs4: the NVFP4-quantized linear projection of
 * Full-Stack FP4 on AMD MI355X (gfx950).
 *
 * Citation key: [FS4 §n] = "Full-Stack FP4: Stable LLM Pretraining with
 * Quantized Projections, Optimizers, and Attention" (arXiv 2607.04422),
 * technical summary on gist.science (Spanish and French editions), section n.
 *
 * The pages name NVFP4 without defining it; this library implements the
 * two-level block format:
 *   - E2M1 element codes, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, bit 3 = sign;
 *   - one E4M3 (FN) decode scale per 16 consecutive elements along the
 *     contraction dimension;
 *   - one FP32 decode scale per tensor, s_t = RNE_fp32(amax / 2688);
 *   - s_b = E4M3 round-to-nearest-even (satfinite) of amax_b / (6 s_t);
 *   - code = sign | E2M1 round-to-nearest-even of |x| / (s_b s_t), the
 *     division exact, ties to the even code; the signed zero when s_b s_t = 0;
 *   - x_hat = e2m1(code) * e4m3(s_b) * s_t.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless a comment says otherwise; the caller
 *     owns every buffer.  The library never allocates, frees, synchronises or
 *     copies to the host; every call is asynchronous on `stream` (a
 *     hipStream_t; NULL = the null stream).
 *   - All arguments are validated on the host BEFORE anything is launched; on
 *     an error status nothing was launched and no output was touched.  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Dimensions are element counts.  Every dimension that is blocked in some
 *     quantized view must be a positive multiple of 16 (FS4_ERR_SHAPE).
 *     Device pointers must be 16-byte aligned (FS4_ERR_ALIGN).
 *   - Inputs must be finite; NaN/Inf inputs give unspecified outputs.
 *   - `ws` is a caller-provided device workspace of at least the size the
 *     matching fs4_*_workspace_bytes() call returns (256-byte aligned).
 *   - Calls are reentrant; calls that share a workspace or an output buffer
 *     must be ordered on one stream.
 *   - Output buffers may overlap neither the inputs, nor each other, nor the
 *     workspace (fs4_newton_schulz checks its iterate buffer; the other calls
 *     do not check).
 */
#ifndef FS4_H
#define FS4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FS4_OK = 0,
  FS4_ERR_NULL = 1,      /* a required pointer is NULL                          */
  FS4_ERR_SHAPE = 2,     /* a dimension is negative, not a multiple of 16, or
                            views/buffers disagree on a dimension                */
  FS4_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned            */
  FS4_ERR_DTYPE = 4,     /* unknown fs4_dtype                                  */
  FS4_ERR_RANK = 5,      /* low-rank r outside [0, 64], or U/V NULL with r > 0  */
  FS4_ERR_WORKSPACE = 6, /* ws_bytes smaller than required                     */
  FS4_ERR_HIP = 7,       /* a kernel launch failed                              */
  FS4_ERR_ARG = 8        /* another argument is out of range (e.g. steps < 0)  */
} fs4_status;

typedef enum { FS4_BF16 = 0, FS4_FP32 = 1 } fs4_dtype;

/* One NVFP4 view of a [rows][cols] tensor; cols is the blocked (contraction)
 * dimension and is contiguous.
 *   codes  [rows][cols/2]   byte j of a row = code[2j] | code[2j+1] << 4
 *   scales [rows][cols/16]  raw E4M3FN block decode scales
 *   tscale 1 float          the FP32 tensor decode scale (on the device)
 * A "row-wise" view of x[R][C] has rows = R, cols = C.  A "column-wise" view
 * of x has rows = C, cols = R: the row-wise quantization of x^T (different
 * blocks, so a different quantization) with the same tensor scale. */
typedef struct {
  uint8_t *codes;
  uint8_t *scales;
  float *tscale;
  int64_t rows;
  int64_t cols;
} fs4_nvfp4;

/* ---------------------------------------------------------------------------
 * fs4_quantize — two-level NVFP4 quantization of x[rows][cols] (bf16 or fp32,
 * row-major), emitting the row-wise view, the column-wise view, or both, with
 * one shared tensor scale.  [FS4 §2.1] (residual held in NVFP4), [FS4 §2.3]
 * (Newton-Schulz operands in NVFP4).
 *   rowwise:  rows = rows, cols = cols (cols % 16 == 0), or NULL
 *   colwise:  rows = cols, cols = rows (rows % 16 == 0), or NULL
 * At least one view must be given.  Both views' tscale receive s_t (they may
 * point to the same float).  rows == 0 or cols == 0 writes s_t = 0 only.
 * Codes and scales are bit-exact with the definition in the file header.
 */
size_t fs4_quantize_workspace_bytes(int64_t rows, int64_t cols);
fs4_status fs4_quantize(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                        const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise,
                        void *ws, size_t ws_bytes, void *stream);

/* fs4_quantize_noalloc — fs4_quantize without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight loops, harnesses that forbid allocation.  The caller passes only the
 * input and the output views; the quantizer's scratch (its 4 KB of amax
 * partials, the same for every input size, fs4_quantize_noalloc_scratch_bytes)
 * lives in a device array of the library that each GPU holds from the first
 * call on it until the process ends.  Nothing is allocated or freed.  Calls
 * that overlap on one GPU (concurrent streams, or threads) share that array
 * and race; serialise them.  Arguments, results and errors as fs4_quantize;
 * also FS4_ERR_HIP when the array's device address cannot be obtained.
 */
size_t fs4_quantize_noalloc_scratch_bytes(void);
fs4_status fs4_quantize_noalloc(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                                const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_gemm_nt — C[M][N] = alpha * s_tA * s_tB * sum_k A_hat[m,k] B_hat[n,k]
 *                         + beta_e * E[M][N]            (E nullable)
 * The block-scaled NT product that every linear and Newton-Schulz product
 * reduces to.  A: view with rows = M, cols = K; B: view with rows = N,
 * cols = K.  C, E fp32 row-major (leading dimension N); C may equal E.
 * Products of the expanded operands are exact and accumulate in fp32.
 */
size_t fs4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
fs4_status fs4_gemm_nt(const fs4_nvfp4 *A, const fs4_nvfp4 *B, float alpha,
                       const float *E, float beta_e, float *C,
                       void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_gemm_plan — introspection, launches nothing: the tile configuration
 * fs4_gemm_nt (and the products of fs4_linear_fwd / fs4_linear_bwd) take for
 * an M x N x K product.  out (host, 4 entries): tile rows, tile columns,
 * tiles, k-splits of the last round's tiles (1: none).
 * Errors: FS4_ERR_NULL (out), FS4_ERR_SHAPE (negative dims, K % 16 != 0).
 */
fs4_status fs4_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t *out);

/* ---------------------------------------------------------------------------
 * fs4_linear_fwd — LoRA-SVD projection forward, [FS4 §2.1]: the weight is
 * W = R + beta U V with U = L2 [N][r], V = L1 [r][K] kept in BF16 and the
 * residual R held in NVFP4:
 *     Y = Q(X) Q(R)^T + beta (X V^T) U^T
 *   X       bf16 [M][K] (M, K multiples of 16)
 *   R_row   NVFP4 view of R: rows = N, cols = K (from fs4_quantize)
 *   U       bf16 [N][r];  V  bf16 [r][K];  0 <= r <= 64 (r = 0: plain NVFP4)
 *   Y       fp32 [M][N]
 *   T_save  fp32 [M][r] receives X V^T (needed by the backward), nullable
 *   X_col_save  column-wise view of X (rows = K, cols = M) for the backward,
 *           nullable; its tscale receives X's tensor scale.
 * The low-rank term uses the unquantized BF16 X.
 */
size_t fs4_linear_fwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int r);
fs4_status fs4_linear_fwd(const void *X, int64_t M, int64_t K, const fs4_nvfp4 *R_row,
                          const void *U, const void *V, int r, float beta,
                          float *Y, float *T_save, const fs4_nvfp4 *X_col_save,
                          void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_linear_bwd — LoRA-SVD projection backward, [FS4 §2.1], each product
 * re-quantized along its own contraction dimension:
 *     dX = Q(dY) Q(R^T)^T + beta (dY U) V     dY blocked along N
 *     dW = Q(dY^T) Q(X^T)^T                   both blocked along M
 *     dU = beta dY^T T,  dV = beta (dY U)^T X
 *   dY      bf16 [M][N]
 *   X       bf16 [M][K]        (for dV; may be NULL when dV is NULL or r = 0)
 *   X_col   column-wise view of X: rows = K, cols = M (from the forward)
 *   R_col   column-wise view of R: rows = K, cols = N (from fs4_quantize)
 *   U, V, r, beta as in the forward;  T fp32 [M][r] = X V^T (forward's T_save)
 *   dX fp32 [M][K];  dW fp32 [N][K] (gradient of the full weight; the update
 *   of the NVFP4 residual);  dU fp32 [N][r], dV fp32 [r][K] (nullable).
 * The pages' Cholesky-QR constraint on the low-rank update is not applied.
 */
size_t fs4_linear_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);
fs4_status fs4_linear_bwd(const void *dY, int64_t M, int64_t N, int64_t K,
                          const void *X, const fs4_nvfp4 *X_col, const fs4_nvfp4 *R_col,
                          const void *U, const void *V, int r, float beta, const float *T,
                          float *dX, float *dW, float *dU, float *dV,
                          void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_newton_schulz — Newton-Schulz orthogonalisation with every GEMM operand
 * in NVFP4, [FS4 §2.3]:
 *     X_0 = G / (||G||_F + eps)          (normalize != 0; else X_0 = G)
 *     repeat `steps` times:
 *       A = Q(X) Q(X)^T;  B = b A + c Q(A) Q(A^T)^T;  X <- a X + Q(B) Q(X^T)^T
 *   G       [m][n], bf16 or fp32 (dt), m <= n, both multiples of 16
 *   X_out   fp32 [m][n]: X_steps
 *   trace_X fp32 [steps+1][m][n]: X_0..X_steps, nullable
 *   trace_A, trace_B fp32 [steps][m][m]: each step's A and B, nullable
 * The Frobenius norm is accumulated in fp64.  steps >= 0.  X_out holds
 * intermediate iterates during the call, so it may not overlap G or a trace
 * buffer (FS4_ERR_ARG).
 * clip_q: 0 for none, else in (0, 1] (FS4_ERR_ARG): the outlier clipping of
 * the Q-Root variant, [FS4 §2.3].  Before each quantization of X, its copy is
 * clipped at p = the nearest-rank clip_q quantile of |X| (as
 * fs4_abs_quantile); the fp32 state, A and B are not clipped.  The pages'
 * shape-dependent (a, b, c) are the caller's (a, b, c).
 */
size_t fs4_newton_schulz_workspace_bytes(int64_t m, int64_t n);
fs4_status fs4_newton_schulz(const void *G, fs4_dtype dt, int64_t m, int64_t n, int steps,
                             float a, float b, float c, int normalize, float eps, double clip_q,
                             float *X_out, float *trace_X, float *trace_A, float *trace_B,
                             void *ws, size_t ws_bytes, void *stream);

/* fs4_ns_shape_coefficients — host only, launches nothing: the quintic
 * coefficients (a, b, c) for an m x n momentum, the shape-dependent
 * coefficients of [FS4 §2.3] (Q-Root) in this reading: they minimise the mean
 * squared distance of `steps` quintic steps to the polar factor (all singular
 * values 1), averaged over the Marchenko-Pastur singular-value law of a
 * Frobenius-normalised m x n Gaussian matrix; found by Nelder-Mead from
 * Muon's (3.4445, -4.7750, 2.0315).  m and n may come in either order.
 *   abc           host float[3] receives (a, b, c), for fs4_newton_schulz
 *   distance_out  host double, nullable: the minimised mean squared distance
 * Errors: FS4_ERR_NULL (abc), FS4_ERR_ARG (m or n < 1, steps outside 1..16).
 * About 0.1 s of host time; callers compute it once per shape.
 */
fs4_status fs4_ns_shape_coefficients(int64_t m, int64_t n, int steps, float *abc, double *distance_out);

/* fs4_newton_schulz_plan — introspection, launches nothing: the tile plans of
 * the three products of one fs4_newton_schulz step on an m x n iterate, in
 * the order A = Q(X) Q(X)^T (m x m x n, symmetric), A^2 (m x m x m,
 * symmetric), and the update, computed transposed (n x m x m).  out (host, 12
 * entries): per product as fs4_gemm_plan's four (symmetric products count the
 * upper triangle's tiles; a split last round has k-splits > 1).
 * Errors: FS4_ERR_NULL, FS4_ERR_SHAPE (as fs4_newton_schulz).
 */
fs4_status fs4_newton_schulz_plan(int64_t m, int64_t n, int64_t *out);

/* ---------------------------------------------------------------------------
 * fs4_abs_quantile — the nearest-rank q-quantile of |x| for the outlier
 * clipping of [FS4 §2.3] (Q-Root, p99): *out = the k-th smallest |x[i]|,
 * k = ceil(q n) computed in fp64 and clamped to [1, n].  Exact: a radix
 * selection over the magnitudes' bit patterns (three passes over x).
 *   x   bf16 or fp32 [n], 1 <= n <= 2^31 (FS4_ERR_SHAPE)
 *   q   in (0, 1] (FS4_ERR_ARG)
 *   out one fp32 on the device (4-byte aligned)
 */
size_t fs4_abs_quantile_workspace_bytes(int64_t n);
fs4_status fs4_abs_quantile(const void *x, fs4_dtype dt, int64_t n, double q, float *out,
                            void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_quantize_clipped — fs4_quantize of clip(x, p), p = the nearest-rank
 * q-quantile of |x| (fs4_abs_quantile): magnitudes above p become p, signs
 * kept, and p is the amax that sets the tensor scale.  Arguments and errors
 * as fs4_quantize, plus q in (0, 1] (FS4_ERR_ARG) and rows * cols <= 2^31.
 */
size_t fs4_quantize_clipped_workspace_bytes(int64_t rows, int64_t cols);
fs4_status fs4_quantize_clipped(const void *x, fs4_dtype dt, int64_t rows, int64_t cols, double q,
                                const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise,
                                void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_lora_project — subspace-constrained gradients of the rank-r branch,
 * [FS4 §2.1] (backward pass: a Cholesky-QR constraint keeps the update of the
 * BF16 branch L2 L1 = U V inside its principal subspace).  With
 * Q_U = CholQR(U) and Q_V = CholQR(V^T), where CholQR(A) = A L^-T for the
 * Cholesky factor L L^T = A^T A:
 *     dU <- Q_U Q_U^T dU          (columns projected onto span(U))
 *     dV <- dV Q_V Q_V^T          (rows projected onto the row space of V)
 * computed in fp64 as U (U^T U)^-1 (U^T dU) and (dV V^T)(V V^T)^-1 V, then
 * rounded to fp32 once.
 *   U  bf16 [N][r], V bf16 [r][K]      the branch's factors
 *   dU fp32 [N][r], dV fp32 [r][K]     their gradients (fs4_linear_bwd's dU
 *       and dV), overwritten in place; either may be NULL to skip that side
 * 0 <= r <= 64 (FS4_ERR_RANK), N >= 0, K >= 0 (FS4_ERR_SHAPE); r = 0 does
 * nothing.  U needs full column rank and V full row rank: where the fp64
 * Cholesky of U^T U (or V V^T) breaks down (a pivot at or below 2^-46 of its
 * diagonal entry), that side's output is all NaN.
 * The residual's gradient (dW of fs4_linear_bwd) is left as it is.
 */
size_t fs4_lora_project_workspace_bytes(int64_t N, int64_t K, int r);
fs4_status fs4_lora_project(const void *U, const void *V, int64_t N, int64_t K, int r,
                            float *dU, float *dV, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_lora_realign — periodic realignment of the rank-r branch with a
 * randomized SVD, [FS4 §2.1] (the subspace is reset every few thousand
 * steps).  With W = beta U V + R:
 *   Y = W Omega^T; q times: Y <- W orth(W^T orth(Y)); Q = orth(Y);
 *   B = Q^T W = sum_i s_i (Q e_i) v_i^T  (the SVD of B, s descending);
 *   U <- bf16(Q e_i sqrt(s_i / beta)), V <- bf16(sqrt(s_i / beta) v_i^T) for
 *   i < r, and R <- fp32(W - beta U V) with those rounded factors,
 * i.e. the randomized range finder of Halko, Martinsson and Tropp with q
 * re-orthonormalised power iterations.
 *   U     bf16 [N][r], in/out         V     bf16 [r][K], in/out
 *   R     fp32 [N][K], in/out: the residual's master copy
 *   Omega fp32 [l][K]: l Gaussian test vectors (drawn by the caller)
 *   sigma fp32 [r], out, nullable: s_0 >= s_1 >= ...
 * 1 <= r <= l <= 64 (FS4_ERR_RANK); N and K positive multiples of 16 with
 * l <= min(N, K) (FS4_ERR_SHAPE); 0 <= power_iters <= 16 and beta > 0
 * (FS4_ERR_ARG).  All sums run in fp64 except the products with W (fp32
 * operands, ~16-bit products, fp32 accumulation), which only shape the basis
 * Q: W = beta U V + R holds afterwards to fp32 rounding whatever Q is.
 */
size_t fs4_lora_realign_workspace_bytes(int64_t N, int64_t K, int l);
fs4_status fs4_lora_realign(void *U, void *V, float *R, int64_t N, int64_t K, int r, float beta,
                            const float *Omega, int l, int power_iters, float *sigma,
                            void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_vstate_encode / fs4_vstate_decode — the Q-AdamW second-moment state
 * codec, [FS4 §2.2]: sqrt, removal of a BF16 tile mean, Hadamard transform,
 * NVFP4; decoding inverts each step and squares.
 *   encode: s = sqrt(v); mu = bf16(mean of s over each 16 x 16 tile);
 *           h = fp32(H/4 (s - mu)) on each 16-element row group (H the
 *           16-point Sylvester Hadamard matrix; H/4 is orthonormal and its own
 *           inverse); q = row-wise NVFP4 of h (one tensor scale).
 *   decode: v_out = fp32((H/4 dequant(q) + mu)^2).
 * Sums run in fp64 in a fixed order (butterflies with strides 1, 2, 4, 8; a
 * tile's sum adds its 16 row-group sums in row order); mu rounds fp64 ->
 * fp32 -> BF16, each to nearest even.
 *   v      fp32 [R][C], non-negative and finite (else unspecified)
 *   q      NVFP4 view, rows = R, cols = C (out of encode, in to decode)
 *   means  bf16 [R/16][C/16]
 *   v_out  fp32 [R][C]
 * R and C positive multiples of 16 (FS4_ERR_SHAPE).  Decode needs no
 * workspace.
 */
size_t fs4_vstate_encode_workspace_bytes(int64_t R, int64_t C);
fs4_status fs4_vstate_encode(const float *v, int64_t R, int64_t C, const fs4_nvfp4 *q, void *means,
                             void *ws, size_t ws_bytes, void *stream);
fs4_status fs4_vstate_decode(const fs4_nvfp4 *q, const void *means, int64_t R, int64_t C, float *v_out,
                             void *stream);

/* ---------------------------------------------------------------------------
 * fs4_mstate_encode / fs4_mstate_decode — the Q-AdamW first-moment state
 * codec, [FS4 §2.2]: Hadamard mixing, then stochastic rounding and adaptive
 * 4/6 block scales.
 *   encode: h = fp32(H/4 m) on each 16-element row group (as for v);
 *           s_t = RNE_fp32(amax(h) / 2688); per block the E4M3 scales for
 *           amax_b / (6 s_t) and amax_b / (4 s_t) are tried and the one whose
 *           round-to-nearest squared error (fp64, summed over the block in
 *           order) is smaller is kept (6 on a tie); every element then rounds
 *           stochastically: y = |h| / (s_b s_t), between E2M1 magnitudes
 *           g_lo <= y < g_hi it takes g_hi exactly when
 *           rnd * 2^-32 < (y - g_lo) / (g_hi - g_lo); y >= 6 gives 6.
 *   decode: m_out = fp32(H/4 dequant(q)).
 *   m      fp32 [R][C], finite
 *   rnd    uint32 [R][C]: one uniform random word per element (the caller
 *          draws them; the same words give the same codes)
 *   q      NVFP4 view, rows = R, cols = C
 * R and C positive multiples of 16 (FS4_ERR_SHAPE).
 */
size_t fs4_mstate_encode_workspace_bytes(int64_t R, int64_t C);
fs4_status fs4_mstate_encode(const float *m, const uint32_t *rnd, int64_t R, int64_t C, const fs4_nvfp4 *q,
                             void *ws, size_t ws_bytes, void *stream);
fs4_status fs4_mstate_decode(const fs4_nvfp4 *q, int64_t R, int64_t C, float *m_out, void *stream);

/* Workspace size for any of the calls above, dispatched on the operation:
 *   FS4_OP_QUANTIZE   d0 = rows, d1 = cols
 *   FS4_OP_GEMM       d0 = M, d1 = N, d2 = K
 *   FS4_OP_LINEAR_FWD d0 = M, d1 = K, d2 = N, r
 *   FS4_OP_LINEAR_BWD d0 = M, d1 = N, d2 = K, r
 *   FS4_OP_NS         d0 = m, d1 = n
 *   FS4_OP_LORA_PROJECT d0 = N, d1 = K, r
 *   FS4_OP_LORA_REALIGN d0 = N, d1 = K, d2 = l
 * Returns 0 for an unknown op. */
typedef enum { FS4_OP_QUANTIZE = 0, FS4_OP_GEMM = 1, FS4_OP_LINEAR_FWD = 2,
               FS4_OP_LINEAR_BWD = 3, FS4_OP_NS = 4, FS4_OP_LORA_PROJECT = 5,
               FS4_OP_LORA_REALIGN = 6 } fs4_op;
size_t fs4_workspace_bytes(fs4_op op, int64_t d0, int64_t d1, int64_t d2, int r);

/* Human-readable name of a status code (static storage). */
const char *fs4_status_str(fs4_status s);

/* Library version string, e.g. "fs4 0.1 gfx950" (static storage). */
const char *fs4_version(void);

/* ---------------------------------------------------------------------------
 * fs4_attention_fwd — NVFP4 mixed-precision attention forward, [FS4 §2.4]
 * (Q-Attn): Q K^T on NVFP4 operands, P V in BF16, per sequence g < G:
 *     S = s_Q s_K Q_hat_g K_hat_g^T / sqrt(D), masked above the diagonal
 *         when causal != 0;  P = softmax(S) by rows;  O_g = P V_g (P rounded
 *         to BF16, V BF16, fp32 accumulation);  LSE_g = log sum_j exp(S_ij)
 *   Q_row, K_row  row-wise NVFP4 views of Q and K as [G*S][D] matrices (blocks
 *                 along D; fs4_quantize of each; the same quantization's
 *                 column-wise views serve the backward's dS products)
 *   V        bf16 [G][S][D]
 *   O        fp32 [G][S][D];  LSE fp32 [G][S], nullable
 *   Vt_save  bf16 [G][D][S], nullable: receives V^T as a side output (the
 *            kernel transposes each V block itself as it stages it)
 *   ws       no workspace is needed (fs4_attention_fwd_workspace_bytes is 0;
 *            ws may be null)
 *   D = 64 or 128; S a positive multiple of 16; G >= 1, G*S < 2^31.
 * Errors: FS4_ERR_SHAPE, FS4_ERR_NULL, FS4_ERR_ALIGN, FS4_ERR_WORKSPACE.
 */
size_t fs4_attention_fwd_workspace_bytes(int64_t G, int64_t S, int64_t D);
fs4_status fs4_attention_fwd(const fs4_nvfp4 *Q_row, const fs4_nvfp4 *K_row, const void *V, int64_t G,
                             int64_t S, int64_t D, int causal, float *O, float *LSE, void *Vt_save,
                             void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * fs4_attention_bwd — the Q-Attn backward, [FS4 §2.4]: the products that
 * take dS on NVFP4 operands, P^T dO and dO V^T in BF16, the forward's
 * quantized Q and K reused.  Per sequence g < G:
 *     P = exp(S - LSE), S recomputed from Q_row, K_row as in the forward
 *     dP = dO V^T,  Delta = rowsum(dO * O),  dS = P * (dP - Delta)   (fp32)
 *     dV = P^T dO                     (P rounded to BF16, dO BF16, fp32 sums)
 *     dQ = s_dS s_K Q(dS) Q_col(K)^T / sqrt(D)
 *     dK = s_dS s_Q Q(dS^T) Q_col(Q)^T / sqrt(D)
 *   where dS is quantized once as the [G*S][S] matrix, one tensor scale over
 *   all sequences: row-wise (blocks along keys) for dQ, column-wise (blocks
 *   along queries) for dK.  Under a causal mask the all-zero blocks of dS
 *   above the diagonal are skipped in dQ and dK (their products are zero).
 *   Q_row, K_row  the forward's row-wise views ([G*S][D], blocks along D)
 *   Q_col, K_col  the column-wise views of the same quantizations ([D][G*S],
 *                 blocks of 16 along the sequence, never across sequences)
 *   V, dO    bf16 [G][S][D];  O fp32 [G][S][D] and LSE fp32 [G][S] from the
 *            forward
 *   dQ, dK, dV  fp32 [G][S][D] outputs
 *   dS       fp32 [G*S][S], nullable: receives the softmax gradient before
 *            its quantization (zeros where masked); without it dS is never
 *            stored in fp32 (the keys are walked twice: dV and the amax of
 *            dS, then dS again, encoded straight into its NVFP4 views)
 *   workspace: fs4_attention_bwd_workspace_bytes(G, S, D) (Delta and dS's
 *   two NVFP4 views, about 1.1 G S^2 bytes), 256-byte aligned.
 *   D = 64 or 128; S a positive multiple of 16; G >= 1, G*S < 2^31 and
 *   G*S*S < 2^31.  All buffers 16-byte aligned (LSE 4).
 * Errors: FS4_ERR_SHAPE, FS4_ERR_NULL, FS4_ERR_ALIGN, FS4_ERR_WORKSPACE (the
 * size call returns 0 for a shape the call rejects).
 */
size_t fs4_attention_bwd_workspace_bytes(int64_t G, int64_t S, int64_t D);
fs4_status fs4_attention_bwd(const fs4_nvfp4 *Q_row, const fs4_nvfp4 *K_row, const fs4_nvfp4 *Q_col,
                             const fs4_nvfp4 *K_col, const void *V, const void *dO, const float *O,
                             const float *LSE, int64_t G, int64_t S, int64_t D, int causal, float *dQ,
                             float *dK, float *dV, float *dS, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* FS4_H */
