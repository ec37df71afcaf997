// Internal helpers shared by the libfs4 kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fs4.h"

namespace fs4 {

constexpr int kBlock = 16;              // elements per E4M3 block scale
constexpr double kTensorDiv = 2688.0;   // 6 (largest E2M1) * 448 (largest E4M3)
constexpr int kMaxRank = 64;

// ----------------------------------------------------------------------------
// E4M3FN decode: exponent field 0 is subnormal (m * 2^-9), else
// 2^(e-7) * (1 + m/8).  Only the finite codes 0..0x7E occur as block scales.
__device__ __host__ inline float e4m3_to_float(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 0xFu, m = byte & 7u;
  if (e == 0) return (float)m * 0.001953125f;            // m * 2^-9, exact
  return __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
}

// Round-to-nearest-even of q >= 0 onto the finite E4M3FN values, values from
// 448 up saturating to 448 (code 0x7E).  q is an fp64 value whose side of
// every E4M3 midpoint is the exact one (see the quantizer).
__device__ inline uint32_t e4m3_rne_satfinite(double q) {
  if (q >= 448.0) return 0x7Eu;
  if (q < 0.015625) {                                    // below 2^-6: subnormal grid 2^-9
    return (uint32_t)__builtin_rint(q * 512.0);          // 0..8; 8 is 2^-6 (code 0x08)
  }
  int e;
  const double mant = __builtin_frexp(q, &e);            // q = mant * 2^e, mant in [0.5, 1)
  // q = 2^(e-1) * (2 mant), 2 mant in [1, 2); mantissa field = round((2 mant - 1) * 8)
  uint32_t m = (uint32_t)__builtin_rint((2.0 * mant - 1.0) * 8.0);
  int eb = e - 1 + 7;                                    // biased exponent, 1..15
  if (m == 8u) { m = 0u; ++eb; }
  uint32_t code = ((uint32_t)eb << 3) | m;
  return code > 0x7Eu ? 0x7Eu : code;
}

// fp64 -> fp32 with directed rounding (x > 0 finite, within fp32 range).
// The nearest-even conversion is off by at most one fp32 step, and for
// non-negative floats the next representable value is the next bit pattern.
__device__ inline float f32_round_up(double x) {
  float f = (float)x;
  if ((double)f < x) f = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) + 1u);
  return f;
}
__device__ inline float f32_round_down(double x) {
  float f = (float)x;
  if ((double)f > x) f = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) - 1u);
  return f;
}

// bf16 raw bits <-> fp32
__device__ inline float bf16_bits_to_float(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
__device__ inline uint32_t float_to_bf16_rne_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ----------------------------------------------------------------------------
// Host-side helpers
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Carves 256-byte aligned sub-buffers out of a workspace (or just sizes them
// when base == nullptr).
struct Carver {
  uint8_t *base;
  size_t off = 0;
  explicit Carver(void *b) : base((uint8_t *)b) {}
  void *take(size_t bytes) {
    void *p = base ? base + off : nullptr;
    off += round_up(bytes ? bytes : 1, 256);
    return p;
  }
};

// An NVFP4 view living in a workspace.
inline fs4_nvfp4 carve_view(Carver &c, int64_t rows, int64_t cols) {
  fs4_nvfp4 v;
  v.rows = rows;
  v.cols = cols;
  v.codes = (uint8_t *)c.take((size_t)(rows * cols / 2));
  v.scales = (uint8_t *)c.take((size_t)(rows * cols / kBlock));
  v.tscale = (float *)c.take(sizeof(float));
  return v;
}

// ----------------------------------------------------------------------------
// Launchers (defined in the .hip files)
constexpr int kAmaxPartials = 1024;      // max partial maxima written by the amax pass
size_t quantize_ws_bytes();
// fs4_quantize's argument checks (everything but the workspace), host only
fs4_status check_quantize_args(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                               const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise);
fs4_status launch_quantize(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                           const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise,
                           void *ws, hipStream_t s);
// The encode pass alone, for a caller whose earlier kernel already wrote npart
// (npart >= 1) partial maxima of |x| (fp32 bits) that cover all of x.  With
// clip (a device scalar p >= 0), x is clipped to magnitude p first and p is
// its amax (the partials are not read).  upper_only: x is square and
// symmetric and only its 64 x 64 tiles on or above the diagonal hold values
// (the others are not read); the row-wise view alone is produced, the lower
// tiles' blocks from their mirror images (identical values, so identical
// codes).
fs4_status launch_quantize_encode(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                                  const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise,
                                  const uint32_t *partials, int npart, hipStream_t s,
                                  const float *clip = nullptr, bool upper_only = false);
// *out = the k-th smallest |x| of x[0..n) (bf16 or fp32), k = ceil(q n) in
// fp64 clamped to [1, n], by exact radix selection; ws needs
// abs_quantile_ws_bytes().  n >= 1.
size_t abs_quantile_ws_bytes();
// Q-AdamW second-moment codec: v fp32 [R][C] -> NVFP4 view q of h and BF16
// tile means [R/16][C/16]; decode back to fp32 (R, C multiples of 16)
size_t vstate_encode_ws_bytes(int64_t R, int64_t C);
fs4_status launch_vstate_encode(const float *v, int64_t R, int64_t C, const fs4_nvfp4 &q,
                                uint16_t *means, void *ws, hipStream_t s);
fs4_status launch_vstate_decode(const fs4_nvfp4 &q, const uint16_t *means, int64_t R, int64_t C, float *out,
                                hipStream_t s);
// Q-AdamW first-moment codec: m fp32 [R][C] with one uint32 random word per
// element -> NVFP4 view q (stochastic rounding, adaptive 4/6 scales); decode
size_t mstate_encode_ws_bytes(int64_t R, int64_t C);
fs4_status launch_mstate_encode(const float *m, const uint32_t *rnd, int64_t R, int64_t C, const fs4_nvfp4 &q,
                                void *ws, hipStream_t s);
fs4_status launch_mstate_decode(const fs4_nvfp4 &q, int64_t R, int64_t C, float *out, hipStream_t s);
fs4_status launch_abs_quantile(const void *x, fs4_dtype dt, int64_t n, double q, float *out, void *ws,
                               hipStream_t s);

// NVFP4 mixed-precision attention forward: Q, K row-wise views of [G*S, D],
// V bf16 [G][S][D]; Vt (nullable) receives V^T [G][D][S] as a side output;
// no workspace (attention_fwd_ws_bytes is 0)
size_t attention_fwd_ws_bytes(int64_t G, int64_t S, int64_t D);
fs4_status launch_attention_fwd(const fs4_nvfp4 &Q, const fs4_nvfp4 &K, const uint16_t *V, int64_t G, int64_t S,
                                int64_t D, int causal, float *O, float *LSE, uint16_t *Vt, hipStream_t s);

// Its backward.  Workspace: Delta, one amax partial per softmax-gradient
// workgroup and dS's two NVFP4 views (row-wise [G*S][S], column-wise
// [S][G*S]).
struct AttnBwdWs {
  float *delta;
  uint32_t *amax;
  int64_t nwg;
  fs4_nvfp4 ds_row, ds_col;
};
AttnBwdWs attention_bwd_carve(Carver &c, int64_t G, int64_t S, int64_t D);
size_t attention_bwd_ws_bytes(int64_t G, int64_t S, int64_t D);
fs4_status launch_attention_bwd(const fs4_nvfp4 &Qr, const fs4_nvfp4 &Kr, const fs4_nvfp4 &Qc,
                                const fs4_nvfp4 &Kc, const uint16_t *V, const uint16_t *dO, const float *O,
                                const float *LSE, int64_t G, int64_t S, int64_t D, int causal, float *dQ,
                                float *dK, float *dV, float *dS, const AttnBwdWs &w, hipStream_t s);

struct LowRankEpilogue {
  const float *L = nullptr;     // fp32 [M][r], scaled by l_scale before use
  const uint16_t *R = nullptr;  // bf16, element (n, j) at R[n * r_sn + j * r_sj]
  int r = 0;
  int64_t r_sn = 0, r_sj = 1;
  float l_scale = 1.0f;
};
// The launcher's choice for an M x N x K product: tile configuration (0:
// 256 x 256, 1: 256 x 192, 2: 128 x 128), the tile count, the tiles that run
// whole and the k-splits of the rest; sym and can_split as for the launch
// (can_split: a split workspace is given and there is no rank-r term).
struct GemmPlan {
  int cfg, bm, bn;
  int64_t tiles, t_full;
  int s_tail;
  double cost;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool sym, bool can_split, int64_t split_floats);
// amax_parts (nullable) receives one max |C| per output tile (fp32 bits, the
// form launch_quantize_encode reduces); *nwg (nullable) their count, which is
// at most gemm_max_workgroups(M, N).  sym: B is the same view as A, there is
// no rank-r term and E, if any, is symmetric, so C is symmetric: only the
// upper triangle's tiles are computed, each stored at both positions (the
// flag is ignored when A and B differ).  split_ws (nullable, split_floats
// floats, at least kGemmSplitFloats to allow every split) lets the tiles of a
// part-filled last round run split along k (fp32 partials, then a reduce
// launch); without it, or with a rank-r term, tiles run whole.
fs4_status launch_gemm_nt(const fs4_nvfp4 &A, const fs4_nvfp4 &B, float alpha, const float *E,
                          float beta_e, float *C, const LowRankEpilogue &lr, hipStream_t s,
                          uint32_t *amax_parts = nullptr, int *nwg = nullptr, bool sym = false,
                          float *split_ws = nullptr, int64_t split_floats = 0, bool mirror = true,
                          float *Ct = nullptr);
// (mirror = false with sym: the tiles below the diagonal are not stored; C
// holds the upper triangle's tiles only.  Ct, for a product that is not
// symmetric and has M % 4 == 0: C is stored transposed there, Ct[n][m], and
// not at C; the tiles run whole.)
// one round of 256 workgroups of split partials, 256 x 256 floats each
constexpr int64_t kGemmSplitFloats = int64_t(256) * 256 * 256;
inline int64_t gemm_max_workgroups(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128); }

// out[a][b] = scale * sum_k P(a, k) Q(b, k) with P(a, k) = P[a*p_sa + k*p_sk],
// Q(b, k) = Q[b*q_sb + k*q_sk]; each operand bf16 or fp32 (p_f32 / q_f32);
// Kc a multiple of 16.  Written row-major [Na][Nb], or [Nb][Na] when
// transpose_out.  `partials` needs small_gemm_partials_bytes(Na, Nb, Kc).
// With amax_parts, the kernel also writes one partial maximum of |P| per
// workgroup (small_gemm_workgroups of them, which together cover all of P).
size_t small_gemm_partials_bytes(int64_t Na, int64_t Nb, int64_t Kc);
int64_t small_gemm_workgroups(int64_t Na, int64_t Nb, int64_t Kc);
fs4_status launch_small_gemm(const void *P, bool p_f32, int64_t p_sa, int64_t p_sk, const void *Q,
                             bool q_f32, int64_t q_sb, int64_t q_sk, int64_t Na, int64_t Nb,
                             int64_t Kc, float scale, float *out, bool transpose_out,
                             float *partials, hipStream_t s, uint32_t *amax_parts = nullptr);
// Skinny rank-r products (r <= 64), bandwidth-shaped:
//   rowred: out[a][j] = scale * sum_k A[a][k] B[j][k], A bf16 [Na][K], B bf16
//           [r][K] (K % 16 == 0, 16-byte aligned rows); optional amax
//           partials of A (rowred_workgroups of them).
//   colred: out[c][j] = scale * sum_m A[m][c] Bm[m][j], A bf16 [M][C] (C % 8
//           == 0, M % 8 == 0), Bm fp32 [M][r]; written [C][r] or, with
//           transpose_out, [r][C].  `bt` is scratch for 2 * M * r BF16.
size_t rowred_partials_bytes(int64_t Na, int r, int64_t K);
int64_t rowred_workgroups(int64_t Na, int64_t K);
fs4_status launch_rowred(const uint16_t *A, const uint16_t *B, int64_t Na, int r, int64_t K,
                         float scale, float *out, float *partials, uint32_t *amax_parts,
                         hipStream_t s);
size_t colred_partials_bytes(int64_t M, int64_t C, int r);
fs4_status launch_colred(const uint16_t *A, const float *Bm, int64_t M, int64_t C, int r,
                         float scale, float *out, bool transpose_out, float *partials,
                         uint16_t *bt, hipStream_t s, bool presplit = false);
//           (presplit: bt already holds Bm's split, as launch_dualred's
//           p_split leaves it; Bm is not read)
//   dualred: both of A's rank-r contractions in one read of A bf16 [M][N]
//           (r <= 32; M, N % 8 == 0; M N, M r < 2^30): P[m][j] = p_scale sum_n A[m][n] U[n][j]
//           with U bf16 [N][r] (transposed into Ut, N r BF16 of scratch),
//           and Q[n][j] = q_scale sum_m A[m][n] Bm[m][j] with Bm fp32 [M][r];
//           `partials` needs dualred_partials_bytes, `bt` 2 * M * r BF16;
//           optional amax partials of A (dualred_workgroups of them);
//           p_split (nullable, 2 * M * r BF16, may be bt) receives P's
//           transposed BF16 hi/lo split for launch_colred(presplit).
size_t dualred_partials_bytes(int64_t M, int64_t N, int r);
int64_t dualred_workgroups(int64_t M, int64_t N);
fs4_status launch_dualred(const uint16_t *A, const uint16_t *U, uint16_t *Ut, const float *Bm, int64_t M,
                          int64_t N, int r, float p_scale, float *P, float q_scale, float *Q,
                          float *partials, uint16_t *bt, uint32_t *amax_parts, uint16_t *p_split,
                          hipStream_t s);
fs4_status launch_transpose_rank(const uint16_t *U, int64_t N, int r, uint16_t *Ut, hipStream_t s);
// Frobenius normalisation X = G / (||G||_F + eps), fp64 accumulation
size_t normalize_ws_bytes();
// XT = (G / (||G||_F + eps))^T in fp32, G [rows][cols] bf16 or fp32 and XT
// [cols][rows] (rows and cols multiples of 16); amax_parts (nullable)
// receives one max |XT| per workgroup, *nparts (nullable) their count (at
// most kNormMaxParts; 0 without amax_parts).
fs4_status launch_normalize_t(const void *G, fs4_dtype dt, int64_t rows, int64_t cols, float eps,
                              float *XT, void *ws, hipStream_t s, uint32_t *amax_parts = nullptr,
                              int *nparts = nullptr);
constexpr int kNormMaxParts = 2048;
// dst [cols][rows] = src [rows][cols] as fp32, the same shape rules and
// partials as launch_normalize_t.
fs4_status launch_transpose_f32(const void *src, fs4_dtype dt, int64_t rows, int64_t cols, float *dst,
                                hipStream_t s, uint32_t *amax_parts = nullptr, int *nparts = nullptr);

// Subspace projection of the rank-r gradients (dU, dV in place; either
// nullable), fp64 Gram matrices, Cholesky and solves; `ws` needs
// lora_project_ws_bytes(N, K, r).
size_t lora_project_ws_bytes(int64_t N, int64_t K, int r);
// red [l][2l] = [A^T A | A^T A] in fp64 for A fp32 [L][l] (l <= 64);
// `part` needs gram_f32_ws_bytes(L, l)
size_t gram_f32_ws_bytes(int64_t L, int l);
fs4_status launch_gram_f32(const float *A, int64_t L, int l, double *part, double *red, hipStream_t s);
// Randomized-SVD realignment of W = beta U V + R (U, V and R updated in
// place); `ws` needs lora_realign_ws_bytes(N, K, l)
size_t lora_realign_ws_bytes(int64_t N, int64_t K, int l);
fs4_status launch_lora_realign(uint16_t *U, uint16_t *V, float *R, int64_t N, int64_t K, int r,
                               float beta, const float *Omega, int l, int power_iters, float *sigma,
                               void *ws, hipStream_t s);
fs4_status launch_lora_project(const uint16_t *U, const uint16_t *V, int64_t N, int64_t K, int r,
                               float *dU, float *dV, void *ws, hipStream_t s);

}  // namespace fs4
