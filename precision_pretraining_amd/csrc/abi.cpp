// libfs4 C ABI: argument validation and orchestration of the HIP kernels.
// Every check runs on the host before anything is launched.
#include "fs4_common.h"

using namespace fs4;

namespace {

inline hipStream_t as_stream(void *s) { return (hipStream_t)s; }

bool dim_ok(int64_t d) { return d > 0 && d % kBlock == 0; }

fs4_status check_ptr(const void *p) {
  if (!p) return FS4_ERR_NULL;
  if (!aligned16(p)) return FS4_ERR_ALIGN;
  return FS4_OK;
}

#define FS4_TRY(x)                      \
  do {                                  \
    fs4_status _st = (x);               \
    if (_st != FS4_OK) return _st;      \
  } while (0)

// A view used as an input (must be fully valid) or an output of given shape.
fs4_status check_view(const fs4_nvfp4 *v, int64_t rows, int64_t cols) {
  if (!v) return FS4_ERR_NULL;
  if (!v->codes || !v->scales || !v->tscale) return FS4_ERR_NULL;
  if (!aligned16(v->codes) || !aligned16(v->scales) || ((uintptr_t)v->tscale & 3u))
    return FS4_ERR_ALIGN;
  if (v->rows != rows || v->cols != cols) return FS4_ERR_SHAPE;
  if (cols % kBlock) return FS4_ERR_SHAPE;
  return FS4_OK;
}

fs4_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return FS4_ERR_WORKSPACE;
  if (need > 0) {
    if (!ws) return FS4_ERR_NULL;
    if ((uintptr_t)ws & 255u) return FS4_ERR_ALIGN;
  }
  return FS4_OK;
}

// ---- workspace layouts -------------------------------------------------------
struct FwdWs {
  fs4_nvfp4 x_row;
  uint32_t *qws;
  float *T;
  float *partials;
};
FwdWs carve_fwd(void *ws, int64_t M, int64_t K, int r, size_t *total) {
  Carver c(ws);
  FwdWs w;
  w.x_row = carve_view(c, M, K);
  w.qws = (uint32_t *)c.take(quantize_ws_bytes());
  w.T = (float *)c.take((size_t)(M * (r > 0 ? r : 1)) * sizeof(float));
  size_t pb = small_gemm_partials_bytes(M, r > 0 ? r : 1, K);
  const size_t p2 = rowred_partials_bytes(M, r > 0 ? r : 1, K);
  w.partials = (float *)c.take(pb > p2 ? pb : p2);
  if (total) *total = c.off;
  return w;
}

struct BwdWs {
  fs4_nvfp4 dy_row, dy_col;
  uint32_t *qws;
  float *P;
  uint16_t *Ut, *bt;
  float *partials;
};
BwdWs carve_bwd(void *ws, int64_t M, int64_t N, int64_t K, int r, size_t *total) {
  Carver c(ws);
  BwdWs w;
  w.dy_row = carve_view(c, M, N);
  w.dy_col = carve_view(c, N, M);
  w.qws = (uint32_t *)c.take(quantize_ws_bytes());
  const int rr = r > 0 ? r : 1;
  w.P = (float *)c.take((size_t)(M * rr) * sizeof(float));
  w.Ut = (uint16_t *)c.take((size_t)(N * rr) * sizeof(uint16_t));
  w.bt = (uint16_t *)c.take((size_t)(2 * M * rr) * sizeof(uint16_t));
  size_t pb = 0;
  for (size_t b : {small_gemm_partials_bytes(M, rr, N), small_gemm_partials_bytes(N, rr, M),
                   small_gemm_partials_bytes(rr, K, M), rowred_partials_bytes(M, rr, N),
                   colred_partials_bytes(M, N, rr), colred_partials_bytes(M, K, rr),
                   dualred_partials_bytes(M, N, rr)})
    pb = b > pb ? b : pb;
  w.partials = (float *)c.take(pb);
  if (total) *total = c.off;
  return w;
}

struct NsWs {
  float *X, *A, *B;
  fs4_nvfp4 x_row, x_col, a_row, b_row;
  uint32_t *qws;
  void *nws;
  uint32_t *amax;   // per-workgroup max |.| of the tensor about to be quantized
  float *split;     // split-k partials of the GEMMs
  int64_t split_floats;
  void *sel_ws;     // the |x| quantile's histogram and state
  float *clip;      // the clip value of the iterate (clipped runs)
};
NsWs carve_ns(void *ws, int64_t m, int64_t n, size_t *total) {
  Carver c(ws);
  NsWs w;
  w.X = (float *)c.take((size_t)(m * n) * sizeof(float));
  w.A = (float *)c.take((size_t)(m * m) * sizeof(float));
  w.B = (float *)c.take((size_t)(m * m) * sizeof(float));
  w.x_row = carve_view(c, m, n);
  w.x_col = carve_view(c, n, m);
  w.a_row = carve_view(c, m, m);
  w.b_row = carve_view(c, m, m);
  w.qws = (uint32_t *)c.take(quantize_ws_bytes());
  w.nws = c.take(normalize_ws_bytes());
  {
    const int64_t np = std::max<int64_t>(gemm_max_workgroups(m, n), kNormMaxParts);
    w.amax = (uint32_t *)c.take((size_t)np * sizeof(uint32_t));
  }
  {
    // partials of at most 8 splits of tiles no larger than 256 x 256 that
    // cover the output at most once
    const int64_t r256 = (m + 255) / 256 * 256, c256 = (std::max(m, n) + 255) / 256 * 256;
    w.split_floats = std::min<int64_t>(kGemmSplitFloats, 8 * r256 * c256);
    w.split = (float *)c.take((size_t)w.split_floats * sizeof(float));
  }
  w.sel_ws = c.take(abs_quantile_ws_bytes());
  w.clip = (float *)c.take(sizeof(float));
  if (total) *total = c.off;
  return w;
}

bool quantile_ok(double q) { return q > 0.0 && q <= 1.0; }

}  // namespace

extern "C" {

const char *fs4_status_str(fs4_status s) {
  switch (s) {
    case FS4_OK: return "FS4_OK";
    case FS4_ERR_NULL: return "FS4_ERR_NULL: a required pointer is NULL";
    case FS4_ERR_SHAPE: return "FS4_ERR_SHAPE: bad or inconsistent dimension";
    case FS4_ERR_ALIGN: return "FS4_ERR_ALIGN: device pointer not 16-byte aligned";
    case FS4_ERR_DTYPE: return "FS4_ERR_DTYPE: unknown dtype";
    case FS4_ERR_RANK: return "FS4_ERR_RANK: low-rank r out of range or factors missing";
    case FS4_ERR_WORKSPACE: return "FS4_ERR_WORKSPACE: workspace too small";
    case FS4_ERR_HIP: return "FS4_ERR_HIP: kernel launch failed";
    case FS4_ERR_ARG: return "FS4_ERR_ARG: argument out of range";
  }
  return "FS4: unknown status";
}

const char *fs4_version(void) { return "fs4 0.1 gfx950"; }

size_t fs4_quantize_workspace_bytes(int64_t, int64_t) { return quantize_ws_bytes(); }

fs4_status fs4_quantize(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                        const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise, void *ws,
                        size_t ws_bytes, void *stream) {
  FS4_TRY(check_quantize_args(x, dt, rows, cols, rowwise, colwise));
  FS4_TRY(check_ws(ws, ws_bytes, quantize_ws_bytes()));
  return launch_quantize(x, dt, rows, cols, rowwise, colwise, ws, as_stream(stream));
}

}  // extern "C"

namespace fs4 {
fs4_status check_quantize_args(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                               const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise) {
  if (dt != FS4_BF16 && dt != FS4_FP32) return FS4_ERR_DTYPE;
  if (rows < 0 || cols < 0) return FS4_ERR_SHAPE;
  if (!rowwise && !colwise) return FS4_ERR_NULL;
  const bool empty = rows == 0 || cols == 0;
  if (!empty) FS4_TRY(check_ptr(x));
  if (rowwise) {
    if (empty) {
      if (!rowwise->tscale) return FS4_ERR_NULL;
    } else {
      FS4_TRY(check_view(rowwise, rows, cols));
    }
  }
  if (colwise) {
    if (empty) {
      if (!colwise->tscale) return FS4_ERR_NULL;
    } else {
      FS4_TRY(check_view(colwise, cols, rows));
    }
  }
  return FS4_OK;
}
}  // namespace fs4

extern "C" {

size_t fs4_abs_quantile_workspace_bytes(int64_t) { return abs_quantile_ws_bytes(); }

fs4_status fs4_abs_quantile(const void *x, fs4_dtype dt, int64_t n, double q, float *out, void *ws,
                            size_t ws_bytes, void *stream) {
  if (dt != FS4_BF16 && dt != FS4_FP32) return FS4_ERR_DTYPE;
  if (n < 1 || n > ((int64_t)1 << 31)) return FS4_ERR_SHAPE;
  if (!quantile_ok(q)) return FS4_ERR_ARG;
  FS4_TRY(check_ptr(x));
  if (!out) return FS4_ERR_NULL;
  if ((uintptr_t)out & 3u) return FS4_ERR_ALIGN;
  FS4_TRY(check_ws(ws, ws_bytes, abs_quantile_ws_bytes()));
  return launch_abs_quantile(x, dt, n, q, out, ws, as_stream(stream));
}

size_t fs4_quantize_clipped_workspace_bytes(int64_t, int64_t) {
  Carver c(nullptr);
  c.take(quantize_ws_bytes());
  c.take(abs_quantile_ws_bytes());
  c.take(sizeof(float));
  return c.off;
}

fs4_status fs4_quantize_clipped(const void *x, fs4_dtype dt, int64_t rows, int64_t cols, double q,
                                const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise, void *ws,
                                size_t ws_bytes, void *stream) {
  if (!quantile_ok(q)) return FS4_ERR_ARG;
  if (rows * cols > ((int64_t)1 << 31)) return FS4_ERR_SHAPE;
  const size_t need = fs4_quantize_clipped_workspace_bytes(rows, cols);
  if (ws_bytes < need) return FS4_ERR_WORKSPACE;
  if (rows == 0 || cols == 0)   // nothing to clip: the plain call's checks and zero scales
    return fs4_quantize(x, dt, rows, cols, rowwise, colwise, ws, ws_bytes, stream);
  if (dt != FS4_BF16 && dt != FS4_FP32) return FS4_ERR_DTYPE;
  if (rows < 0 || cols < 0) return FS4_ERR_SHAPE;
  if (!rowwise && !colwise) return FS4_ERR_NULL;
  FS4_TRY(check_ptr(x));
  if (rowwise) FS4_TRY(check_view(rowwise, rows, cols));
  if (colwise) FS4_TRY(check_view(colwise, cols, rows));
  FS4_TRY(check_ws(ws, ws_bytes, need));
  Carver c(ws);
  c.take(quantize_ws_bytes());
  void *sel = c.take(abs_quantile_ws_bytes());
  float *clip = (float *)c.take(sizeof(float));
  hipStream_t s = as_stream(stream);
  FS4_TRY(launch_abs_quantile(x, dt, rows * cols, q, clip, sel, s));
  return launch_quantize_encode(x, dt, rows, cols, rowwise, colwise, nullptr, 0, s, clip);
}

size_t fs4_vstate_encode_workspace_bytes(int64_t R, int64_t C) {
  if (!dim_ok(R) || !dim_ok(C)) return 0;
  return vstate_encode_ws_bytes(R, C);
}

fs4_status fs4_vstate_encode(const float *v, int64_t R, int64_t C, const fs4_nvfp4 *q, void *means, void *ws,
                             size_t ws_bytes, void *stream) {
  if (!dim_ok(R) || !dim_ok(C)) return FS4_ERR_SHAPE;
  FS4_TRY(check_ptr(v));
  FS4_TRY(check_view(q, R, C));
  FS4_TRY(check_ptr(means));
  FS4_TRY(check_ws(ws, ws_bytes, vstate_encode_ws_bytes(R, C)));
  return launch_vstate_encode(v, R, C, *q, (uint16_t *)means, ws, as_stream(stream));
}

fs4_status fs4_vstate_decode(const fs4_nvfp4 *q, const void *means, int64_t R, int64_t C, float *v_out,
                             void *stream) {
  if (!dim_ok(R) || !dim_ok(C)) return FS4_ERR_SHAPE;
  FS4_TRY(check_view(q, R, C));
  FS4_TRY(check_ptr(means));
  FS4_TRY(check_ptr(v_out));
  return launch_vstate_decode(*q, (const uint16_t *)means, R, C, v_out, as_stream(stream));
}

size_t fs4_mstate_encode_workspace_bytes(int64_t R, int64_t C) {
  if (!dim_ok(R) || !dim_ok(C)) return 0;
  return mstate_encode_ws_bytes(R, C);
}

fs4_status fs4_mstate_encode(const float *m, const uint32_t *rnd, int64_t R, int64_t C, const fs4_nvfp4 *q,
                             void *ws, size_t ws_bytes, void *stream) {
  if (!dim_ok(R) || !dim_ok(C)) return FS4_ERR_SHAPE;
  FS4_TRY(check_ptr(m));
  FS4_TRY(check_ptr(rnd));
  FS4_TRY(check_view(q, R, C));
  FS4_TRY(check_ws(ws, ws_bytes, mstate_encode_ws_bytes(R, C)));
  return launch_mstate_encode(m, rnd, R, C, *q, ws, as_stream(stream));
}

fs4_status fs4_mstate_decode(const fs4_nvfp4 *q, int64_t R, int64_t C, float *m_out, void *stream) {
  if (!dim_ok(R) || !dim_ok(C)) return FS4_ERR_SHAPE;
  FS4_TRY(check_view(q, R, C));
  FS4_TRY(check_ptr(m_out));
  return launch_mstate_decode(*q, R, C, m_out, as_stream(stream));
}

size_t fs4_gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

fs4_status fs4_gemm_nt(const fs4_nvfp4 *A, const fs4_nvfp4 *B, float alpha, const float *E,
                       float beta_e, float *C, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (!A || !B) return FS4_ERR_NULL;
  if (A->rows < 0 || B->rows < 0 || A->cols < 0) return FS4_ERR_SHAPE;
  if (A->cols != B->cols || A->cols % kBlock) return FS4_ERR_SHAPE;
  FS4_TRY(check_view(A, A->rows, A->cols));
  FS4_TRY(check_view(B, B->rows, B->cols));
  FS4_TRY(check_ptr(C));
  if (E && !aligned16(E)) return FS4_ERR_ALIGN;
  return launch_gemm_nt(*A, *B, alpha, E, beta_e, C, LowRankEpilogue(), as_stream(stream));
}

fs4_status fs4_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t *out) {
  if (!out) return FS4_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || K % kBlock) return FS4_ERR_SHAPE;
  const GemmPlan p = plan_gemm(M, N, K, false, false, 0);
  out[0] = p.bm;
  out[1] = p.bn;
  out[2] = p.tiles;
  out[3] = p.s_tail;
  return FS4_OK;
}

size_t fs4_linear_fwd_workspace_bytes(int64_t M, int64_t K, int64_t, int r) {
  size_t total = 0;
  carve_fwd(nullptr, M, K, r, &total);
  return total;
}

fs4_status fs4_linear_fwd(const void *X, int64_t M, int64_t K, const fs4_nvfp4 *R_row,
                          const void *U, const void *V, int r, float beta, float *Y,
                          float *T_save, const fs4_nvfp4 *X_col_save, void *ws, size_t ws_bytes,
                          void *stream) {
  if (!dim_ok(M) || !dim_ok(K)) return FS4_ERR_SHAPE;
  FS4_TRY(check_ptr(X));
  if (!R_row) return FS4_ERR_NULL;
  const int64_t N = R_row->rows;
  if (N <= 0) return FS4_ERR_SHAPE;
  FS4_TRY(check_view(R_row, N, K));
  if (r < 0 || r > kMaxRank) return FS4_ERR_RANK;
  if (r > 0) {
    if (!U || !V) return FS4_ERR_RANK;
    FS4_TRY(check_ptr(U));
    FS4_TRY(check_ptr(V));
    if (T_save) FS4_TRY(check_ptr(T_save));
  }
  FS4_TRY(check_ptr(Y));
  if (X_col_save) FS4_TRY(check_view(X_col_save, K, M));
  size_t need = 0;
  carve_fwd(nullptr, M, K, r, &need);
  FS4_TRY(check_ws(ws, ws_bytes, need));

  hipStream_t s = as_stream(stream);
  FwdWs w = carve_fwd(ws, M, K, r, nullptr);
  LowRankEpilogue lr;
  if (r > 0) {
    float *T = T_save ? T_save : w.T;
    // T[m][j] = sum_k X[m][k] V[j][k]; this pass reads all of X, so it also
    // yields X's amax partials for the quantizer when they fit
    const int64_t nwg = rowred_workgroups(M, K);
    const bool fuse = nwg <= kAmaxPartials;
    FS4_TRY(launch_rowred((const uint16_t *)X, (const uint16_t *)V, M, r, K, 1.0f, T, w.partials,
                          fuse ? w.qws : nullptr, s));
    if (fuse)
      FS4_TRY(launch_quantize_encode(X, FS4_BF16, M, K, &w.x_row, X_col_save, w.qws, (int)nwg, s));
    else
      FS4_TRY(launch_quantize(X, FS4_BF16, M, K, &w.x_row, X_col_save, w.qws, s));
    lr.L = T;
    lr.R = (const uint16_t *)U;
    lr.r = r;
    lr.r_sn = r;
    lr.r_sj = 1;
    lr.l_scale = beta;
  } else {
    FS4_TRY(launch_quantize(X, FS4_BF16, M, K, &w.x_row, X_col_save, w.qws, s));
  }
  return launch_gemm_nt(w.x_row, *R_row, 1.0f, nullptr, 0.0f, Y, lr, s);
}

size_t fs4_linear_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  size_t total = 0;
  carve_bwd(nullptr, M, N, K, r, &total);
  return total;
}

fs4_status fs4_linear_bwd(const void *dY, int64_t M, int64_t N, int64_t K, const void *X,
                          const fs4_nvfp4 *X_col, const fs4_nvfp4 *R_col, const void *U,
                          const void *V, int r, float beta, const float *T, float *dX, float *dW,
                          float *dU, float *dV, void *ws, size_t ws_bytes, void *stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return FS4_ERR_SHAPE;
  FS4_TRY(check_ptr(dY));
  FS4_TRY(check_view(X_col, K, M));
  FS4_TRY(check_view(R_col, K, N));
  if (r < 0 || r > kMaxRank) return FS4_ERR_RANK;
  if (r > 0) {
    if (!U || !V || !T) return FS4_ERR_RANK;
    FS4_TRY(check_ptr(U));
    FS4_TRY(check_ptr(V));
    FS4_TRY(check_ptr(T));
    if (dU) FS4_TRY(check_ptr(dU));
    if (dV) {
      FS4_TRY(check_ptr(dV));
      FS4_TRY(check_ptr(X));
    }
  }
  FS4_TRY(check_ptr(dX));
  FS4_TRY(check_ptr(dW));
  size_t need = 0;
  carve_bwd(nullptr, M, N, K, r, &need);
  FS4_TRY(check_ws(ws, ws_bytes, need));

  hipStream_t s = as_stream(stream);
  BwdWs w = carve_bwd(ws, M, N, K, r, nullptr);
  LowRankEpilogue lr;
  // dU comes out of the same read of dY as P when r <= 32
  const bool dual = r > 0 && r <= 32 && dU && M * N < ((int64_t)1 << 30) && M * r < ((int64_t)1 << 30);
  if (r > 0) {
    // P[m][j] = sum_n dY[m][n] U[n][j] (U transposed once so both operands
    // run along n); this pass reads all of dY, so it also yields dY's amax
    // partials for the quantizer when they fit.  With dual, the same pass
    // forms dU[n][j] = beta sum_m dY[m][n] T[m][j].
    const int64_t nwg = dual ? dualred_workgroups(M, N) : rowred_workgroups(M, N);
    const bool fuse = nwg <= kAmaxPartials;
    if (dual) {
      // (its last launch leaves P's BF16 split in w.bt for the dV pass)
      FS4_TRY(launch_dualred((const uint16_t *)dY, (const uint16_t *)U, w.Ut, T, M, N, r, 1.0f, w.P, beta, dU,
                             w.partials, w.bt, fuse ? w.qws : nullptr, dV ? w.bt : nullptr, s));
    } else {
      FS4_TRY(launch_transpose_rank((const uint16_t *)U, N, r, w.Ut, s));
      FS4_TRY(launch_rowred((const uint16_t *)dY, w.Ut, M, r, N, 1.0f, w.P, w.partials,
                            fuse ? w.qws : nullptr, s));
    }
    if (fuse)
      FS4_TRY(launch_quantize_encode(dY, FS4_BF16, M, N, &w.dy_row, &w.dy_col, w.qws, (int)nwg, s));
    else
      FS4_TRY(launch_quantize(dY, FS4_BF16, M, N, &w.dy_row, &w.dy_col, w.qws, s));
    lr.L = w.P;
    lr.R = (const uint16_t *)V;   // R(k, j) = V[j][k]
    lr.r = r;
    lr.r_sn = 1;
    lr.r_sj = K;
    lr.l_scale = beta;
  } else {
    FS4_TRY(launch_quantize(dY, FS4_BF16, M, N, &w.dy_row, &w.dy_col, w.qws, s));
  }
  FS4_TRY(launch_gemm_nt(w.dy_row, *R_col, 1.0f, nullptr, 0.0f, dX, lr, s));
  FS4_TRY(launch_gemm_nt(w.dy_col, *X_col, 1.0f, nullptr, 0.0f, dW, LowRankEpilogue(), s));
  // column contractions over the M tokens
  if (r > 0 && dU && !dual) {
    // dU[n][j] = beta sum_m dY[m][n] T[m][j]
    FS4_TRY(launch_colred((const uint16_t *)dY, T, M, N, r, beta, dU, false, w.partials, w.bt, s));
  }
  if (r > 0 && dV) {
    // dV[j][k] = beta sum_m P[m][j] X[m][k]
    FS4_TRY(launch_colred((const uint16_t *)X, w.P, M, K, r, beta, dV, true, w.partials, w.bt, s, dual));
  }
  return FS4_OK;
}

size_t fs4_newton_schulz_workspace_bytes(int64_t m, int64_t n) {
  size_t total = 0;
  carve_ns(nullptr, m, n, &total);
  return total;
}

fs4_status fs4_newton_schulz_plan(int64_t m, int64_t n, int64_t *out) {
  if (!out) return FS4_ERR_NULL;
  if (!dim_ok(m) || !dim_ok(n) || m > n) return FS4_ERR_SHAPE;
  size_t total = 0;
  const NsWs w = carve_ns(nullptr, m, n, &total);
  // the three products as fs4_newton_schulz launches them: A = Q(X) Q(X)^T and
  // A^2 = Q(A) Q(A)^T (symmetric, m x m x n and m x m x m) and the transposed
  // update X'^T = Q_col(X)^T Q_row(B)^T (n x m x m)
  const int64_t shapes[3][3] = {{m, m, n}, {m, m, m}, {n, m, m}};
  for (int i = 0; i < 3; ++i) {
    const GemmPlan p = plan_gemm(shapes[i][0], shapes[i][1], shapes[i][2], i < 2, true, w.split_floats);
    out[4 * i + 0] = p.bm;
    out[4 * i + 1] = p.bn;
    out[4 * i + 2] = p.tiles;
    out[4 * i + 3] = p.s_tail;
  }
  return FS4_OK;
}

fs4_status fs4_newton_schulz(const void *G, fs4_dtype dt, int64_t m, int64_t n, int steps, float a,
                             float b, float c, int normalize, float eps, double clip_q, float *X_out,
                             float *trace_X, float *trace_A, float *trace_B, void *ws,
                             size_t ws_bytes, void *stream) {
  if (dt != FS4_BF16 && dt != FS4_FP32) return FS4_ERR_DTYPE;
  if (!dim_ok(m) || !dim_ok(n) || m > n) return FS4_ERR_SHAPE;
  if (steps < 0) return FS4_ERR_ARG;
  if (clip_q != 0.0 && !quantile_ok(clip_q)) return FS4_ERR_ARG;
  if (clip_q != 0.0 && m * n > ((int64_t)1 << 31)) return FS4_ERR_SHAPE;
  FS4_TRY(check_ptr(G));
  FS4_TRY(check_ptr(X_out));
  if (trace_X) FS4_TRY(check_ptr(trace_X));
  if (trace_A) FS4_TRY(check_ptr(trace_A));
  if (trace_B) FS4_TRY(check_ptr(trace_B));
  size_t need = 0;
  carve_ns(nullptr, m, n, &need);
  FS4_TRY(check_ws(ws, ws_bytes, need));
  // X_out holds iterates during the call: it may overlap neither G nor a
  // trace buffer
  {
    const size_t xb = (size_t)(m * n) * sizeof(float), gb = (size_t)(m * n) * (dt == FS4_BF16 ? 2 : 4);
    auto overlap = [](const void *p, size_t pb, const void *q, size_t qb) {
      const uintptr_t a0 = (uintptr_t)p, b0 = (uintptr_t)q;
      return p && q && a0 < b0 + qb && b0 < a0 + pb;
    };
    if (overlap(X_out, xb, G, gb) ||
        overlap(X_out, xb, trace_X, (size_t)(steps + 1) * xb) ||
        overlap(X_out, xb, trace_A, (size_t)steps * (size_t)(m * m) * sizeof(float)) ||
        overlap(X_out, xb, trace_B, (size_t)steps * (size_t)(m * m) * sizeof(float)))
      return FS4_ERR_ARG;
  }

  hipStream_t s = as_stream(stream);
  NsWs w = carve_ns(ws, m, n, nullptr);
  const int64_t mn = m * n, mm = m * m;
  // The iterate is kept transposed, XT = X^T [n][m].  Quantizing XT gives
  // Q_col(X) as its row-wise view and Q_row(X) as its column-wise view (the
  // same blocks and tensor scale as quantizing X), and the update is computed
  // as X'^T = a X^T + Q_col(X)^T Q_row(B)^T: an n x m output whose tiles fill
  // the chip better than the m x n one.  Iterate k lives in w.X or X_out,
  // alternating so that the last one is in w.X; X_out and each trace_X[k]
  // get it transposed back.
  // Untraced, the last update stores X_steps straight into X_out transposed,
  // so X_{steps-1} must not live there: iterates then alternate so that
  // X_{steps-1} is in w.X.
  const bool direct = steps > 0 && !trace_X;
  auto slot = [&](int k) -> float * { return ((steps - k - (direct ? 1 : 0)) % 2 == 0) ? w.X : X_out; };
  float *cur = slot(0);
  // Each producer (normalisation, GEMM epilogue) leaves per-workgroup amax
  // partials of its output in w.amax, so each quantization is one encode
  // pass.
  int np = 0;
  if (normalize) FS4_TRY(launch_normalize_t(G, dt, m, n, eps, cur, w.nws, s, w.amax, &np));
  else FS4_TRY(launch_transpose_f32(G, dt, m, n, cur, s, w.amax, &np));
  auto quantize = [&](const float *x, int64_t rows, int64_t cols, const fs4_nvfp4 *rv,
                      const fs4_nvfp4 *cv) -> fs4_status {
    if (np > 0) return launch_quantize_encode(x, FS4_FP32, rows, cols, rv, cv, w.amax, np, s);
    return launch_quantize(x, FS4_FP32, rows, cols, rv, cv, w.qws, s);
  };
  auto trace = [&](int k) -> fs4_status {
    return trace_X ? launch_transpose_f32(slot(k), FS4_FP32, n, m, trace_X + (int64_t)k * mn, s) : FS4_OK;
  };
  FS4_TRY(trace(0));
  for (int k = 0; k < steps; ++k) {
    float *A = trace_A ? trace_A + (int64_t)k * mm : w.A;
    float *B = trace_B ? trace_B + (int64_t)k * mm : w.B;
    float *next = slot(k + 1);
    // A = Q(X) Q(X)^T is computed (and stored) exactly symmetric, so its
    // column-wise quantization is its row-wise one bit for bit, and
    // A^2 = Q_row(A) Q_col(A)^T = Q(A) Q(A)^T is symmetric as well.
    if (clip_q != 0.0) {
      // the iterate's quantized copy is clipped at the clip_q quantile of |X|
      FS4_TRY(launch_abs_quantile(cur, FS4_FP32, mn, clip_q, w.clip, w.sel_ws, s));
      FS4_TRY(launch_quantize_encode(cur, FS4_FP32, n, m, &w.x_col, &w.x_row, nullptr, 0, s, w.clip));
    } else {
      FS4_TRY(quantize(cur, n, m, &w.x_col, &w.x_row));
    }
    // Unless traced, A and B keep only their upper triangle's tiles: the
    // quantizer reads those and writes each lower block from its mirror
    // image, and the A^2 product reads its bA term where it stores.
    FS4_TRY(launch_gemm_nt(w.x_row, w.x_row, 1.0f, nullptr, 0.0f, A, LowRankEpilogue(), s, w.amax, &np, true,
                           w.split, w.split_floats, trace_A != nullptr));
    if (trace_A) FS4_TRY(quantize(A, m, m, &w.a_row, nullptr));
    else FS4_TRY(launch_quantize_encode(A, FS4_FP32, m, m, &w.a_row, nullptr, w.amax, np, s, nullptr, true));
    FS4_TRY(launch_gemm_nt(w.a_row, w.a_row, c, A, b, B, LowRankEpilogue(), s, w.amax, &np, true, w.split,
                           w.split_floats, trace_B != nullptr));
    if (trace_B) FS4_TRY(quantize(B, m, m, &w.b_row, nullptr));
    else FS4_TRY(launch_quantize_encode(B, FS4_FP32, m, m, &w.b_row, nullptr, w.amax, np, s, nullptr, true));
    if (direct && k + 1 == steps)
      return launch_gemm_nt(w.x_col, w.b_row, 1.0f, cur, a, nullptr, LowRankEpilogue(), s, nullptr, nullptr, false,
                            nullptr, 0, true, X_out);
    FS4_TRY(launch_gemm_nt(w.x_col, w.b_row, 1.0f, cur, a, next, LowRankEpilogue(), s, w.amax, &np, false,
                           w.split, w.split_floats));
    cur = next;
    FS4_TRY(trace(k + 1));
  }
  return launch_transpose_f32(cur, FS4_FP32, n, m, X_out, s);
}

size_t fs4_lora_project_workspace_bytes(int64_t N, int64_t K, int r) {
  if (N < 0 || K < 0 || r < 0 || r > kMaxRank) return 0;
  return lora_project_ws_bytes(N, K, r);
}

fs4_status fs4_lora_project(const void *U, const void *V, int64_t N, int64_t K, int r, float *dU,
                            float *dV, void *ws, size_t ws_bytes, void *stream) {
  if (r < 0 || r > kMaxRank) return FS4_ERR_RANK;
  if (N < 0 || K < 0) return FS4_ERR_SHAPE;
  if (r == 0) return FS4_OK;
  const bool do_u = dU && N > 0, do_v = dV && K > 0;
  if (do_u) {
    FS4_TRY(check_ptr(dU));
    FS4_TRY(check_ptr(U));
  }
  if (do_v) {
    FS4_TRY(check_ptr(dV));
    FS4_TRY(check_ptr(V));
  }
  if (!do_u && !do_v) return FS4_OK;
  FS4_TRY(check_ws(ws, ws_bytes, lora_project_ws_bytes(N, K, r)));
  return launch_lora_project((const uint16_t *)U, (const uint16_t *)V, N, K, r, do_u ? dU : nullptr,
                             do_v ? dV : nullptr, ws, as_stream(stream));
}

size_t fs4_lora_realign_workspace_bytes(int64_t N, int64_t K, int l) {
  if (!dim_ok(N) || !dim_ok(K) || l < 1 || l > kMaxRank) return 0;
  return lora_realign_ws_bytes(N, K, l);
}

fs4_status fs4_lora_realign(void *U, void *V, float *R, int64_t N, int64_t K, int r, float beta,
                            const float *Omega, int l, int power_iters, float *sigma, void *ws,
                            size_t ws_bytes, void *stream) {
  if (r < 1 || r > kMaxRank || l < r || l > kMaxRank) return FS4_ERR_RANK;
  if (!dim_ok(N) || !dim_ok(K) || l > N || l > K) return FS4_ERR_SHAPE;
  if (power_iters < 0 || power_iters > 16 || !(beta > 0.0f) || !(beta < 3.0e38f)) return FS4_ERR_ARG;
  FS4_TRY(check_ptr(U));
  FS4_TRY(check_ptr(V));
  FS4_TRY(check_ptr(R));
  FS4_TRY(check_ptr(Omega));
  if (sigma && ((uintptr_t)sigma & 3u)) return FS4_ERR_ALIGN;
  FS4_TRY(check_ws(ws, ws_bytes, lora_realign_ws_bytes(N, K, l)));
  return launch_lora_realign((uint16_t *)U, (uint16_t *)V, R, N, K, r, beta, Omega, l, power_iters,
                             sigma, ws, as_stream(stream));
}

size_t fs4_attention_fwd_workspace_bytes(int64_t G, int64_t S, int64_t D) {
  if (G < 1 || !dim_ok(S) || (D != 64 && D != 128)) return 0;
  return attention_fwd_ws_bytes(G, S, D);
}

fs4_status fs4_attention_fwd(const fs4_nvfp4 *Q_row, const fs4_nvfp4 *K_row, const void *V, int64_t G, int64_t S,
                             int64_t D, int causal, float *O, float *LSE, void *Vt_save, void *ws, size_t ws_bytes,
                             void *stream) {
  if (G < 1 || !dim_ok(S)) return FS4_ERR_SHAPE;
  if (D != 64 && D != 128) return FS4_ERR_SHAPE;
  if (G > ((int64_t)1 << 31) / S) return FS4_ERR_SHAPE;   // G*S rows index 32-bit grids
  FS4_TRY(check_view(Q_row, G * S, D));
  FS4_TRY(check_view(K_row, G * S, D));
  FS4_TRY(check_ptr(V));
  FS4_TRY(check_ptr(O));
  if (LSE && ((uintptr_t)LSE & 3u)) return FS4_ERR_ALIGN;
  if (Vt_save) FS4_TRY(check_ptr(Vt_save));
  FS4_TRY(check_ws(ws, ws_bytes, attention_fwd_ws_bytes(G, S, D)));
  return launch_attention_fwd(*Q_row, *K_row, (const uint16_t *)V, G, S, D, causal != 0, O, LSE,
                              (uint16_t *)Vt_save, as_stream(stream));
}

size_t fs4_attention_bwd_workspace_bytes(int64_t G, int64_t S, int64_t D) {
  if (G < 1 || !dim_ok(S) || (D != 64 && D != 128)) return 0;
  if (G > ((int64_t)1 << 31) / S || G * S > (((int64_t)1 << 31) - 1) / S) return 0;
  return attention_bwd_ws_bytes(G, S, D);
}

fs4_status fs4_attention_bwd(const fs4_nvfp4 *Q_row, const fs4_nvfp4 *K_row, const fs4_nvfp4 *Q_col,
                             const fs4_nvfp4 *K_col, const void *V, const void *dO, const float *O,
                             const float *LSE, int64_t G, int64_t S, int64_t D, int causal, float *dQ, float *dK,
                             float *dV, float *dS, void *ws, size_t ws_bytes, void *stream) {
  if (G < 1 || !dim_ok(S)) return FS4_ERR_SHAPE;
  if (D != 64 && D != 128) return FS4_ERR_SHAPE;
  if (G > ((int64_t)1 << 31) / S) return FS4_ERR_SHAPE;                  // G*S rows index 32-bit grids
  if (G * S > (((int64_t)1 << 31) - 1) / S) return FS4_ERR_SHAPE;        // dS's G*S*S elements
  FS4_TRY(check_view(Q_row, G * S, D));
  FS4_TRY(check_view(K_row, G * S, D));
  FS4_TRY(check_view(Q_col, D, G * S));
  FS4_TRY(check_view(K_col, D, G * S));
  FS4_TRY(check_ptr(V));
  FS4_TRY(check_ptr(dO));
  FS4_TRY(check_ptr(O));
  FS4_TRY(check_ptr(dQ));
  FS4_TRY(check_ptr(dK));
  FS4_TRY(check_ptr(dV));
  if (!LSE) return FS4_ERR_NULL;
  if ((uintptr_t)LSE & 3u) return FS4_ERR_ALIGN;
  if (dS) FS4_TRY(check_ptr(dS));
  FS4_TRY(check_ws(ws, ws_bytes, attention_bwd_ws_bytes(G, S, D)));
  Carver c(ws);
  const AttnBwdWs w = attention_bwd_carve(c, G, S, D);
  return launch_attention_bwd(*Q_row, *K_row, *Q_col, *K_col, (const uint16_t *)V, (const uint16_t *)dO, O, LSE,
                              G, S, D, causal != 0, dQ, dK, dV, dS, w, as_stream(stream));
}

size_t fs4_workspace_bytes(fs4_op op, int64_t d0, int64_t d1, int64_t d2, int r) {
  switch (op) {
    case FS4_OP_QUANTIZE: return fs4_quantize_workspace_bytes(d0, d1);
    case FS4_OP_GEMM: return fs4_gemm_workspace_bytes(d0, d1, d2);
    case FS4_OP_LINEAR_FWD: return fs4_linear_fwd_workspace_bytes(d0, d1, d2, r);
    case FS4_OP_LINEAR_BWD: return fs4_linear_bwd_workspace_bytes(d0, d1, d2, r);
    case FS4_OP_NS: return fs4_newton_schulz_workspace_bytes(d0, d1);
    case FS4_OP_LORA_PROJECT: return fs4_lora_project_workspace_bytes(d0, d1, r);
    case FS4_OP_LORA_REALIGN: return fs4_lora_realign_workspace_bytes(d0, d1, (int)d2);
  }
  return 0;
}

}  // extern "C"
