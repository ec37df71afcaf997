// Periodic realignment of the LoRA-SVD branch, for gfx950.
//
// Full-Stack FP4 [FS4 §2.1, realignment] resets the BF16 subspace every few
// thousand steps with a randomized SVD.  With W = beta U V + R (R the
// residual's fp32 master copy), l Gaussian test vectors Omega [l][K] and q
// power iterations, the randomized range finder of Halko, Martinsson and
// Tropp gives an orthonormal basis Q [N][l] of (W W^T)^q W Omega^T; then
// B = Q^T W and the top r singular triplets of B replace the branch:
//   U <- bf16(Q e_i sqrt(s_i / beta)),  V <- bf16(sqrt(s_i / beta) v_i^T),
//   R <- fp32(W - beta U V)  (with the rounded factors).
//
// Layout of the computation (Z [K][l] holds B^T = W^T Q throughout):
//   W = R + beta U V                         lowrank_update_kernel
//   Y = W Omega^T                            skinny product (lowrank.hip)
//   q times: Q = orth(Y); Z = W^T Q; Zq = orth(Z); Y = W Zq
//   Q = orth(Y); Z = W^T Q
//   Z^T Z = B B^T = E diag(s^2) E^T          Gram (fp64) + sym_eig_kernel
//   U = Q (E_r diag(sqrt(s / beta))), V^T = Z (E_r diag(1 / sqrt(s beta)))
//   R = W - beta U V                         lowrank_update_kernel
// orth(Y) = Y (Y^T Y)^{-1/2} = Y E diag(lambda^{-1/2}) E^T, from the fp64
// Gram matrix of Y and its eigendecomposition: any orthonormal basis of the
// range serves, since B's SVD absorbs the choice.
//
// The eigensolver is cyclic Jacobi in one workgroup (fp64, n = l <= 64):
// each step rotates n/2 disjoint (p, q) pairs of a round-robin schedule,
// rows first, then columns and the eigenvector matrix, one barrier apart.
#include "fs4_common.h"

namespace fs4 {
namespace {

#define FS4_STATUS_TRY(x)              \
  do {                                 \
    const fs4_status _st = (x);        \
    if (_st != FS4_OK) return _st;     \
  } while (0)

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxL = kMaxRank;

// out[n][k] = base[n][k] + s * sum_j A[n][j] B[j][k]; A bf16 [N][r], B bf16
// [r][K]; base and out fp32 [N][K] (they may be the same buffer); fp64 sums.
// One 64 x 64 tile per workgroup; thread (ty, tx) owns rows ty*4 .. +4 and
// columns tx*4 .. +4 (16-byte loads and stores; K % 16 == 0).
__global__ __launch_bounds__(kThreads) void lowrank_update_kernel(const float *base, float *out,
                                                                  const uint16_t *A, const uint16_t *B,
                                                                  int64_t N, int64_t K, int r,
                                                                  double s) {
  __shared__ double As[kTile][kMaxRank + 1];
  __shared__ double Bs[kMaxRank][kTile + 1];
  const int64_t tiles_k = (K + kTile - 1) / kTile;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_k) * kTile, k0 = (int64_t)(blockIdx.x % tiles_k) * kTile;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  for (int e = t; e < kTile * r; e += kThreads) {
    const int i = e / r, j = e % r;
    As[i][j] = n0 + i < N ? (double)bf16_bits_to_float(A[(n0 + i) * r + j]) : 0.0;
  }
  for (int e = t; e < r * kTile; e += kThreads) {
    const int j = e / kTile, c = e % kTile;
    Bs[j][c] = k0 + c < K ? (double)bf16_bits_to_float(B[(int64_t)j * K + k0 + c]) : 0.0;
  }
  __syncthreads();
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int j = 0; j < r; ++j) {
    double av[4], bv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) av[a] = As[ty * 4 + a][j];
#pragma unroll
    for (int b = 0; b < 4; ++b) bv[b] = Bs[j][tx * 4 + b];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] += av[a] * bv[b];
  }
  const int64_t kk = k0 + tx * 4;
  if (kk >= K) return;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t n = n0 + ty * 4 + a;
    if (n >= N) break;
    const float4 bse = *(const float4 *)(base + n * K + kk);
    float4 o;
    o.x = (float)((double)bse.x + s * acc[a][0]);
    o.y = (float)((double)bse.y + s * acc[a][1]);
    o.z = (float)((double)bse.z + s * acc[a][2]);
    o.w = (float)((double)bse.w + s * acc[a][3]);
    *(float4 *)(out + n * K + kk) = o;
  }
}

// out(n, j) = sum_m X[n][m] C[m][j], X fp32 [L][l], C fp64 [l][J]; out is
// fp32 or BF16 (rounded to nearest even) at out[n * o_sn + j * o_sj].
template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void rmul_kernel(const float *X, const double *C, int64_t L,
                                                        int l, int J, void *out, int64_t o_sn,
                                                        int64_t o_sj) {
  __shared__ double Cs[kMaxL][kMaxL + 1];
  for (int e = threadIdx.x; e < l * J; e += kThreads) Cs[e / J][e % J] = C[e];
  __syncthreads();
  const int64_t total = L * J;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t n = e / J;
    const int j = (int)(e % J);
    const float *x = X + n * l;
    double v = 0.0;
    for (int m = 0; m < l; ++m) v += (double)x[m] * Cs[m][j];
    if constexpr (BF16_OUT)
      ((uint16_t *)out)[n * o_sn + j * o_sj] = (uint16_t)float_to_bf16_rne_bits((float)v);
    else
      ((float *)out)[n * o_sn + j * o_sj] = (float)v;
  }
}

// Symmetric eigendecomposition of the n x n matrix red[i][j] (row stride 2n,
// fp64) by cyclic Jacobi, then
//   mode 0 (orthonormaliser): M[i][j] = sum_m E[i][m] w_m E[j][m],
//          w_m = lambda_m^{-1/2} (0 for lambda_m <= 1e-24 lambda_max)
//   mode 1 (final): for the r largest eigenvalues (descending), s_i =
//          sqrt(lambda_i), Cu[m][i] = E[m][i] sqrt(s_i / beta),
//          Cv[m][i] = E[m][i] / sqrt(s_i beta) (0 where s_i = 0), sigma[i] = s_i
__global__ __launch_bounds__(kThreads) void sym_eig_kernel(const double *red, int n, int mode, int r,
                                                           double beta, double *M, double *Cu,
                                                           double *Cv, float *sigma) {
  __shared__ double A[kMaxL][kMaxL + 1];
  __shared__ double E[kMaxL][kMaxL + 1];
  __shared__ double cs[kMaxL / 2], sn[kMaxL / 2];
  __shared__ int P[kMaxL / 2], Q[kMaxL / 2];
  __shared__ double part[kThreads];
  __shared__ int done;
  __shared__ int perm[kMaxL];
  const int t = threadIdx.x;
  for (int e = t; e < n * n; e += kThreads) {
    const int i = e / n, j = e % n;
    A[i][j] = red[(size_t)i * 2 * n + j];
    E[i][j] = i == j ? 1.0 : 0.0;
  }
  const int m = (n + 1) & ~1;   // players in the round robin; index n is a bye when n is odd
  const int half = m / 2;
  __syncthreads();
  for (int sweep = 0; sweep < 30; ++sweep) {
    // convergence: off-diagonal mass against the diagonal's
    double off = 0.0, dia = 0.0;
    for (int e = t; e < n * n; e += kThreads) {
      const int i = e / n, j = e % n;
      const double v = A[i][j] * A[i][j];
      if (i == j) dia += v;
      else off += v;
    }
    part[t] = off;
    __syncthreads();
    if (t == 0) {
      double so = 0.0;
      for (int i = 0; i < kThreads; ++i) so += part[i];
      part[0] = so;
    }
    __syncthreads();
    const double off_all = part[0];
    __syncthreads();
    part[t] = dia;
    __syncthreads();
    if (t == 0) {
      double sd = 0.0;
      for (int i = 0; i < kThreads; ++i) sd += part[i];
      done = !(off_all > 1e-30 * sd);
    }
    __syncthreads();
    if (done) break;
    for (int step = 0; step < m - 1; ++step) {
      if (t < half) {
        auto who = [&](int pos) { return pos == 0 ? 0 : ((pos - 1 + step) % (m - 1)) + 1; };
        int p = who(t), q = who(m - 1 - t);
        if (p > q) {
          const int x = p;
          p = q;
          q = x;
        }
        double c = 1.0, s = 0.0;
        if (q < n) {
          const double apq = A[p][q];
          if (apq != 0.0) {
            const double theta = (A[q][q] - A[p][p]) / (2.0 * apq);
            const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (__builtin_fabs(theta) + __builtin_sqrt(theta * theta + 1.0));
            c = 1.0 / __builtin_sqrt(tt * tt + 1.0);
            s = tt * c;
          }
        }
        P[t] = p;
        Q[t] = q < n ? q : p;   // a bye pairs p with itself and rotates nothing
        cs[t] = c;
        sn[t] = s;
      }
      __syncthreads();
      // rows p and q of A
      for (int e = t; e < half * n; e += kThreads) {
        const int k = e / n, j = e % n;
        const int p = P[k], q = Q[k];
        if (p == q) continue;
        const double c = cs[k], s = sn[k];
        const double a = A[p][j], b = A[q][j];
        A[p][j] = c * a - s * b;
        A[q][j] = s * a + c * b;
      }
      __syncthreads();
      // columns p and q of A and of E
      for (int e = t; e < half * n; e += kThreads) {
        const int k = e / n, i = e % n;
        const int p = P[k], q = Q[k];
        if (p == q) continue;
        const double c = cs[k], s = sn[k];
        const double a = A[i][p], b = A[i][q];
        A[i][p] = c * a - s * b;
        A[i][q] = s * a + c * b;
        const double ea = E[i][p], eb = E[i][q];
        E[i][p] = c * ea - s * eb;
        E[i][q] = s * ea + c * eb;
      }
      __syncthreads();
    }
  }
  // order by eigenvalue, largest first (ties by index)
  for (int i = t; i < n; i += kThreads) {
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (A[j][j] > A[i][i]) || (A[j][j] == A[i][i] && j < i);
    perm[rank] = i;
  }
  __syncthreads();
  if (mode == 0) {
    const double lmax = A[perm[0]][perm[0]];
    for (int e = t; e < n * n; e += kThreads) {
      const int i = e / n, j = e % n;
      double v = 0.0;
      for (int k = 0; k < n; ++k) {
        const double lam = A[k][k];
        const double w = lam > 1e-24 * lmax ? 1.0 / __builtin_sqrt(lam) : 0.0;
        v += E[i][k] * w * E[j][k];
      }
      M[e] = v;
    }
  } else {
    for (int e = t; e < n * r; e += kThreads) {
      const int k = e / r, i = e % r;
      const int c = perm[i];
      const double lam = A[c][c];
      const double sg = lam > 0.0 ? __builtin_sqrt(lam) : 0.0;
      Cu[e] = E[k][c] * __builtin_sqrt(sg / beta);
      Cv[e] = sg > 0.0 ? E[k][c] / __builtin_sqrt(sg * beta) : 0.0;
      if (k == 0 && sigma) sigma[i] = (float)sg;
    }
  }
}

struct RealignWs {
  float *W, *Y, *Qb, *Z, *Zq, *sg_part;
  double *g_part, *red, *M, *Cu, *Cv;
};
RealignWs carve_realign(void *ws, int64_t N, int64_t K, int l, size_t *total) {
  Carver c(ws);
  RealignWs w;
  w.W = (float *)c.take((size_t)(N * K) * sizeof(float));
  w.Y = (float *)c.take((size_t)(N * l) * sizeof(float));
  w.Qb = (float *)c.take((size_t)(N * l) * sizeof(float));
  w.Z = (float *)c.take((size_t)(K * l) * sizeof(float));
  w.Zq = (float *)c.take((size_t)(K * l) * sizeof(float));
  const size_t p1 = small_gemm_partials_bytes(N, l, K), p2 = small_gemm_partials_bytes(K, l, N);
  w.sg_part = (float *)c.take(p1 > p2 ? p1 : p2);
  const size_t g1 = gram_f32_ws_bytes(N, l), g2 = gram_f32_ws_bytes(K, l);
  w.g_part = (double *)c.take(g1 > g2 ? g1 : g2);
  w.red = (double *)c.take((size_t)l * 2 * l * sizeof(double));
  w.M = (double *)c.take((size_t)l * l * sizeof(double));
  w.Cu = (double *)c.take((size_t)l * l * sizeof(double));
  w.Cv = (double *)c.take((size_t)l * l * sizeof(double));
  if (total) *total = c.off;
  return w;
}

unsigned rmul_blocks(int64_t L, int J) {
  int64_t b = (L * J + kThreads - 1) / kThreads;
  return (unsigned)(b > 4096 ? 4096 : (b < 1 ? 1 : b));
}

}  // namespace

size_t lora_realign_ws_bytes(int64_t N, int64_t K, int l) {
  size_t total = 0;
  carve_realign(nullptr, N, K, l, &total);
  return total;
}

fs4_status launch_lora_realign(uint16_t *U, uint16_t *V, float *R, int64_t N, int64_t K, int r,
                               float beta, const float *Omega, int l, int power_iters, float *sigma,
                               void *ws, hipStream_t s) {
  RealignWs w = carve_realign(ws, N, K, l, nullptr);
  const unsigned tiles = (unsigned)(((N + kTile - 1) / kTile) * ((K + kTile - 1) / kTile));
  // W = R + beta U V
  lowrank_update_kernel<<<tiles, kThreads, 0, s>>>(R, w.W, U, V, N, K, r, (double)beta);
  // the products with W: Y = W X^T for X [l][K] (or K-major when x_kmajor),
  // Z = W^T Y
  auto w_times = [&](const float *X, bool x_kmajor, float *out) {
    return launch_small_gemm(w.W, true, K, 1, X, true, x_kmajor ? 1 : K, x_kmajor ? l : 1, N, l, K,
                             1.0f, out, false, w.sg_part, s);
  };
  auto wt_times = [&](const float *Yn, float *out) {
    return launch_small_gemm(w.W, true, 1, K, Yn, true, 1, l, K, l, N, 1.0f, out, false, w.sg_part, s);
  };
  // orth(X [L][l]) into out: X (X^T X)^{-1/2}
  auto orth = [&](const float *X, int64_t L, float *out) -> fs4_status {
    FS4_STATUS_TRY(launch_gram_f32(X, L, l, w.g_part, w.red, s));
    sym_eig_kernel<<<1, kThreads, 0, s>>>(w.red, l, 0, 0, 1.0, w.M, nullptr, nullptr, nullptr);
    rmul_kernel<false><<<rmul_blocks(L, l), kThreads, 0, s>>>(X, w.M, L, l, l, out, l, 1);
    return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
  };
  FS4_STATUS_TRY(w_times(Omega, false, w.Y));
  for (int it = 0; it < power_iters; ++it) {
    FS4_STATUS_TRY(orth(w.Y, N, w.Qb));
    FS4_STATUS_TRY(wt_times(w.Qb, w.Z));
    FS4_STATUS_TRY(orth(w.Z, K, w.Zq));
    FS4_STATUS_TRY(w_times(w.Zq, true, w.Y));
  }
  FS4_STATUS_TRY(orth(w.Y, N, w.Qb));
  FS4_STATUS_TRY(wt_times(w.Qb, w.Z));
  // Z^T Z = B B^T: its eigenvectors and singular values give the factors
  FS4_STATUS_TRY(launch_gram_f32(w.Z, K, l, w.g_part, w.red, s));
  sym_eig_kernel<<<1, kThreads, 0, s>>>(w.red, l, 1, r, (double)beta, nullptr, w.Cu, w.Cv, sigma);
  rmul_kernel<true><<<rmul_blocks(N, r), kThreads, 0, s>>>(w.Qb, w.Cu, N, l, r, U, r, 1);
  rmul_kernel<true><<<rmul_blocks(K, r), kThreads, 0, s>>>(w.Z, w.Cv, K, l, r, V, 1, K);
  // R = W - beta U V with the new BF16 factors
  lowrank_update_kernel<<<tiles, kThreads, 0, s>>>(w.W, R, U, V, N, K, r, -(double)beta);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
