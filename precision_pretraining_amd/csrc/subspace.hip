// Subspace-constrained low-rank gradients of the LoRA-SVD projection, for
// gfx950.
//
// Full-Stack FP4 [FS4 §2.1, backward pass] holds the update of the BF16
// branch L2 L1 = U V to its principal subspace with a Cholesky-QR
// constraint.  With Q_U = CholQR(U) and Q_V = CholQR(V^T) (S = A^T A = L L^T,
// Q = A L^{-T}) the constrained gradients are the orthogonal projections
//
//   dU <- Q_U Q_U^T dU = U (U^T U)^{-1} (U^T dU)
//   dV <- dV Q_V Q_V^T = (dV V^T) (V V^T)^{-1} V
//
// computed here in the second form, which needs only the r x r Gram
// matrices and their Cholesky factors, never Q itself.
//
// Both sides have the same shape once written over "samples": for U the
// samples are the N rows (a(n, i) = U[n][i], g(n, j) = dU[n][j]); for V the
// K columns (a(k, i) = V[i][k], g(k, j) = dV[j][k]).  Then
//   S = sum_s a(s) a(s)^T,  M = sum_s a(s) g(s)^T   (r x r each)
//   Z = S^{-1} M
//   g(s, j) <- sum_i a(s, i) Z[i][j]
// Four launches, each covering the active sides through blockIdx.y (or x):
//   1. partial sums of [S | M] over chunks of samples (fp64),
//   2. their reduction, one thread per entry, in a fixed order,
//   3. one workgroup per side: Z = S^{-1} M by Gauss-Jordan elimination of
//      [S | M] without pivoting (S is symmetric positive definite, so its
//      pivots are the squared diagonal of the Cholesky factor of S, and a
//      pivot breaks down exactly where the Cholesky factorisation would),
//      one barrier per column,
//   4. the update of g in place (reads a and Z only).
// Everything accumulates in fp64 (the BF16 and fp32 inputs are exact there);
// g is rounded to fp32 once.  A Gram matrix whose Cholesky factorisation
// breaks down in fp64 (a pivot at or below 2^-46 of its original diagonal
// entry) makes Z, and so that side's output, NaN.
#include "fs4_common.h"

namespace fs4 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;        // samples staged in LDS per pass
constexpr int kMaxGroups = 256;   // partial-sum workgroups per side

struct Side {
  const uint16_t *A;    // bf16: a(s, i) = A[s * a_ss + i * a_si] (or fp32 from Af)
  int64_t a_ss, a_si;
  float *G;             // fp32: g(s, j) = G[s * g_ss + j * g_si], updated in place
  int64_t g_ss, g_si;
  int64_t L;            // samples
  int groups;           // partial-sum workgroups
  double *part;         // [groups][r][2r]
  double *red;          // [r][2r]: [S | M]
  double *Z;            // [r][r]
  const float *Af;      // when set, a(s, i) = Af[s * a_ss + i * a_si] in fp32
};
struct Sides {
  Side s[2];
  int r;
};

// Ownership of the r x 2r matrix [S | M]: thread t owns column j = t % 2r
// and rows i = g + G k (k < NQ), with G = floor(256 / 2r) row groups and
// g = t / 2r; threads past G * 2r and rows past r own nothing real.  NQ is
// the power of two >= ceil(r / G) (1 .. 32).  Entries that do not exist
// compute on in-range stand-in operands and are never stored, so the inner
// loops carry no per-entry branches.
struct Own {
  int G, g, j;
  bool active;
  __device__ Own(int r) {
    const int r2 = 2 * r;
    G = kThreads / r2;
    g = (int)threadIdx.x / r2;
    j = (int)threadIdx.x % r2;
    active = g < G;
  }
};
inline int nq_for(int r) {
  const int G = kThreads / (2 * r);
  const int need = (r + G - 1) / G;
  int nq = 1;
  while (nq < need) nq *= 2;
  return nq;
}

// 1. part[w][i][j] = sum over this workgroup's samples of a(s, i) w(s, j),
//    w(s, j) = a(s, j) for j < r and g(s, j - r) for j >= r
template <int NQ>
__global__ __launch_bounds__(kThreads) void gram_partial_kernel(Sides args) {
  const Side sd = args.s[blockIdx.y];
  // the grid spans the larger side; the other side's surplus workgroups have
  // no partial slot (uniform per workgroup, before any barrier)
  if ((int)blockIdx.x >= sd.groups) return;
  const int r = args.r, r2 = 2 * r, t = threadIdx.x;
  constexpr int kRow = 2 * kMaxRank + 1;   // a(s, 0..r-1), then g(s, 0..r-1)
  __shared__ double st[kChunk * kRow];
  const Own ow(r);
  const int jj = ow.active ? ow.j : 0;
  int ia[NQ];
  double acc[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int i = ow.g + ow.G * k;
    ia[k] = i < r ? i : 0;
    acc[k] = 0.0;
  }
  // the dimension that is contiguous in memory walks fastest over the lanes
  const bool s_fast = sd.a_ss == 1;
  for (int64_t c0 = (int64_t)blockIdx.x * kChunk; c0 < sd.L; c0 += (int64_t)sd.groups * kChunk) {
    for (int e = t; e < kChunk * r; e += kThreads) {
      const int s = s_fast ? e % kChunk : e / r, i = s_fast ? e / kChunk : e % r;
      const int64_t gs = c0 + s;
      const bool in = gs < sd.L;
      const int64_t ai = gs * sd.a_ss + i * sd.a_si;
      st[s * kRow + i] = in ? (sd.Af ? (double)sd.Af[ai] : (double)bf16_bits_to_float(sd.A[ai])) : 0.0;
      st[s * kRow + r + i] = in ? (double)sd.G[gs * sd.g_ss + i * sd.g_si] : 0.0;
    }
    __syncthreads();
    for (int s = 0; s < kChunk; ++s) {
      const double *row = st + s * kRow;
      const double w = row[jj];
#pragma unroll
      for (int k = 0; k < NQ; ++k) acc[k] += row[ia[k]] * w;
    }
    __syncthreads();
  }
  if (!ow.active) return;
  double *out = sd.part + (size_t)blockIdx.x * r * r2;
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int i = ow.g + ow.G * k;
    if (i < r) out[i * r2 + ow.j] = acc[k];
  }
}

// 2. red[o] = sum over workgroups w of part[w][o], one thread per entry:
//    16 running sums over w mod 16 (independent loads in flight), added in a
//    fixed order
__global__ __launch_bounds__(kThreads) void gram_reduce_kernel(Sides args) {
  const Side sd = args.s[blockIdx.y];
  const int nout = 2 * args.r * args.r;
  const int o = blockIdx.x * kThreads + threadIdx.x;
  if (o >= nout) return;
  double acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = 0.0;
  int w = 0;
  for (; w + 16 <= sd.groups; w += 16) {
#pragma unroll
    for (int u = 0; u < 16; ++u) acc[u] += sd.part[(size_t)(w + u) * nout + o];
  }
  for (int u = 0; w + u < sd.groups; ++u) acc[u] += sd.part[(size_t)(w + u) * nout + o];
#pragma unroll
  for (int h = 8; h > 0; h >>= 1) {
#pragma unroll
    for (int u = 0; u < h; ++u) acc[u] += acc[u + h];
  }
  sd.red[o] = acc[0];
}

// 3. one workgroup per side: Gauss-Jordan elimination of [S | M] (r x 2r)
//    with the matrix in registers (the ownership above).  Step c needs row c
//    and column c: their owners publish them to LDS at the end of step c - 1
//    (double-buffered by parity, so one barrier per step).  Row c is divided
//    by the pivot; every other row loses its column-c multiple of row c.
//    Columns left of c are unit vectors by then and stay so.  Afterwards
//    the right half is Z.
template <int NQ>
__global__ __launch_bounds__(kThreads) void gram_solve_kernel(Sides args) {
  const Side sd = args.s[blockIdx.x];
  const int r = args.r, r2 = 2 * r;
  // rows and columns up to 255 so that stand-in indices stay in range
  __shared__ double rowb[2][kThreads];
  __shared__ double colb[2][kThreads];
  __shared__ double diag0[kMaxRank];
  const Own ow(r);
  const int j = ow.active ? ow.j : r2;        // r2: a column no step publishes
  double v[NQ];
  int ri[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int i = ow.g + ow.G * k;
    const bool live = ow.active && i < r;
    ri[k] = i;
    v[k] = live ? sd.red[i * r2 + j] : 0.0;
    if (live && i == j) diag0[i] = v[k];
    if (live && i == 0) rowb[0][j] = v[k];
    if (live && j == 0) colb[0][i] = v[k];
  }
  __syncthreads();
  bool bad = false;
  for (int c = 0; c < r; ++c) {
    const int b = c & 1;
    // every LDS read of the step first, so that they are in flight together
    const double rj = rowb[b][j];
    double cv[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) cv[k] = colb[b][ri[k]];
    // a pivot at or below 2^-46 of its original diagonal entry (64 units of
    // fp64 rounding) is a breakdown: the rank is deficient to within the
    // arithmetic
    const double piv = rowb[b][c];
    const bool ok = piv > 0x1p-46 * diag0[c];
    bad = bad || !ok;
    const double pj = rj / (ok ? piv : 1.0);
#pragma unroll
    for (int k = 0; k < NQ; ++k) v[k] = (ri[k] == c) ? pj : v[k] - cv[k] * pj;
    // publish row c + 1 (one owner row per thread at most) and column c + 1
    const int cn = c + 1;
    if (cn < r && ow.active && ow.g == cn % ow.G) {
      const int kp = cn / ow.G;
      double x = v[0];
#pragma unroll
      for (int k = 1; k < NQ; ++k) x = (k == kp) ? v[k] : x;
      rowb[b ^ 1][j] = x;
    }
    if (j == cn) {
#pragma unroll
      for (int k = 0; k < NQ; ++k) colb[b ^ 1][ri[k]] = v[k];
    }
    __syncthreads();
  }
  if (!ow.active || j < r) return;
  const double nan = __builtin_nan("");
#pragma unroll
  for (int k = 0; k < NQ; ++k)
    if (ri[k] < r) sd.Z[ri[k] * r + (j - r)] = bad ? nan : v[k];
}

// 4. g(s, j) = sum_i a(s, i) Z[i][j], rounded to fp32
__global__ __launch_bounds__(kThreads) void gram_apply_kernel(Sides args) {
  const Side sd = args.s[blockIdx.y];
  const int r = args.r, t = threadIdx.x;
  __shared__ double Zs[kMaxRank][kMaxRank + 1];
  for (int o = t; o < r * r; o += kThreads) Zs[o / r][o % r] = sd.Z[o];
  __syncthreads();
  const int64_t total = sd.L * r;
  const bool s_fast = sd.g_ss == 1;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + t; e < total; e += (int64_t)gridDim.x * kThreads) {
    const int64_t s = s_fast ? e % sd.L : e / r;
    const int j = (int)(s_fast ? e / sd.L : e % r);
    const uint16_t *arow = sd.A + s * sd.a_ss;
    double v = 0.0;
    for (int i = 0; i < r; ++i) v += (double)bf16_bits_to_float(arow[i * sd.a_si]) * Zs[i][j];
    sd.G[s * sd.g_ss + j * sd.g_si] = (float)v;
  }
}

int groups_for(int64_t L) {
  const int64_t g = (L + kChunk - 1) / kChunk;
  return (int)(g < 1 ? 1 : (g > kMaxGroups ? kMaxGroups : g));
}

}  // namespace

size_t gram_f32_ws_bytes(int64_t L, int l) {
  return (size_t)groups_for(L) * l * 2 * l * sizeof(double);
}

fs4_status launch_gram_f32(const float *A, int64_t L, int l, double *part, double *red, hipStream_t s) {
  Sides a;
  a.r = l;
  // the same matrix on both sides of [S | M]: red = [A^T A | A^T A]
  a.s[0] = Side{nullptr, l, 1, const_cast<float *>(A), l, 1, L, groups_for(L), part, red, nullptr, A};
  const int nq = nq_for(l);
#define FS4_GRAMF(NQ)                                                                        \
  case NQ:                                                                                   \
    gram_partial_kernel<NQ><<<dim3(a.s[0].groups, 1), kThreads, 0, s>>>(a);                  \
    break;
  switch (nq) {
    FS4_GRAMF(1) FS4_GRAMF(2) FS4_GRAMF(4) FS4_GRAMF(8) FS4_GRAMF(16) FS4_GRAMF(32)
    default: return FS4_ERR_RANK;
  }
#undef FS4_GRAMF
  gram_reduce_kernel<<<dim3((2 * l * l + kThreads - 1) / kThreads, 1), kThreads, 0, s>>>(a);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

size_t lora_project_ws_bytes(int64_t N, int64_t K, int r) {
  Carver c(nullptr);
  const int rr = r > 0 ? r : 1;
  for (int side = 0; side < 2; ++side) {
    c.take((size_t)groups_for(side ? K : N) * rr * 2 * rr * sizeof(double));
    c.take((size_t)rr * 2 * rr * sizeof(double));
    c.take((size_t)rr * rr * sizeof(double));
  }
  return c.off;
}

fs4_status launch_lora_project(const uint16_t *U, const uint16_t *V, int64_t N, int64_t K, int r,
                               float *dU, float *dV, void *ws, hipStream_t s) {
  if (r <= 0) return FS4_OK;
  Carver c(ws);
  const int rr = r;
  double *part_u = (double *)c.take((size_t)groups_for(N) * rr * 2 * rr * sizeof(double));
  double *red_u = (double *)c.take((size_t)rr * 2 * rr * sizeof(double));
  double *z_u = (double *)c.take((size_t)rr * rr * sizeof(double));
  double *part_v = (double *)c.take((size_t)groups_for(K) * rr * 2 * rr * sizeof(double));
  double *red_v = (double *)c.take((size_t)rr * 2 * rr * sizeof(double));
  double *z_v = (double *)c.take((size_t)rr * rr * sizeof(double));
  Sides a;
  a.r = r;
  int n = 0;
  if (dU && N > 0) {
    a.s[n++] = Side{U, r, 1, dU, r, 1, N, groups_for(N), part_u, red_u, z_u, nullptr};
  }
  if (dV && K > 0) {
    a.s[n++] = Side{V, 1, K, dV, 1, K, K, groups_for(K), part_v, red_v, z_v, nullptr};
  }
  if (n == 0) return FS4_OK;
  int gmax = 1;
  int64_t lmax = 1;
  for (int i = 0; i < n; ++i) {
    gmax = a.s[i].groups > gmax ? a.s[i].groups : gmax;
    lmax = a.s[i].L > lmax ? a.s[i].L : lmax;
  }
  const int nq = nq_for(r);
#define FS4_GRAM(NQ)                                                                        \
  case NQ:                                                                                  \
    gram_partial_kernel<NQ><<<dim3(gmax, n), kThreads, 0, s>>>(a);                          \
    gram_reduce_kernel<<<dim3((2 * r * r + kThreads - 1) / kThreads, n), kThreads, 0, s>>>(a); \
    gram_solve_kernel<NQ><<<n, kThreads, 0, s>>>(a);                                        \
    break;
  switch (nq) {
    FS4_GRAM(1) FS4_GRAM(2) FS4_GRAM(4) FS4_GRAM(8) FS4_GRAM(16) FS4_GRAM(32)
    default: return FS4_ERR_RANK;
  }
#undef FS4_GRAM
  int64_t blocks = (lmax * r + kThreads - 1) / kThreads;
  if (blocks > 2048) blocks = 2048;
  gram_apply_kernel<<<dim3((unsigned)blocks, n), kThreads, 0, s>>>(a);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
