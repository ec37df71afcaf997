// Shape-dependent Newton-Schulz coefficients (host code, no kernels).
//
// Full-Stack FP4 [FS4 §2.3] stabilises the NVFP4 Newton-Schulz iteration
// with quintic coefficients (a, b, c) tuned to the matrix's aspect ratio,
// without printing them or the criterion.  Taken here: for an m x n momentum
// (m <= n) the coefficients minimise the mean squared distance of the
// 5-fold quintic p(s) = a s + b s^3 + c s^5 to 1 (the polar factor's
// singular values), averaged over the singular-value law of a Frobenius-
// normalised m x n Gaussian matrix.  That law is Marchenko-Pastur: with
// y = m / n the eigenvalues of G G^T / n lie on [(1 - sqrt y)^2,
// (1 + sqrt y)^2] with density sqrt((l+ - l)(l - l-)) / (2 pi y l), and the
// normalised singular values are sqrt(l / m).  The average is a Gauss-
// Chebyshev (second kind) quadrature, whose weight absorbs the density's
// square-root edges; the minimum is found by Nelder-Mead from Muon's quintic.
#include <cmath>
#include <vector>

#include "fs4_common.h"

namespace {

struct Quadrature {
  std::vector<double> s, w;   // normalised singular values and weights (sum 1)
};

Quadrature mp_quadrature(int64_t m, int64_t n, int points) {
  const double y = (double)m / (double)n;
  const double lo = (1.0 - std::sqrt(y)) * (1.0 - std::sqrt(y)), hi = (1.0 + std::sqrt(y)) * (1.0 + std::sqrt(y));
  Quadrature q;
  q.s.resize(points);
  q.w.resize(points);
  double tot = 0.0;
  for (int k = 1; k <= points; ++k) {
    const double th = (double)k * M_PI / (double)(points + 1);
    const double lam = 0.5 * (hi + lo) + 0.5 * (hi - lo) * std::cos(th);
    const double w = std::sin(th) * std::sin(th) / lam;   // the common factors cancel in the normalisation
    q.s[k - 1] = std::sqrt(lam / (double)m);
    q.w[k - 1] = w;
    tot += w;
  }
  for (double &w : q.w) w /= tot;
  return q;
}

double distance(const Quadrature &q, const double *abc, int steps) {
  double acc = 0.0;
  for (size_t i = 0; i < q.s.size(); ++i) {
    double s = q.s[i];
    for (int k = 0; k < steps; ++k) {
      const double s2 = s * s;
      s = s * (abc[0] + s2 * (abc[1] + s2 * abc[2]));
    }
    acc += q.w[i] * (s - 1.0) * (s - 1.0);
  }
  return acc;
}

// Nelder-Mead (reflection 1, expansion 2, contraction 1/2, shrink 1/2) on
// three variables; stops when the simplex's values and extent are both tiny.
void nelder_mead(const Quadrature &q, int steps, double *x) {
  double p[4][3], f[4];
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 3; ++j) p[i][j] = x[j];
    if (i > 0) p[i][i - 1] += (x[i - 1] != 0.0 ? 0.05 * x[i - 1] : 0.00025);
    f[i] = distance(q, p[i], steps);
  }
  for (int it = 0; it < 40000; ++it) {
    // order the vertices by value
    for (int a = 0; a < 4; ++a)
      for (int b = a + 1; b < 4; ++b)
        if (f[b] < f[a]) {
          std::swap(f[a], f[b]);
          for (int j = 0; j < 3; ++j) std::swap(p[a][j], p[b][j]);
        }
    double extent = 0.0;
    for (int i = 1; i < 4; ++i)
      for (int j = 0; j < 3; ++j) extent = std::fmax(extent, std::fabs(p[i][j] - p[0][j]));
    if (extent < 1e-10 && f[3] - f[0] < 1e-14) break;
    double c[3];
    for (int j = 0; j < 3; ++j) c[j] = (p[0][j] + p[1][j] + p[2][j]) / 3.0;
    double r[3], e[3], k[3];
    for (int j = 0; j < 3; ++j) r[j] = c[j] + (c[j] - p[3][j]);
    const double fr = distance(q, r, steps);
    if (fr < f[0]) {
      for (int j = 0; j < 3; ++j) e[j] = c[j] + 2.0 * (c[j] - p[3][j]);
      const double fe = distance(q, e, steps);
      const double *keep = fe < fr ? e : r;
      for (int j = 0; j < 3; ++j) p[3][j] = keep[j];
      f[3] = fe < fr ? fe : fr;
    } else if (fr < f[2]) {
      for (int j = 0; j < 3; ++j) p[3][j] = r[j];
      f[3] = fr;
    } else {
      const bool outside = fr < f[3];
      for (int j = 0; j < 3; ++j) k[j] = outside ? c[j] + 0.5 * (r[j] - c[j]) : c[j] + 0.5 * (p[3][j] - c[j]);
      const double fk = distance(q, k, steps);
      if (fk < (outside ? fr : f[3])) {
        for (int j = 0; j < 3; ++j) p[3][j] = k[j];
        f[3] = fk;
      } else {
        for (int i = 1; i < 4; ++i) {
          for (int j = 0; j < 3; ++j) p[i][j] = p[0][j] + 0.5 * (p[i][j] - p[0][j]);
          f[i] = distance(q, p[i], steps);
        }
      }
    }
  }
  int best = 0;
  for (int i = 1; i < 4; ++i)
    if (f[i] < f[best]) best = i;
  for (int j = 0; j < 3; ++j) x[j] = p[best][j];
}

}  // namespace

extern "C" fs4_status fs4_ns_shape_coefficients(int64_t m, int64_t n, int steps, float *abc, double *distance_out) {
  if (!abc) return FS4_ERR_NULL;
  if (m <= 0 || n <= 0 || steps < 1 || steps > 16) return FS4_ERR_ARG;
  if (m > n) std::swap(m, n);
  const Quadrature q = mp_quadrature(m, n, 400);
  double x[3] = {3.4445, -4.7750, 2.0315};
  nelder_mead(q, steps, x);
  for (int j = 0; j < 3; ++j) abc[j] = (float)x[j];
  if (distance_out) {
    const double xf[3] = {(double)abc[0], (double)abc[1], (double)abc[2]};
    *distance_out = distance(q, xf, steps);
  }
  return FS4_OK;
}
