// Gauss quadrature rules for the Gaussian selector at general alpha
// (Technical Summary: EntmaxKV, §2.B.2): the expectations E[(Z - tau)_+^r]
// of its normalisation have a closed form only for r in {1, 2}, so for other
// r the kernel sums them with the rules built here, on the host, once per
// call.
//
// A rule for a weight w on an interval is fixed by the three-term
// recurrence of the weight's orthonormal polynomials,
//   x p_k(x) = b_(k+1) p_(k+1)(x) + a_k p_k(x) + b_k p_(k-1)(x),
// p_0 = 1/sqrt(mu0), mu0 the weight's mass.  The n nodes are the zeros of
// p_n, i.e. the eigenvalues of the symmetric tridiagonal matrix with
// diagonal a_0..a_(n-1) and off-diagonal b_1..b_(n-1); each is isolated
// here by bisection on a Sturm count (the number of negative pivots of the
// LDL^T factorisation of the matrix minus x equals the number of
// eigenvalues below x).  The weight of node x_i is the Christoffel number
// 1 / sum_(k<n) p_k(x_i)^2.
#include <math.h>

#include "gauss_rule.h"

namespace ekv {
namespace {

// Eigenvalues of the symmetric tridiagonal (a[0..n), b2[1..n) = squared
// off-diagonal), ascending, each to the last bit by bisection.
void tridiag_eigenvalues(int n, const double *a, const double *b2, double *x) {
  // Gershgorin bounds
  double lo = INFINITY, hi = -INFINITY;
  for (int i = 0; i < n; ++i) {
    const double r = (i > 0 ? sqrt(b2[i]) : 0.0) + (i + 1 < n ? sqrt(b2[i + 1]) : 0.0);
    lo = fmin(lo, a[i] - r);
    hi = fmax(hi, a[i] + r);
  }
  // number of eigenvalues strictly below t
  auto below = [&](double t) {
    int cnt = 0;
    double q = a[0] - t;
    if (q < 0.0) ++cnt;
    for (int i = 1; i < n; ++i) {
      // a zero pivot (t an eigenvalue of the leading block) is replaced by
      // a tiny positive one, i.e. counted as non-negative
      const double prev = q != 0.0 ? q : 1e-300;
      q = (a[i] - t) - b2[i] / prev;
      if (q < 0.0) ++cnt;
    }
    return cnt;
  };
  for (int k = 0; k < n; ++k) {  // the k-th smallest eigenvalue
    double l = lo, h = hi;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (l + h);
      if (mid <= l || mid >= h) break;
      if (below(mid) > k) h = mid;
      else l = mid;
    }
    x[k] = 0.5 * (l + h);
  }
}

// Nodes and Christoffel weights from the recurrence (a, b2) and mass mu0.
void gauss_rule(int n, const double *a, const double *b2, double mu0,
                double *x, double *w) {
  tridiag_eigenvalues(n, a, b2, x);
  for (int i = 0; i < n; ++i) {
    double pm = 0.0, p = 1.0 / sqrt(mu0), sum = p * p;
    for (int k = 0; k + 1 < n; ++k) {
      const double pn = ((x[i] - a[k]) * p - (k > 0 ? sqrt(b2[k]) * pm : 0.0)) /
                        sqrt(b2[k + 1]);
      pm = p;
      p = pn;
      sum += p * p;
    }
    w[i] = 1.0 / sum;
  }
}

}  // namespace

// Gauss-Jacobi: weight (1 + x)^beta on [-1, 1], beta > -1.  The monic
// Jacobi recurrence for (1 - x)^a (1 + x)^b with a = 0:
//   a_k = b^2 / ((2k + b)(2k + b + 2)),
//   b_k^2 = 4 k^2 (k + b)^2 / ((2k + b)^2 (2k + b + 1)(2k + b - 1)),
// and mass mu0 = 2^(b+1) / (b + 1).
bool gauss_jacobi_rule(double beta, int n, double *x, double *w) {
  if (!(beta > -1.0) || n < 1 || n > kMaxRuleNodes) return false;
  double a[kMaxRuleNodes], b2[kMaxRuleNodes];
  for (int k = 0; k < n; ++k) {
    const double s = 2.0 * k + beta;
    a[k] = s != 0.0 ? beta * beta / (s * (s + 2.0)) : 0.0;  // 0/0 at k = 0, beta = 0
    if (k > 0) {
      const double kk = static_cast<double>(k);
      b2[k] = 4.0 * kk * kk * (kk + beta) * (kk + beta) /
              (s * s * (s + 1.0) * (s - 1.0));
    }
  }
  b2[0] = 0.0;
  gauss_rule(n, a, b2, pow(2.0, beta + 1.0) / (beta + 1.0), x, w);
  return true;
}

// Gauss-Hermite for the standard normal density: the monic probabilists'
// Hermite polynomials satisfy He_(k+1) = x He_k - k He_(k-1), so a_k = 0,
// b_k^2 = k, and the density has mass 1.
bool gauss_hermite_rule(int n, double *x, double *w) {
  if (n < 1 || n > kMaxRuleNodes) return false;
  double a[kMaxRuleNodes], b2[kMaxRuleNodes];
  for (int k = 0; k < n; ++k) {
    a[k] = 0.0;
    b2[k] = static_cast<double>(k);
  }
  gauss_rule(n, a, b2, 1.0, x, w);
  return true;
}

}  // namespace ekv
