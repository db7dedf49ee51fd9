// Quadrature rules of the Gaussian selector at general alpha: built on the
// host (quadrature.hip) and passed to the threshold kernel by value.
#pragma once

namespace ekv {

constexpr int kMaxRuleNodes = 64;  // largest rule the builders accept
constexpr int kJacobiNodes = 24;   // rule for y^r on [0, Y] (see select.hip)
constexpr int kHermiteNodes = 16;  // rule for the standard normal density

// Gauss-Jacobi nodes and weights for (1 + x)^beta on [-1, 1], beta > -1.
bool gauss_jacobi_rule(double beta, int n, double *x, double *w);
// Gauss-Hermite nodes and weights for the standard normal density.
bool gauss_hermite_rule(int n, double *x, double *w);

// Kernel argument: the exponent r and both rules in float.
struct GaussRule {
  float r;
  float jx[kJacobiNodes], jw[kJacobiNodes];
  float hx[kHermiteNodes], hw[kHermiteNodes];
};

}  // namespace ekv
