// Per-iteration Newton-Schulz coefficients.
//
// The DeepSpeed RFC "Enable Correct and High-Performance Muon Optimizer under
// ZeRO CPU Offload" (section 5, Roadmap) lists Newton-Schulz with
// coefficients optimised for each iteration ("Polar Express") so that fewer
// iterations reach the same accuracy; it gives no table.  Each iteration maps
// every singular value x of the iterate to p(x) = a x + b x^3 + c x^5, so the
// schedule is built on scalars: iteration t takes the odd quintic closest to
// 1 in the maximum norm on the interval the singular values occupy at that
// point, and the values then occupy that polynomial's image.  Pure host code.
#include <algorithm>
#include <cmath>

#include "muon.h"

namespace {

struct Quintic {
  double a, b, c;
  double operator()(double x) const {
    const double x2 = x * x;
    return x * (a + x2 * (b + x2 * c));
  }
};

// Solve the 4 x 4 system held in m[r][0..3] x = m[r][4] in place (Gaussian
// elimination, partial pivoting); the solution lands in m[r][4].
bool solve4(double m[4][5]) {
  for (int col = 0; col < 4; ++col) {
    int piv = col;
    for (int r = col + 1; r < 4; ++r)
      if (std::fabs(m[r][col]) > std::fabs(m[piv][col])) piv = r;
    if (m[piv][col] == 0.0) return false;
    if (piv != col)
      for (int k = 0; k < 5; ++k) std::swap(m[piv][k], m[col][k]);
    for (int r = col + 1; r < 4; ++r) {
      const double f = m[r][col] / m[col][col];
      for (int k = col; k < 5; ++k) m[r][k] -= f * m[col][k];
    }
  }
  for (int r = 3; r >= 0; --r) {
    double v = m[r][4];
    for (int k = r + 1; k < 4; ++k) v -= m[r][k] * m[k][4];
    m[r][4] = v / m[r][r];
  }
  return true;
}

// Best approximation of 1 on [lo, hi] (0 < lo < hi) by an odd quintic, by
// Remez exchange.  The error 1 - p of the best p takes its extreme value with
// alternating signs at four points; p' is a quadratic in x^2, so p has at
// most two interior extrema and the two ends are alternation points.  A
// round fits p(x_i) + s_i E = 1, s = (+1, -1, +1, -1), on the current points
// and moves the two interior points to the new extrema of p.
bool best_quintic(double lo, double hi, Quintic* best, double* err) {
  const double kPi = 3.14159265358979323846;
  double x[4] = {lo, 0.0, 0.0, hi};
  // start: extrema of the degree-3 Chebyshev polynomial mapped onto [lo, hi]
  for (int i = 1; i <= 2; ++i) x[i] = 0.5 * (lo + hi) - 0.5 * (hi - lo) * std::cos(kPi * i / 3.0);
  // fit p(x_i) + s_i E = 1 on the current points
  auto fit = [&](Quintic* p, double* e) {
    double m[4][5];
    for (int i = 0; i < 4; ++i) {
      const double xi = x[i], x3 = xi * xi * xi;
      m[i][0] = xi;
      m[i][1] = x3;
      m[i][2] = x3 * xi * xi;
      m[i][3] = (i % 2 == 0) ? 1.0 : -1.0;
      m[i][4] = 1.0;
    }
    if (!solve4(m)) return false;
    *p = Quintic{m[0][4], m[1][4], m[2][4]};
    *e = m[3][4];
    return true;
  };
  Quintic p{0.0, 0.0, 0.0};
  double e = 0.0;
  // The exchange converges quadratically; the points then settle within the
  // rounding noise of the fit, which grows as the interval narrows.
  for (int round = 0; round < 100; ++round) {
    if (!fit(&p, &e)) return false;
    // interior extrema: p'(x) = a + 3 b s + 5 c s^2 = 0 with s = x^2
    const double qa = 5.0 * p.c, qb = 3.0 * p.b, qc = p.a;
    const double disc = qb * qb - 4.0 * qa * qc;
    if (qa == 0.0 || !(disc >= 0.0)) return false;
    const double q = -0.5 * (qb + std::copysign(std::sqrt(disc), qb));
    if (q == 0.0) return false;
    double s1 = q / qa, s2 = qc / q;
    if (s1 > s2) std::swap(s1, s2);
    if (!(lo * lo < s1 && s1 < s2 && s2 < hi * hi)) return false;
    const double x1 = std::sqrt(s1), x2 = std::sqrt(s2);
    const double moved = std::max(std::fabs(x1 - x[1]), std::fabs(x2 - x[2]));
    x[1] = x1;
    x[2] = x2;
    if (moved <= 1e-12 * (hi - lo)) break;
  }
  if (!fit(&p, &e)) return false;
  *best = p;
  *err = std::fabs(e);
  return std::isfinite(p.a) && std::isfinite(p.b) && std::isfinite(p.c) && std::isfinite(e);
}

}  // namespace

extern "C" muon_status_t muon_ns_minimax_coeffs(int32_t steps, double lo, double margin,
                                                float* out, double* bound) {
  // margins outside [0.01, 0.1] are refused: with bf16 iterates, low-rank
  // inputs measured a relative error of 0.36 at margin 0 (values that
  // rounding pushes past the top of the interval meet the polynomial's steep
  // rise) and up to 0.14 at margin 0.2 (a wider interval, a coarser fit)
  if (out == nullptr || steps < 1 || steps > 1024 || !(lo > 0.0 && lo < 1.0) ||
      !(margin >= 0.01 && margin <= 0.1))
    return MUON_EINVAL;
  // As the interval shrinks to {1} the best polynomial tends to the one that
  // matches 1 to third order there: p(1) = 1, p'(1) = p''(1) = 0, i.e.
  // (15/8, -5/4, 3/8), with p'(x) = (15/8) (1 - x^2)^2 >= 0.
  const Quintic limit{15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0};
  double l = lo, u = 1.0, e = 1.0 - lo;
  for (int t = 0; t < steps; ++t) {
    const double top = u * (1.0 + margin);
    Quintic p;
    if (top - l < 1e-3) {
      p = limit;  // increasing: its extremes on [l, top] sit at the ends
      e = std::max(1.0 - p(l), p(top) - 1.0);
    } else if (!best_quintic(l, top, &p, &e)) {
      return MUON_EINVAL;
    }
    out[3 * t + 0] = static_cast<float>(p.a);
    out[3 * t + 1] = static_cast<float>(p.b);
    out[3 * t + 2] = static_cast<float>(p.c);
    l = 1.0 - e;
    u = 1.0 + e;
  }
  if (bound != nullptr) *bound = e;
  return MUON_OK;
}
