// Spectral step of subspace calibration (JSSA abstract on weekinpapers,
// Abstract: the marginal bound on the score-preservation error has a
// closed-form spectral solution): the top-r eigenvectors of a symmetric
// d x d operator, once per KV head, offline. Host code: d = 128 takes a few
// cyclic Jacobi sweeps of 8128 plane rotations each.
//
// Cyclic Jacobi (Golub and Van Loan, Matrix Computations, the symmetric
// Schur decomposition and the cyclic Jacobi method): for every off-diagonal
// pair (p, q) a plane rotation J with cos c and sin s is chosen so that
// (J^T A J)[p][q] = 0, with tau = (a_qq - a_pp) / (2 a_pq),
// t = sign(tau) / (|tau| + sqrt(1 + tau^2)), c = 1 / sqrt(1 + t^2), s = t c;
// A <- J^T A J and V <- V J. Sweeps repeat until the off-diagonal mass is
// negligible against the diagonal; the diagonal then holds the eigenvalues
// and the columns of V the eigenvectors.
#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "internal.hpp"

namespace jssa {

bool symmetric_top_eigen(int d, int r, const double* M, double* V, double* w) {
  std::vector<double> A(M, M + size_t(d) * d), U(size_t(d) * d, 0.0);
  for (int i = 0; i < d; ++i) U[size_t(i) * d + i] = 1.0;
  auto a = [&](int i, int k) -> double& { return A[size_t(i) * d + k]; };
  auto u = [&](int i, int k) -> double& { return U[size_t(i) * d + k]; };
  // symmetrise (the input is symmetric up to rounding)
  for (int i = 0; i < d; ++i)
    for (int k = i + 1; k < d; ++k) a(i, k) = a(k, i) = 0.5 * (a(i, k) + a(k, i));
  bool converged = false;
  for (int sweep = 0; sweep < 64 && !converged; ++sweep) {
    double off2 = 0.0, tot2 = 0.0;
    for (int i = 0; i < d; ++i) {
      tot2 += a(i, i) * a(i, i);
      for (int k = i + 1; k < d; ++k) off2 += 2.0 * a(i, k) * a(i, k);
    }
    tot2 += off2;
    if (off2 <= 1e-30 * tot2 || tot2 == 0.0) {
      converged = true;
      break;
    }
    for (int p = 0; p < d - 1; ++p) {
      for (int q = p + 1; q < d; ++q) {
        const double apq = a(p, q);
        if (apq == 0.0) continue;
        const double tau = (a(q, q) - a(p, p)) / (2.0 * apq);
        const double t = (tau >= 0.0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int k = 0; k < d; ++k) {              // A <- A J (columns p, q)
          const double akp = a(k, p), akq = a(k, q);
          a(k, p) = c * akp - s * akq;
          a(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {              // A <- J^T A (rows p, q)
          const double apk = a(p, k), aqk = a(q, k);
          a(p, k) = c * apk - s * aqk;
          a(q, k) = s * apk + c * aqk;
        }
        a(p, q) = a(q, p) = 0.0;
        for (int k = 0; k < d; ++k) {              // V <- V J
          const double ukp = u(k, p), ukq = u(k, q);
          u(k, p) = c * ukp - s * ukq;
          u(k, q) = s * ukp + c * ukq;
        }
      }
    }
  }
  std::vector<int> order(d);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return a(x, x) > a(y, y); });
  for (int c = 0; c < r; ++c) {
    const int col = order[c];
    int big = 0;
    for (int i = 1; i < d; ++i)
      if (std::fabs(u(i, col)) > std::fabs(u(big, col))) big = i;
    const double sg = u(big, col) < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) V[size_t(i) * r + c] = sg * u(i, col);
    w[c] = a(col, col);
  }
  return converged;
}

}  // namespace jssa
