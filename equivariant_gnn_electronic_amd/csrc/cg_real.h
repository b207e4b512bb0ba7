// Real Clebsch-Gordan couplings on the host (MALOQ Sec. III-B1, Eq. (1)).
//
// Complex CG coefficients come from Racah's closed formula; they are changed
// to the real basis of the irreps (polar axis y, degree 1 ~ (x, y, z), no
// Condon-Shortley phase), made real by removing a global phase, normalised,
// and signed so that the first entry of magnitude > 1e-9 in row-major
// (i, j, M) order is positive.  Used to build the device tables of the decode
// and of Matrix <-> Label; any degree works.
#pragma once

#include <cmath>
#include <complex>
#include <vector>

namespace egnn {
namespace cg {

inline double fact(int n) {
  double r = 1.0;
  for (int i = 2; i <= n; ++i) r *= i;
  return r;
}

// <j1 m1 j2 m2 | J M>, integer angular momenta, Condon-Shortley convention.
inline double cg_complex(int j1, int m1, int j2, int m2, int J, int M) {
  if (M != m1 + m2) return 0.0;
  if (J < std::abs(j1 - j2) || J > j1 + j2) return 0.0;
  if (std::abs(m1) > j1 || std::abs(m2) > j2 || std::abs(M) > J) return 0.0;
  double pre = std::sqrt((2.0 * J + 1.0) * fact(J + j1 - j2) * fact(J - j1 + j2) * fact(j1 + j2 - J) /
                         fact(j1 + j2 + J + 1));
  pre *= std::sqrt(fact(J + M) * fact(J - M) * fact(j1 - m1) * fact(j1 + m1) * fact(j2 - m2) * fact(j2 + m2));
  double sum = 0.0;
  for (int k = 0; k <= j1 + j2 + J; ++k) {
    int a[6] = {k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k};
    bool ok = true;
    for (int v : a) ok = ok && v >= 0;
    if (!ok) continue;
    double den = 1.0;
    for (int v : a) den *= fact(v);
    sum += ((k & 1) ? -1.0 : 1.0) / den;
  }
  return pre * sum;
}

// Row m (= -l..l) of the complex -> real change of basis: S_m = sum_mu U[m][mu] Y_mu.
inline std::complex<double> U(int l, int m, int mu) {
  const double r2 = 1.0 / std::sqrt(2.0);
  const std::complex<double> I(0.0, 1.0);
  if (m == 0) return mu == 0 ? 1.0 : 0.0;
  if (m > 0) {
    if (mu == m) return ((m & 1) ? -1.0 : 1.0) * r2;
    if (mu == -m) return r2;
    return 0.0;
  }
  const int a = -m;
  if (mu == a) return ((a & 1) ? -1.0 : 1.0) * r2 / I;
  if (mu == -a) return -r2 / I;
  return 0.0;
}

// Real coupling Q[i][j][M] (i: la, j: lb, M: L), row-major.
inline std::vector<double> real_coupling(int la, int lb, int L) {
  const int na = 2 * la + 1, nb = 2 * lb + 1, nL = 2 * L + 1;
  std::vector<std::complex<double>> q(static_cast<size_t>(na) * nb * nL);
  for (int i = -la; i <= la; ++i)
    for (int j = -lb; j <= lb; ++j)
      for (int N = -L; N <= L; ++N) {
        std::complex<double> acc = 0.0;
        for (int a = -la; a <= la; ++a) {
          std::complex<double> ua = U(la, i, a);
          if (ua == 0.0) continue;
          for (int b = -lb; b <= lb; ++b) {
            std::complex<double> ub = U(lb, j, b);
            if (ub == 0.0) continue;
            const int M = a + b;
            if (std::abs(M) > L) continue;
            acc += ua * ub * cg_complex(la, a, lb, b, L, M) * std::conj(U(L, N, M));
          }
        }
        q[((i + la) * nb + (j + lb)) * nL + (N + L)] = acc;
      }
  size_t big = 0;
  for (size_t t = 0; t < q.size(); ++t)
    if (std::abs(q[t]) > std::abs(q[big])) big = t;
  const std::complex<double> phase = q[big] / std::abs(q[big]);
  std::vector<double> r(q.size());
  for (size_t t = 0; t < q.size(); ++t) r[t] = (q[t] / phase).real();
  double nrm = 0.0;
  for (int i = 0; i < na; ++i)
    for (int j = 0; j < nb; ++j) nrm += r[(i * nb + j) * nL] * r[(i * nb + j) * nL];
  nrm = std::sqrt(nrm);
  for (double &v : r) v /= nrm;
  for (double v : r)
    if (std::fabs(v) > 1e-9) {
      if (v < 0)
        for (double &w : r) w = -w;
      break;
    }
  return r;
}

}  // namespace cg
}  // namespace egnn
