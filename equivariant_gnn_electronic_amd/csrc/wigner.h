// Edge frame and Wigner-D rows, as inline host+device code.
//
// MALOQ Sec. III-C1 / Fig. 3(b,c): every edge is rotated onto +y; the
// embedding of degree l is multiplied by D^l(R) of that rotation.
//
// D^l is built from D^1 = R by the Ivanic-Ruedenberg recursion for real
// spherical harmonics (J. Ivanic, K. Ruedenberg, J. Phys. Chem. 100, 6342
// (1996), with the 1998 erratum): every entry of D^l is a combination of
// products of D^1 entries with entries of D^(l-1) in neighbouring rows.
// In the basis used here (polar axis y, degree 1 proportional to (x, y, z),
// no Condon-Shortley phase) the recursion applies with D^1 = R itself.
#pragma once

#include "common.h"

namespace egnn {

// R_e = (R_y(a) R_x(b))^T taking the unit edge direction to +y, zero roll.
// Formed in fp64 and rounded once: the recursion multiplies R into every
// degree, so an fp32 normalisation's error (~2e-7 in R) grows to ~1e-6 by
// degree 8, against ~5e-7 from a correctly rounded R (measured on the host
// over 2e5 random directions).  A handful of fp64 operations per edge.
__host__ __device__ inline void edge_rotation(float vx, float vy, float vz, float R[3][3]) {
  const double X = vx, Y = vy, Z = vz;
  const double inv = 1.0 / sqrt(X * X + Y * Y + Z * Z);
  const double x = X * inv, y = Y * inv, z = Z * inv;
  const double s = sqrt(x * x + z * z);
  double ca = 1.0, sa = 0.0;
  if (s > 0.0) {
    ca = z / s;
    sa = x / s;
  }
  const double cb = y, sb = s;
  R[0][0] = float(ca);      R[0][1] = 0.0f;       R[0][2] = float(-sa);
  R[1][0] = float(sa * sb); R[1][1] = float(cb);  R[1][2] = float(ca * sb);
  R[2][0] = float(sa * cb); R[2][1] = float(-sb); R[2][2] = float(ca * cb);
}

// One level of the recursion: rows |m| <= MROWS of D^L from the full D^(L-1).
// Dp: (2L-1)^2 row-major, Dl: (2L+1)^2 row-major (only rows |m| <= MROWS written).
template <int L, int MROWS>
__host__ __device__ inline void ir_level(const float (&R1)[3][3], const float *Dp, float *Dl) {
  constexpr int WP = 2 * L - 1;
  auto rp = [&](int mu, int nu) -> float { return Dp[(mu + L - 1) * WP + (nu + L - 1)]; };
  auto r1 = [&](int i, int j) -> float { return R1[i + 1][j + 1]; };
  auto P = [&](int i, int mu, int mp) -> float {
    if (mp == L) return r1(i, 1) * rp(mu, L - 1) - r1(i, -1) * rp(mu, -L + 1);
    if (mp == -L) return r1(i, 1) * rp(mu, -L + 1) + r1(i, -1) * rp(mu, L - 1);
    return r1(i, 0) * rp(mu, mp);
  };
#pragma unroll
  for (int m = -MROWS; m <= MROWS; ++m) {
#pragma unroll
    for (int mp = -L; mp <= L; ++mp) {
      const int am = cabs(m);
      const float denom = (cabs(mp) == L) ? float((2 * L) * (2 * L - 1)) : float((L + mp) * (L - mp));
      const float d0 = (m == 0) ? 1.0f : 0.0f;
      const float u = sqrtf(float((L + m) * (L - m)) / denom);
      const float v = 0.5f * sqrtf((1.0f + d0) * float((L + am - 1) * (L + am)) / denom) * (1.0f - 2.0f * d0);
      const float w = -0.5f * sqrtf(float((L - am - 1) * (L - am)) / denom) * (1.0f - d0);
      float val = 0.0f;
      if ((L + m) * (L - m) != 0) val += u * P(0, m, mp);
      if (m == 0) {
        val += v * (P(1, 1, mp) + P(-1, -1, mp));
      } else if (m > 0) {
        float V = P(1, m - 1, mp) * (m == 1 ? 1.41421356237309515f : 1.0f);
        if (m != 1) V -= P(-1, -m + 1, mp);
        val += v * V;
        if ((L - am - 1) * (L - am) != 0) val += w * (P(1, m + 1, mp) + P(-1, -m - 1, mp));
      } else {
        float V = P(-1, -m - 1, mp) * (m == -1 ? 1.41421356237309515f : 1.0f);
        if (m != -1) V += P(1, m + 1, mp);
        val += v * V;
        if ((L - am - 1) * (L - am) != 0) val += w * (P(1, m - 1, mp) - P(-1, -m + 1, mp));
      }
      Dl[(m + L) * (2 * L + 1) + (mp + L)] = val;
    }
  }
}

// Rows |m| <= MMAX of D^L stored in the layout of egnn_edge_geom.
template <int L, int MMAX>
__host__ __device__ inline void store_rows(const float *Dl, float *out) {
  constexpr int mr = cmin(L, MMAX);
  constexpr int off = d_block_offset(L, MMAX);
#pragma unroll
  for (int m = -mr; m <= mr; ++m)
#pragma unroll
    for (int mp = -L; mp <= L; ++mp) out[off + (m + mr) * (2 * L + 1) + (mp + L)] = Dl[(m + L) * (2 * L + 1) + (mp + L)];
}

// Level L of the recursion and the levels above it.  Level L is needed in
// rows |m| <= MMAX for storage and, for each later level, in one more row
// than that level needs: rows |m| <= min(L, MMAX + LMAX - L).
template <int L, int LMAX, int MMAX>
__host__ __device__ inline void wigner_up(const float (&R)[3][3], const float *Dp, float *out) {
  if constexpr (L <= LMAX) {
    constexpr int ROWS = cmin(L, MMAX + (LMAX - L));
    float Dl[(2 * L + 1) * (2 * L + 1)];
    ir_level<L, ROWS>(R, Dp, Dl);
    store_rows<L, MMAX>(Dl, out);
    wigner_up<L + 1, LMAX, MMAX>(R, Dl, out);
  }
}

// Stored rows |m| <= MMAX of D^l(R), l = 0..LMAX, in the layout of egnn_edge_geom.
template <int LMAX, int MMAX>
__host__ __device__ inline void wigner_rows(const float (&R)[3][3], float *out) {
  out[0] = 1.0f;
  if constexpr (LMAX >= 1) {
    float D1[9];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) D1[i * 3 + j] = R[i][j];
    store_rows<1, MMAX>(D1, out);
    wigner_up<2, LMAX, MMAX>(R, D1, out);
  }
}

// Gaussian radial basis with cosine envelope.
__host__ __device__ inline float rbf_value(float d, int k, int n_rbf, float r_cut) {
  const float step = r_cut / float(n_rbf - 1);
  const float mu = float(k) * step;
  const float t = (d - mu) / step;
  const float env = 0.5f * (cosf(3.14159265358979323846f * d / r_cut) + 1.0f);
  return expf(-0.5f * t * t) * env;
}

}  // namespace egnn
