"""Real spherical harmonics, Wigner-D matrices, edge frames and real CG couplings (fp64).

Test infrastructure only (see oracle/__init__.py).

Basis (a reading: the pages write states as complex |l, m> and never fix a
real basis, axis order or sign):
  Y_{l,m}(x, y, z) = S_{l,m}(z, x, y), m = -l..l,
where S_{l,m}(X, Y, Z) are the orthonormal real tesseral harmonics about the
Z axis without the Condon-Shortley phase: proportional to cos(m phi) for m > 0
and sin(|m| phi) for m < 0.  The polar axis of Y is therefore y -- the common
axis every edge is rotated onto (MALOQ Sec. III-C1, Fig. 3(b)) -- and Y_1 is
proportional to (x, y, z), so the l = 1 Wigner block is the rotation matrix.

Wigner-D (MALOQ Sec. III-C1: a rotation R of the system multiplies each
degree-l block of an embedding by D^l(R)) is taken by its defining identity
  D^l(R) Y^l(r) = Y^l(R r)  for every unit vector r,
solved by least squares over a fixed spherical point set (exact, since the
span of Y^l is rotation invariant).
"""
from __future__ import annotations

from functools import lru_cache
from math import comb, factorial, pi, sqrt

import numpy as np


def coeff_index(l, m):
    """Row of coefficient (l, m) in an irreps block: l^2 + l + m."""
    return l * l + l + m


def _legendre_deriv(l, m):
    """Polynomial coefficients (ascending powers) of d^m/dt^m P_l(t).

    P_l(t) = 2^-l sum_k (-1)^k C(l,k) C(2l-2k, l) t^(l-2k)  (explicit sum form).
    """
    c = np.zeros(l + 1)
    for k in range(l // 2 + 1):
        c[l - 2 * k] += (-1) ** k * comb(l, k) * comb(2 * l - 2 * k, l) / 2.0 ** l
    for _ in range(m):
        c = np.array([i * c[i] for i in range(1, len(c))]) if len(c) > 1 else np.zeros(1)
    return c


def real_sh(l, r):
    """Y_{l,m}(r) for unit vectors r [..., 3]; returns [..., 2l+1] ordered m = -l..l.

    With polar axis y and azimuth phi measured from z towards x,
      Y_{l,0}   = N_{l0} P_l(y)
      Y_{l,+m}  = sqrt(2) N_{lm} P_l^(m)(y) Re (z + i x)^m
      Y_{l,-m}  = sqrt(2) N_{lm} P_l^(m)(y) Im (z + i x)^m
    where P_l^(m) is the m-th derivative of the Legendre polynomial (no
    Condon-Shortley phase) and N_{lm} = sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!).
    The factor (1 - y^2)^(m/2) of the associated Legendre function is carried
    by |z + i x|^m = rho^m, which is valid on the unit sphere.
    """
    r = np.asarray(r, dtype=np.float64)
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    out = np.zeros(r.shape[:-1] + (2 * l + 1,))
    w = z + 1j * x
    for m in range(0, l + 1):
        n_lm = sqrt((2 * l + 1) / (4 * pi) * factorial(l - m) / factorial(l + m))
        p = np.polynomial.polynomial.polyval(y, _legendre_deriv(l, m))
        if m == 0:
            out[..., l] = n_lm * p
        else:
            wm = w ** m
            out[..., l + m] = sqrt(2.0) * n_lm * p * wm.real
            out[..., l - m] = sqrt(2.0) * n_lm * p * wm.imag
    return out


@lru_cache(maxsize=None)
def _fit_points(l):
    """Deterministic points on the unit sphere (Fibonacci lattice), 6l + 6 of them."""
    n = 6 * l + 6
    i = np.arange(n) + 0.5
    yy = 1.0 - 2.0 * i / n
    rho = np.sqrt(1.0 - yy * yy)
    phi = i * pi * (3.0 - sqrt(5.0))
    return np.stack([rho * np.sin(phi), yy, rho * np.cos(phi)], axis=-1)


@lru_cache(maxsize=None)
def _fit_pinv(l):
    a = real_sh(l, _fit_points(l))          # [P, 2l+1]
    return np.linalg.pinv(a)                # [2l+1, P]


def wigner_d(l, R):
    """D^l(R) for rotation matrices R [..., 3, 3]; returns [..., 2l+1, 2l+1].

    Solves D Y^l(p_i) = Y^l(R p_i) over the fit points p_i in the least-squares
    sense (the system is consistent, so this is the exact D up to rounding).
    """
    R = np.asarray(R, dtype=np.float64)
    pts = _fit_points(l)                              # [P, 3]
    rp = np.einsum("...ab,pb->...pa", R, pts)         # [..., P, 3]
    b = real_sh(l, rp)                                # [..., P, 2l+1]
    # a @ D^T = b  =>  D^T = pinv(a) @ b
    dt = np.einsum("kp,...pj->...kj", _fit_pinv(l), b)
    return np.swapaxes(dt, -1, -2)


def edge_frame(vec):
    """Rotation R_e taking the unit edge direction to +y, with zero roll.

    MALOQ Sec. III-C1 / Fig. 3(b,c): every edge is rotated onto the common +y
    axis through Euler angles (alpha, beta, gamma).  Reading: gamma (the roll
    about y) is 0; the layer output does not depend on it.
      r = vec/|vec| = (x, y, z), s = sqrt(x^2 + z^2)
      (cos a, sin a) = (z/s, x/s)  (or (1, 0) when s = 0), cos b = y, sin b = s
      R_e = (R_y(a) R_x(b))^T
    """
    v = np.asarray(vec, dtype=np.float64)
    r = v / np.linalg.norm(v, axis=-1, keepdims=True)
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    s = np.sqrt(x * x + z * z)
    safe = s > 0
    ca = np.where(safe, z / np.where(safe, s, 1.0), 1.0)
    sa = np.where(safe, x / np.where(safe, s, 1.0), 0.0)
    cb, sb = y, s
    one, zero = np.ones_like(x), np.zeros_like(x)
    ry = np.stack([np.stack([ca, zero, sa], -1),
                   np.stack([zero, one, zero], -1),
                   np.stack([-sa, zero, ca], -1)], -2)
    rx = np.stack([np.stack([one, zero, zero], -1),
                   np.stack([zero, cb, -sb], -1),
                   np.stack([zero, sb, cb], -1)], -2)
    return np.swapaxes(ry @ rx, -1, -2)


def wigner_blocks(R, lmax):
    """[D^0(R), ..., D^lmax(R)] for rotations R [..., 3, 3]."""
    return [wigner_d(l, R) for l in range(lmax + 1)]


def rotation_from_euler_zyz(a, b, c):
    """Rz(a) Ry(b) Rz(c) as a 3x3 matrix (used to make test rotations)."""
    def rz(t):
        return np.array([[np.cos(t), -np.sin(t), 0], [np.sin(t), np.cos(t), 0], [0, 0, 1.0]])

    def ry(t):
        return np.array([[np.cos(t), 0, np.sin(t)], [0, 1.0, 0], [-np.sin(t), 0, np.cos(t)]])
    return rz(a) @ ry(b) @ rz(c)


_CG_ROTATIONS = (rotation_from_euler_zyz(0.3, 1.1, 2.0), rotation_from_euler_zyz(1.7, 0.4, -0.9))


@lru_cache(maxsize=None)
def real_coupling(la, lb, L):
    """Real coupling tensor Q[i, j, M] of shape (2la+1, 2lb+1, 2L+1).

    MALOQ Sec. III-B1, Eq. (1): the product la (x) lb decomposes into degrees
    L = |la-lb| .. la+lb through Clebsch-Gordan coefficients.  In the real
    basis above the coefficients of one L form the (unique up to sign)
    intertwiner
        (D^la(R) (x) D^lb(R)) Q = Q D^L(R)     for all R,
    normalised so that sum_ij Q[i,j,M] Q[i,j,M'] = delta_MM'.  Reading (sign):
    the first entry with |Q| > 1e-9 in row-major (i, j, M) order is positive.
    Computed as the null space of the intertwining equations for two generic
    rotations (they generate a dense subgroup of SO(3)).
    """
    if not (abs(la - lb) <= L <= la + lb):
        raise ValueError("triangle rule violated")
    na, nb, nL = 2 * la + 1, 2 * lb + 1, 2 * L + 1
    rows = []
    for R in _CG_ROTATIONS:
        da, db, dL = wigner_d(la, R), wigner_d(lb, R), wigner_d(L, R)
        # vec index (i, j, M) row-major; A vec(Q) = (Da (x) Db (x) I) vec(Q) - (I (x) I (x) DL^T) vec(Q)
        left = np.kron(np.kron(da, db), np.eye(nL))
        right = np.kron(np.eye(na * nb), dL.T)
        rows.append(left - right)
    A = np.concatenate(rows, axis=0)
    _, s, vt = np.linalg.svd(A)
    null = vt[-1]
    if s[-1] > 1e-8 or (len(s) > 1 and s[-2] < 1e-6):
        raise RuntimeError(f"coupling ({la},{lb},{L}) null space not one-dimensional")
    Q = null.reshape(na, nb, nL)
    # normalise: sum_ij Q[:,:,M]^2 = 1 for each M (Schur: all M share one norm)
    Q = Q / np.sqrt(np.sum(Q[:, :, 0] ** 2))
    flat = Q.ravel()
    first = flat[np.argmax(np.abs(flat) > 1e-9)]
    if first < 0:
        Q = -Q
    return Q
