"""Pins of the oracle's real spherical harmonics, Wigner-D, edge frame and CG couplings.

Each check ties the oracle to something outside itself: scipy's complex
spherical harmonics, sympy's Wigner small-d and Clebsch-Gordan routines,
quadrature orthonormality, group identities and closed forms.
"""
import numpy as np
import pytest
from scipy.special import sph_harm_y
from scipy.spatial.transform import Rotation as Rot

from oracle import so3

LMAX = 8   # the degrees the layer is built for go up to 8 (f and g orbital labels)


def _unit(n, seed):
    v = np.random.default_rng(seed).standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def _real_from_complex(l, yc_of_m):
    """Real tesseral harmonics (no Condon-Shortley phase) from complex Y_l^m (with it).

    S_{l,m}  = sqrt(2) (-1)^m Re Y_l^m,   S_{l,-m} = sqrt(2) (-1)^m Im Y_l^m  (m > 0).
    """
    out = [None] * (2 * l + 1)
    out[l] = yc_of_m(0).real
    for m in range(1, l + 1):
        y = yc_of_m(m)
        out[l + m] = np.sqrt(2) * (-1) ** m * y.real
        out[l - m] = np.sqrt(2) * (-1) ** m * y.imag
    return np.stack(out, axis=-1)


@pytest.mark.parametrize("l", range(LMAX + 1))
def test_sh_matches_scipy(l):
    r = _unit(200, l)
    x, y, z = r.T
    theta = np.arccos(np.clip(y, -1, 1))       # polar axis y
    phi = np.arctan2(x, z)                     # azimuth from z towards x
    ref = _real_from_complex(l, lambda m: sph_harm_y(l, m, theta, phi))
    np.testing.assert_allclose(so3.real_sh(l, r), ref, atol=1e-12)


def test_sh_orthonormal_quadrature():
    # Gauss-Legendre in y times a uniform grid in phi: exact for degree <= 2*LMAX
    t, wt = np.polynomial.legendre.leggauss(2 * LMAX + 2)
    nphi = 4 * LMAX + 4
    ph = 2 * np.pi * np.arange(nphi) / nphi
    T, P = np.meshgrid(t, ph, indexing="ij")
    rho = np.sqrt(1 - T ** 2)
    pts = np.stack([rho * np.sin(P), T, rho * np.cos(P)], -1).reshape(-1, 3)
    w = (wt[:, None] * np.full(nphi, 2 * np.pi / nphi)[None, :]).ravel()
    Y = np.concatenate([so3.real_sh(l, pts) for l in range(LMAX + 1)], axis=1)
    G = (Y * w[:, None]).T @ Y
    np.testing.assert_allclose(G, np.eye(Y.shape[1]), atol=1e-12)


def test_sh_degree_one_is_xyz():
    r = _unit(50, 7)
    np.testing.assert_allclose(so3.real_sh(1, r), np.sqrt(3 / (4 * np.pi)) * r, atol=1e-14)


@pytest.mark.parametrize("l", range(LMAX + 1))
def test_sh_addition_theorem(l):
    r = _unit(100, 11 + l)
    np.testing.assert_allclose((so3.real_sh(l, r) ** 2).sum(-1), (2 * l + 1) / (4 * np.pi), atol=1e-12)


def test_sh_pole_is_zonal():
    # at +y only m = 0 survives, with value sqrt((2l+1)/(4 pi))
    for l in range(LMAX + 1):
        v = so3.real_sh(l, np.array([[0.0, 1.0, 0.0]]))[0]
        expect = np.zeros(2 * l + 1)
        expect[l] = np.sqrt((2 * l + 1) / (4 * np.pi))
        np.testing.assert_allclose(v, expect, atol=1e-14)


def test_wigner_group_properties():
    Rs = Rot.random(6, random_state=5).as_matrix()
    for l in range(LMAX + 1):
        D = so3.wigner_d(l, Rs)
        np.testing.assert_allclose(D @ np.swapaxes(D, -1, -2),
                                   np.broadcast_to(np.eye(2 * l + 1), D.shape), atol=1e-12)
        np.testing.assert_allclose(np.linalg.det(D), 1.0, atol=1e-11)
        D01 = so3.wigner_d(l, Rs[0] @ Rs[1])
        np.testing.assert_allclose(D01, D[0] @ D[1], atol=1e-12)
    np.testing.assert_allclose(so3.wigner_d(1, Rs), Rs, atol=1e-13)


def test_wigner_defining_identity_on_fresh_points():
    Rs = Rot.random(4, random_state=9).as_matrix()
    r = _unit(37, 3)
    for l in range(LMAX + 1):
        D = so3.wigner_d(l, Rs)
        lhs = np.einsum("qmn,pn->qpm", D, so3.real_sh(l, r))
        rhs = so3.real_sh(l, np.einsum("qab,pb->qpa", Rs, r))
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def _U(l):
    """Complex -> real change of basis: S = U Y_c (Y_c with the Condon-Shortley phase)."""
    U = np.zeros((2 * l + 1, 2 * l + 1), dtype=complex)
    U[l, l] = 1
    for m in range(1, l + 1):
        U[l + m, l + m] = (-1) ** m / np.sqrt(2)
        U[l + m, l - m] = 1 / np.sqrt(2)
        U[l - m, l + m] = (-1) ** m / (1j * np.sqrt(2))
        U[l - m, l - m] = -1 / (1j * np.sqrt(2))
    return U


@pytest.mark.parametrize("l", range(LMAX + 1))
def test_wigner_matches_sympy_small_d(l):
    """Rotation about x (the Y axis of the z-polar frame (X,Y,Z) = (z,x,y)).

    With U(R) Y_lm = sum_m' Y_lm' d_m'm(beta) for the active rotation about Y,
    Y_lm(R r) = sum_m' d_m'm(-beta) Y_lm'(r) = sum_m' d_mm'(beta) Y_lm'(r),
    so the complex-basis matrix is d(beta) itself and the real one U d U^H.
    """
    import sympy
    from sympy.physics.wigner import wigner_d_small
    beta = 0.7314
    # sympy's d^l_{m m'}(beta), rows and columns m = -l..l (the same matrix as
    # sympy.physics.quantum.spin.Rotation.d, which is minutes slower at l = 8)
    d = np.array(wigner_d_small(l, sympy.Float(beta, 30)).evalf(30).tolist(), dtype=complex)
    assert np.abs(d.imag).max() < 1e-12
    d = d.real
    c, s = np.cos(beta), np.sin(beta)
    Rx = np.array([[1, 0, 0], [0, c, -s], [0, s, c]])
    U = _U(l)
    ref = U @ d @ U.conj().T
    assert np.abs(ref.imag).max() < 1e-12
    np.testing.assert_allclose(so3.wigner_d(l, Rx), ref.real, atol=1e-12)


def test_edge_frame():
    v = np.random.default_rng(4).standard_normal((64, 3)) * 3
    v = np.concatenate([v, [[0, 2.0, 0], [0, -1.5, 0], [1e-3, 0, 0]]])
    R = so3.edge_frame(v)
    r = v / np.linalg.norm(v, axis=1, keepdims=True)
    np.testing.assert_allclose(np.einsum("eab,eb->ea", R, r), np.tile([0, 1.0, 0], (len(v), 1)), atol=1e-13)
    np.testing.assert_allclose(R @ np.swapaxes(R, 1, 2), np.broadcast_to(np.eye(3), R.shape), atol=1e-13)
    np.testing.assert_allclose(np.linalg.det(R), 1.0, atol=1e-13)
    # zero roll: R_e = R_x(-b) R_y(-a), so R_e^T maps the x axis into the plane orthogonal
    # to y... check the explicit construction for one generic edge
    x, y, z = r[0]
    s = np.hypot(x, z)
    a, b = np.arctan2(x, z), np.arctan2(s, y)
    Ry = np.array([[np.cos(a), 0, np.sin(a)], [0, 1, 0], [-np.sin(a), 0, np.cos(a)]])
    Rx = np.array([[1, 0, 0], [0, np.cos(b), -np.sin(b)], [0, np.sin(b), np.cos(b)]])
    np.testing.assert_allclose(R[0], (Ry @ Rx).T, atol=1e-14)


def _cg_real_from_sympy(la, lb, L):
    from sympy.physics.wigner import clebsch_gordan
    C = np.zeros((2 * la + 1, 2 * lb + 1, 2 * L + 1))
    for ma in range(-la, la + 1):
        for mb in range(-lb, lb + 1):
            M = ma + mb
            if abs(M) <= L:
                C[ma + la, mb + lb, M + L] = float(clebsch_gordan(la, lb, L, ma, mb, M))
    Ua, Ub, UL = _U(la), _U(lb), _U(L)
    Q = np.einsum("ia,jb,abM,NM->ijN", Ua, Ub, C, UL.conj())
    k = np.argmax(np.abs(Q).ravel())
    Q = Q / (Q.ravel()[k] / abs(Q.ravel()[k]))
    assert np.abs(Q.imag).max() < 1e-12
    Q = Q.real
    Q /= np.sqrt((Q[:, :, 0] ** 2).sum())
    flat = Q.ravel()
    if flat[np.argmax(np.abs(flat) > 1e-9)] < 0:
        Q = -Q
    return Q


TRIPLES = [(la, lb, L) for la in range(3) for lb in range(3) for L in range(abs(la - lb), la + lb + 1)]


@pytest.mark.parametrize("la,lb,L", TRIPLES)
def test_cg_matches_sympy(la, lb, L):
    np.testing.assert_allclose(so3.real_coupling(la, lb, L), _cg_real_from_sympy(la, lb, L), atol=1e-11)


@pytest.mark.parametrize("la,lb", [(a, b) for a in range(3) for b in range(3)])
def test_cg_transform_orthogonal(la, lb):
    T = np.concatenate([so3.real_coupling(la, lb, L).reshape((2 * la + 1) * (2 * lb + 1), -1)
                        for L in range(abs(la - lb), la + lb + 1)], axis=1)
    np.testing.assert_allclose(T.T @ T, np.eye(T.shape[0]), atol=1e-12)


def test_cg_closed_forms_1x1():
    eps = np.zeros((3, 3, 3))
    for i, j, k, s in [(0, 1, 2, 1), (1, 2, 0, 1), (2, 0, 1, 1), (0, 2, 1, -1), (2, 1, 0, -1), (1, 0, 2, -1)]:
        eps[i, j, k] = s
    np.testing.assert_allclose(so3.real_coupling(1, 1, 0)[:, :, 0], np.eye(3) / np.sqrt(3), atol=1e-13)
    np.testing.assert_allclose(so3.real_coupling(1, 1, 1), eps / np.sqrt(2), atol=1e-13)
    Q2 = so3.real_coupling(1, 1, 2)
    for M in range(5):
        np.testing.assert_allclose(Q2[:, :, M], Q2[:, :, M].T, atol=1e-13)
        assert abs(np.trace(Q2[:, :, M])) < 1e-13


def test_cg_intertwines_at_l4():
    R = Rot.random(random_state=21).as_matrix()
    for (la, lb, L) in [(2, 2, 4), (2, 2, 3), (1, 2, 3), (2, 1, 1)]:
        Q = so3.real_coupling(la, lb, L)
        lhs = np.einsum("ia,jb,abM->ijM", so3.wigner_d(la, R), so3.wigner_d(lb, R), Q)
        rhs = np.einsum("ijN,NM->ijM", Q, so3.wigner_d(L, R))
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)
