"""Pins of the Label -> Matrix decode: label counts, round trips, closed forms, covariance."""
import numpy as np
from scipy.spatial.transform import Rotation as Rot

from oracle import decode, so3


def test_label_counts():
    items, n = decode.label_layout()
    assert n == [9, 17, 13, 5, 1]
    assert sum((2 * L + 1) * c for L, c in enumerate(n)) == 13 * 13
    assert decode.orbital_offsets() == ([0, 1, 2, 5, 8], 13)
    # the 8,064-atom GST cell with 13 orbitals per atom
    assert 8064 * decode.orbital_offsets()[1] == 104832


def test_round_trips():
    rng = np.random.default_rng(0)
    H = rng.standard_normal((7, 13, 13))
    np.testing.assert_allclose(decode.label_to_matrix(decode.matrix_to_label(H)), H, atol=1e-12)
    _, n = decode.label_layout()
    h = [rng.standard_normal((7, 2 * L + 1, c)) for L, c in enumerate(n)]
    for a, b in zip(decode.matrix_to_label(decode.label_to_matrix(h)), h):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_ss_block_and_pp_trace():
    rng = np.random.default_rng(1)
    C = 5
    f = rng.standard_normal((3, 25, C))
    _, n = decode.label_layout()
    w = [rng.standard_normal((c, C)) for c in n]
    H = decode.hblocks(f, w)
    h0 = np.einsum("ec,kc->ek", f[:, 0, :], w[0])
    # s-s blocks (shells 0,1 x 0,1) are the L=0 labels k = 0..3 (Q^{000} = 1)
    np.testing.assert_allclose(H[:, 0, 0], h0[:, 0], atol=1e-13)
    np.testing.assert_allclose(H[:, 0, 1], h0[:, 1], atol=1e-13)
    np.testing.assert_allclose(H[:, 1, 0], h0[:, 2], atol=1e-13)
    np.testing.assert_allclose(H[:, 1, 1], h0[:, 3], atol=1e-13)
    # the p-p block of shells (2,2) is h0 I/sqrt(3) + antisymmetric (L=1) + traceless symmetric (L=2)
    items, _ = decode.label_layout()
    k0 = next(k for a, b, L, k in items if (a, b, L) == (2, 2, 0))
    blk = H[:, 2:5, 2:5]
    np.testing.assert_allclose(np.trace(blk, axis1=1, axis2=2), np.sqrt(3) * h0[:, k0], atol=1e-12)


def test_hamiltonian_blocks_covariant():
    """H^{ab} transforms as D^{la} H D^{lb}^T when the irreps rotate (Eq. (1) is equivariant)."""
    rng = np.random.default_rng(2)
    C = 4
    f = rng.standard_normal((5, 25, C))
    _, n = decode.label_layout()
    w = [rng.standard_normal((c, C)) for c in n]
    Q = Rot.random(random_state=3).as_matrix()
    fr = np.empty_like(f)
    for l in range(5):
        sl = slice(l * l, (l + 1) ** 2)
        fr[:, sl, :] = np.einsum("mn,enc->emc", so3.wigner_d(l, Q), f[:, sl, :])
    Dorb = np.zeros((13, 13))
    off, _ = decode.orbital_offsets()
    for o, l in zip(off, decode.SHELL_L):
        Dorb[o:o + 2 * l + 1, o:o + 2 * l + 1] = so3.wigner_d(l, Q)
    np.testing.assert_allclose(decode.hblocks(fr, w), Dorb @ decode.hblocks(f, w) @ Dorb.T, atol=1e-12)


def test_f_shell_blocks_covariant():
    """With f shells (s s p p d f: 20 orbitals, labels up to L = 6, irreps at
    lmax 6) the blocks still transform as D^{la} H D^{lb}^T."""
    shells = (0, 0, 1, 1, 2, 3)
    rng = np.random.default_rng(12)
    C = 3
    f = rng.standard_normal((4, 49, C))
    _, n = decode.label_layout(shells)
    assert sum((2 * L + 1) * c for L, c in enumerate(n)) == 20 * 20 and len(n) == 7
    w = [rng.standard_normal((c, C)) for c in n]
    Q = Rot.random(random_state=13).as_matrix()
    fr = np.empty_like(f)
    for l in range(7):
        sl = slice(l * l, (l + 1) ** 2)
        fr[:, sl, :] = np.einsum("mn,enc->emc", so3.wigner_d(l, Q), f[:, sl, :])
    off, n_orb = decode.orbital_offsets(shells)
    Dorb = np.zeros((n_orb, n_orb))
    for o, l in zip(off, shells):
        Dorb[o:o + 2 * l + 1, o:o + 2 * l + 1] = so3.wigner_d(l, Q)
    np.testing.assert_allclose(decode.hblocks(fr, w, shells), Dorb @ decode.hblocks(f, w, shells) @ Dorb.T,
                               atol=1e-11)
