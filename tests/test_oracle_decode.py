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


G_SHELLS = (0, 1, 2, 3, 4)      # s p d f g: 25 orbitals, labels up to L = 8 (irreps at lmax 8)


def test_g_shell_label_counts_and_round_trips():
    items, n = decode.label_layout(G_SHELLS)
    # n_L = ordered shell pairs (la, lb) with |la - lb| <= L <= la + lb, counted by hand
    assert n == [5, 12, 16, 17, 15, 10, 6, 3, 1]
    assert sum((2 * L + 1) * c for L, c in enumerate(n)) == 25 * 25
    rng = np.random.default_rng(20)
    H = rng.standard_normal((4, 25, 25))
    np.testing.assert_allclose(decode.label_to_matrix(decode.matrix_to_label(H, G_SHELLS), G_SHELLS), H, atol=1e-12)
    h = [rng.standard_normal((4, 2 * L + 1, c)) for L, c in enumerate(n)]
    for a, b in zip(decode.matrix_to_label(decode.label_to_matrix(h, G_SHELLS), G_SHELLS), h):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_g_g_block_trace_and_ss_entry():
    """The degree-0 part of l (x) l is the identity over 2l + 1: the trace of the
    g-g block (offset 16, 9 x 9) is sqrt(9) = 3 times its L = 0 label, and the s-s
    entry is the first L = 0 label itself."""
    rng = np.random.default_rng(21)
    C = 4
    f = rng.standard_normal((3, 81, C))
    _, n = decode.label_layout(G_SHELLS)
    w = [rng.standard_normal((c, C)) for c in n]
    H = decode.hblocks(f, w, G_SHELLS)
    items, _ = decode.label_layout(G_SHELLS)
    h0 = np.einsum("ec,kc->ek", f[:, 0, :], w[0])
    k_gg = next(k for a, b, L, k in items if (a, b, L) == (4, 4, 0))
    blk = H[:, 16:25, 16:25]
    np.testing.assert_allclose(np.trace(blk, axis1=1, axis2=2), 3.0 * h0[:, k_gg], atol=1e-12)
    np.testing.assert_allclose(H[:, 0, 0], h0[:, 0], atol=1e-13)


def test_g_shell_blocks_covariant():
    """s p d f g blocks from lmax-8 irreps transform as D^{la} H D^{lb}^T."""
    rng = np.random.default_rng(22)
    C = 3
    f = rng.standard_normal((4, 81, C))
    _, n = decode.label_layout(G_SHELLS)
    w = [rng.standard_normal((c, C)) for c in n]
    Q = Rot.random(random_state=23).as_matrix()
    fr = np.empty_like(f)
    for l in range(9):
        sl = slice(l * l, (l + 1) ** 2)
        fr[:, sl, :] = np.einsum("mn,enc->emc", so3.wigner_d(l, Q), f[:, sl, :])
    off, n_orb = decode.orbital_offsets(G_SHELLS)
    Dorb = np.zeros((n_orb, n_orb))
    for o, l in zip(off, G_SHELLS):
        Dorb[o:o + 2 * l + 1, o:o + 2 * l + 1] = so3.wigner_d(l, Q)
    np.testing.assert_allclose(decode.hblocks(fr, w, G_SHELLS), Dorb @ decode.hblocks(f, w, G_SHELLS) @ Dorb.T,
                               atol=1e-10)


def _periodic_graph_and_blocks(seed=30, n_orb=13):
    import synth
    from oracle import neighbors
    s = synth.make_structure("tiny")
    g = neighbors.build_graph(s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut)
    dst = neighbors.dst_of_edges(g["row_ptr"])
    rng = np.random.default_rng(seed)
    he = rng.standard_normal((len(g["src"]), n_orb, n_orb))
    hn = rng.standard_normal((s.n_dst, n_orb, n_orb))
    return s, g, dst, he, hn


def test_bsr_assembly_equals_dense_images():
    """Every image's dense matrix H(S) (blocks placed by hand: edge (s -> d, S)
    at rows of s and columns of d, on-site blocks on the S = 0 diagonal) equals
    the BSR expanded image by image; rows are sorted and every block is kept once."""
    s, g, dst, he, hn = _periodic_graph_and_blocks()
    n = he.shape[1]
    rp, col, sh, val = decode.assemble_bsr(g["src"], dst, g["shift"], he, hn, s.n_src)
    assert rp[-1] == len(g["src"]) + s.n_dst == len(col)
    keys = {tuple(k) for k in np.unique(g["shift"].astype(np.int64), axis=0)} | {(0, 0, 0)}
    N = s.n_src * n
    for S in keys:
        dense = np.zeros((N, N))
        for e in range(len(g["src"])):
            if tuple(g["shift"][e]) == S:
                a, b = g["src"][e] * n, dst[e] * n
                dense[a:a + n, b:b + n] += he[e]
        if S == (0, 0, 0):
            for i in range(s.n_dst):
                dense[i * n:(i + 1) * n, i * n:(i + 1) * n] += hn[i]
        got = np.zeros((N, N))
        for i in range(s.n_src):
            for b in range(rp[i], rp[i + 1]):
                if tuple(int(v) for v in sh[b]) == S:
                    got[i * n:(i + 1) * n, col[b] * n:(col[b] + 1) * n] += val[b]
        np.testing.assert_array_equal(got, dense)
    for i in range(s.n_src):
        k = [(int(col[b]),) + tuple(int(v) for v in sh[b]) for b in range(rp[i], rp[i + 1])]
        assert k == sorted(k) and len(set(k)) == len(k)


def test_bsr_bloch_sum_hermitian_for_symmetric_pairs():
    """Blocks built as f(|r|) B(Z_s, Z_d) with B(Z_d, Z_s) = B(Z_s, Z_d)^T and
    symmetric on-site blocks: the Bloch sum H(k) = sum_S H(S) exp(2 pi i k.S)
    of the assembled matrix is Hermitian at every k (the reverse edge
    (d -> s, -S) carries the transposed block)."""
    import synth
    s, g, dst, _, _ = _periodic_graph_and_blocks()
    species = synth.make_structure("tiny").species
    n = 4
    rng = np.random.default_rng(31)
    B = rng.standard_normal((2, 2, n, n))
    B[1, 0] = B[0, 1].T
    B[0, 0] = B[0, 0] + B[0, 0].T
    B[1, 1] = B[1, 1] + B[1, 1].T
    d = np.asarray(g["dist"], np.float64)
    he = np.exp(-d)[:, None, None] * B[species[g["src"]], species[dst]]
    hn = np.stack([B[species[i], species[i]] for i in range(s.n_dst)])
    rp, col, sh, val = decode.assemble_bsr(g["src"], dst, g["shift"], he, hn, s.n_src)
    for k in rng.uniform(-0.5, 0.5, (3, 3)):
        H = np.zeros((s.n_src * n, s.n_src * n), complex)
        for i in range(s.n_src):
            for b in range(rp[i], rp[i + 1]):
                ph = np.exp(2j * np.pi * float(k @ sh[b].astype(np.float64)))
                H[i * n:(i + 1) * n, col[b] * n:(col[b] + 1) * n] += ph * val[b]
        np.testing.assert_allclose(H, H.conj().T, atol=1e-12)
        assert np.abs(H.imag).max() > 1e-3
