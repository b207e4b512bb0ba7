"""Pins of Matrix <-> Label over whole matrices with per-element bases.

Closed forms on the pages' toy water example (minimal basis, Fig. 2(b) of
MALOQ), round trips and norm conservation (T of Eq. (1) is orthogonal),
covariance under a rotation of each molecule, the padding of absent shells,
and agreement with direct slicing when every element carries every shell.
"""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation as Rot

import synth
from oracle import decode, labels, so3


def _edges(batch):
    return batch.src.astype(np.int64), batch.dst().astype(np.int64)


def _water():
    mol_ptr = np.array([0, 3])
    species = np.array([0, 1, 1])               # O, H, H
    sh, masks = synth.WATER_SHELLS, synth.WATER_MASKS
    lay = labels.orbital_layout(mol_ptr, species, sh, masks)
    src = np.array([1, 2, 0, 2, 0, 1])          # destination-sorted, fully connected
    dst = np.array([0, 0, 1, 1, 2, 2])
    return mol_ptr, species, sh, masks, lay, src, dst


def test_water_layout():
    _, _, sh, masks, lay, _, _ = _water()
    atom_orb, atom_mol, mol_norb, mat_off = lay
    assert list(atom_orb) == [0, 4, 5]          # O: s p (4 orbitals), then H s, H s
    assert list(atom_mol) == [0, 0, 0]
    assert list(mol_norb) == [6] and list(mat_off) == [0, 36]
    _, n = decode.label_layout(sh)
    assert n == [2, 3, 1] and sum((2 * L + 1) * c for L, c in enumerate(n)) == 16


def test_water_closed_forms():
    """s-s labels are the entry itself, s-p labels the p row/column in m order,
    the p-p L = 0 label the trace over sqrt(3), and absent shells give zeros."""
    mol_ptr, species, sh, masks, lay, src, dst = _water()
    rng = np.random.default_rng(5)
    H = rng.standard_normal((6, 6))
    he, hn = labels.matrix_to_labels(H.ravel(), src, dst, None, species, lay, sh, masks)
    # label index q = hoff[L] + (M + L) * n_L + k with n = [2, 3, 1], hoff = [0, 2, 11]
    q = lambda L, M, k: [0, 2, 11][L] + (M + L) * [2, 3, 1][L] + k
    O = hn[0]
    assert np.isclose(O[q(0, 0, 0)], H[0, 0])
    for M in (-1, 0, 1):
        assert np.isclose(O[q(1, M, 0)], H[0, 2 + M])      # pair (s, p): row s, p columns
        assert np.isclose(O[q(1, M, 1)], H[2 + M, 0])      # pair (p, s)
    P = H[1:4, 1:4]
    assert np.isclose(O[q(0, 0, 1)], np.trace(P) / np.sqrt(3))
    A = 0.5 * (P - P.T)
    S = 0.5 * (P + P.T) - np.trace(P) / 3 * np.eye(3)
    assert np.isclose(sum(O[q(1, M, 2)] ** 2 for M in (-1, 0, 1)), np.sum(A * A))
    assert np.isclose(sum(O[q(2, M, 0)] ** 2 for M in range(-2, 3)), np.sum(S * S))
    # H on-site: one s-s label, zeros elsewhere
    for a, row in ((1, 4), (2, 5)):
        assert np.isclose(hn[a][0], H[row, row]) and np.all(hn[a][1:] == 0)
    # edge H1 -> O (e = 0): rows = H1's s orbital, columns = O's s, p
    e = he[0]
    assert np.isclose(e[q(0, 0, 0)], H[4, 0])
    for M in (-1, 0, 1):
        assert np.isclose(e[q(1, M, 0)], H[4, 2 + M])
    nz = {q(0, 0, 0)} | {q(1, M, 0) for M in (-1, 0, 1)}
    assert all(e[i] == 0 for i in range(16) if i not in nz)
    # edge O -> H1 (e = 2): rows = O's s, p, column = H1's s
    e = he[2]
    assert np.isclose(e[q(0, 0, 0)], H[0, 4])
    for M in (-1, 0, 1):
        assert np.isclose(e[q(1, M, 1)], H[2 + M, 4])
    # edge H2 -> H1 (e = 3): the one s-s label
    assert np.isclose(he[3][0], H[5, 4]) and np.all(he[3][1:] == 0)
    # a fully connected graph covers every block: Label -> Matrix gives H back
    H2 = labels.labels_to_matrix(he, hn, src, dst, None, species, lay, sh, masks)
    np.testing.assert_allclose(H2, H.ravel(), atol=1e-13)


def _svp_batch(seed=3, n_mols=4, keep=1.0):
    b = synth.make_molecule_batch(seed, n_mols, 3, 9, keep=keep)
    lay = labels.orbital_layout(b.mol_ptr, b.species, synth.SVP_SHELLS, synth.SVP_MASKS)
    return b, lay


def test_svp_counts():
    _, n_orb = labels.species_templates(synth.SVP_SHELLS, synth.SVP_MASKS)
    assert list(n_orb[:-1]) == [5, 14, 14, 14, 14, 18, 18] and n_orb[-1] == 0
    _, n = decode.label_layout(synth.SVP_SHELLS)
    assert sum((2 * L + 1) * c for L, c in enumerate(n)) == 18 * 18
    assert len(n) == 5                          # labels up to L = 4 (d x d)


def test_round_trips_and_norm():
    b, lay = _svp_batch()
    sh, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    src, dst = _edges(b)
    H = synth.make_matrix_values(3, lay[3][-1]).astype(np.float64)
    he, hn = labels.matrix_to_labels(H, src, dst, None, b.species, lay, sh, masks)
    # T is orthogonal and a fully connected graph covers each entry once
    assert np.isclose(np.sum(he * he) + np.sum(hn * hn), np.sum(H * H), rtol=1e-12)
    np.testing.assert_allclose(labels.labels_to_matrix(he, hn, src, dst, None, b.species, lay, sh, masks), H,
                               atol=1e-12)
    # Label -> Matrix -> Label keeps every present label and zeroes the padding
    g = synth.make_label_values(4, len(src), he.shape[1]).astype(np.float64)
    gn = synth.make_label_values(5, b.n_atoms, he.shape[1]).astype(np.float64)
    H3 = labels.labels_to_matrix(g, gn, src, dst, None, b.species, lay, sh, masks)
    ge, gn2 = labels.matrix_to_labels(H3, src, dst, None, b.species, lay, sh, masks)
    pad_e = (he == 0)                           # labels of absent shell pairs (exact zeros)
    np.testing.assert_allclose(ge[~pad_e], g[~pad_e], atol=1e-12)
    assert np.all(ge[pad_e] == 0)
    np.testing.assert_allclose(gn2[hn != 0], gn[hn != 0], atol=1e-12)


def test_padding_follows_species():
    """A label is padding exactly when its shell pair is missing from (Z_i, Z_j)."""
    b, lay = _svp_batch(seed=6)
    sh, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    src, dst = _edges(b)
    H = synth.make_matrix_values(6, lay[3][-1]).astype(np.float64)
    he, _ = labels.matrix_to_labels(H, src, dst, None, b.species, lay, sh, masks)
    items, n = decode.label_layout(sh)
    hoff = np.concatenate([[0], np.cumsum([(2 * L + 1) * c for L, c in enumerate(n)])])
    for e in range(len(src)):
        mi, mj = masks[b.species[src[e]]], masks[b.species[dst[e]]]
        for a, bb, L, k in items:
            present = (mi >> a) & 1 and (mj >> bb) & 1
            vals = he[e, [hoff[L] + (M + L) * n[L] + k for M in range(-L, L + 1)]]
            assert np.any(vals != 0) if present else np.all(vals == 0)


def test_uniform_basis_is_direct_slicing():
    """Every element with every shell: labels are Eq. (1) on the plain N_orb x N_orb slices."""
    b = synth.make_molecule_batch(7, 3, 2, 5)
    sh = decode.SHELL_L
    masks = (0b11111,) * 3
    species = np.asarray(b.species) % 3
    lay = labels.orbital_layout(b.mol_ptr, species, sh, masks)
    src, dst = _edges(b)
    H = synth.make_matrix_values(7, lay[3][-1]).astype(np.float64)
    he, hn = labels.matrix_to_labels(H, src, dst, None, species, lay, sh, masks)
    blocks = []
    for s, d in zip(src, dst):
        m = b.mol_ptr.searchsorted(d, side="right") - 1
        n_b = 13 * (b.mol_ptr[m + 1] - b.mol_ptr[m])
        Hm = H[lay[3][m]:lay[3][m + 1]].reshape(n_b, n_b)
        i, j = 13 * (s - b.mol_ptr[m]), 13 * (d - b.mol_ptr[m])
        blocks.append(Hm[i:i + 13, j:j + 13])
    ref = labels.flat_labels(decode.matrix_to_label(np.array(blocks)))
    np.testing.assert_allclose(he, ref, atol=1e-13)


def _g_batch(seed, n_mols=2):
    b = synth.make_molecule_batch(seed, n_mols, 2, 6, fractions=synth.G_FRACTIONS)
    return b, labels.orbital_layout(b.mol_ptr, b.species, synth.G_SHELLS, synth.G_MASKS)


def test_g_shell_counts_round_trips_and_norm():
    """s p d f g full list (labels up to L = 8): 5 / 9 / 25 orbitals per element,
    625 labels per block, T orthogonal (norm kept, both round trips)."""
    _, n_orb = labels.species_templates(synth.G_SHELLS, synth.G_MASKS)
    assert list(n_orb[:-1]) == [4, 9, 25]
    b, lay = _g_batch(9, 3)
    sh, masks = synth.G_SHELLS, synth.G_MASKS
    src, dst = _edges(b)
    H = synth.make_matrix_values(9, lay[3][-1]).astype(np.float64)
    he, hn = labels.matrix_to_labels(H, src, dst, None, b.species, lay, sh, masks)
    assert he.shape[1] == 625
    assert np.isclose(np.sum(he * he) + np.sum(hn * hn), np.sum(H * H), rtol=1e-12)
    np.testing.assert_allclose(labels.labels_to_matrix(he, hn, src, dst, None, b.species, lay, sh, masks), H,
                               atol=1e-12)


@pytest.mark.parametrize("basis", ["svp", "g"])
def test_labels_covariant(basis):
    """Rotating a molecule's orbitals (H -> D H D^T, D block-diagonal per atom's
    own shells) rotates every label's degree-L part by D^L (def2-SVP-like
    shells, and the s p d f g list with labels up to L = 8)."""
    if basis == "svp":
        b, lay = _svp_batch(seed=8, n_mols=2)
        sh, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    else:
        b, lay = _g_batch(10, 2)
        sh, masks = synth.G_SHELLS, synth.G_MASKS
    src, dst = _edges(b)
    atom_orb, atom_mol, mol_norb, mat_off = lay
    H = synth.make_matrix_values(8, mat_off[-1]).astype(np.float64)
    Hr = H.copy()
    Rs = [Rot.random(random_state=20 + m).as_matrix() for m in range(b.n_mols)]
    for m in range(b.n_mols):
        n_b = mol_norb[m]
        D = np.zeros((n_b, n_b))
        for a in range(b.mol_ptr[m], b.mol_ptr[m + 1]):
            o = atom_orb[a]
            for s_, l in enumerate(sh):
                if (masks[b.species[a]] >> s_) & 1:
                    D[o:o + 2 * l + 1, o:o + 2 * l + 1] = so3.wigner_d(l, Rs[m])
                    o += 2 * l + 1
        Hm = H[mat_off[m]:mat_off[m + 1]].reshape(n_b, n_b)
        Hr[mat_off[m]:mat_off[m + 1]] = (D @ Hm @ D.T).ravel()
    he, hn = labels.matrix_to_labels(H, src, dst, None, b.species, lay, sh, masks)
    he_r, hn_r = labels.matrix_to_labels(Hr, src, dst, None, b.species, lay, sh, masks)
    mol_e = atom_mol[dst]
    for rows, rows_r, mol in ((he, he_r, mol_e), (hn, hn_r, atom_mol)):
        h = labels.unflat_labels(rows, sh)
        hr = labels.unflat_labels(rows_r, sh)
        for L in range(len(h)):
            for m in range(b.n_mols):
                sel = mol == m
                DL = so3.wigner_d(L, Rs[m])
                np.testing.assert_allclose(hr[L][sel], np.einsum("MN,eNk->eMk", DL, h[L][sel]), atol=1e-11)


def test_skipped_edges_and_partial_graphs():
    """Edges across structures or with an image shift have no block; a partial
    graph writes only its own blocks."""
    b, lay = _svp_batch(seed=9, n_mols=3, keep=0.6)
    sh, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    src, dst = _edges(b)
    H = synth.make_matrix_values(9, lay[3][-1]).astype(np.float64)
    # one edge into atom 0 from the last molecule, one with a shift
    src2 = np.concatenate([[b.n_atoms - 1], src])
    dst2 = np.concatenate([[0], dst])
    shift = np.zeros((len(src2), 3), np.int8)
    shift[1, 2] = 1
    he, hn = labels.matrix_to_labels(H, src2, dst2, shift, b.species, lay, sh, masks)
    assert np.all(he[0] == 0) and np.all(he[1] == 0)
    he_ref, _ = labels.matrix_to_labels(H, src, dst, None, b.species, lay, sh, masks)
    np.testing.assert_array_equal(he[2:], np.where(shift[2:, :1] == 0, he_ref[1:], 0))
    H2 = labels.labels_to_matrix(he, hn, src2, dst2, shift, b.species, lay, sh, masks)
    # covered entries come back, the rest stay zero
    covered = np.zeros(H.shape, bool)
    covered[labels.labels_to_matrix(np.ones_like(he), np.ones_like(hn), src2, dst2, shift, b.species, lay, sh,
                                    masks) != 0] = True
    np.testing.assert_allclose(H2[covered], H[covered], atol=1e-12)
    assert np.all(H2[~covered] == 0)
    assert covered.sum() < H.size               # keep = 0.6 leaves blocks out


def test_out_of_range_species_carries_nothing():
    sh, masks = synth.WATER_SHELLS, synth.WATER_MASKS
    mol_ptr = np.array([0, 3])
    species = np.array([0, 7, 1])               # 7 is not an element of the table
    atom_orb, atom_mol, mol_norb, mat_off = labels.orbital_layout(mol_ptr, species, sh, masks)
    assert list(atom_orb) == [0, 4, 4] and list(mol_norb) == [5]


def test_no_edges():
    _, species, sh, masks, lay, _, _ = _water()
    H = np.arange(36, dtype=np.float64)
    he, hn = labels.matrix_to_labels(H, np.zeros(0, np.int64), np.zeros(0, np.int64), None, species, lay, sh, masks)
    assert he.shape == (0, 16) and hn.shape == (3, 16)
    H2 = labels.labels_to_matrix(he, hn, np.zeros(0, np.int64), np.zeros(0, np.int64), None, species, lay, sh, masks)
    # only the on-site blocks come back
    Hm = H.reshape(6, 6)
    ref = np.zeros((6, 6))
    ref[:4, :4], ref[4, 4], ref[5, 5] = Hm[:4, :4], Hm[4, 4], Hm[5, 5]
    np.testing.assert_allclose(H2.reshape(6, 6), ref, atol=1e-12)
