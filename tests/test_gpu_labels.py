"""Matrix <-> Label on the GPU vs the fp64 oracle, through the C ABI (needs an MI355X).

Layouts and skip counts are compared exactly.  Labels and matrix entries are
fp32 sums of a few CG terms of fp32 values (at most 2 min(la, lb) + 1 terms
per label or entry), so each carries a few fp32 roundings of sum |c h|: the
bar is 1e-5 normwise relative and max-abs <= 1e-5 * max|ref|.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import labels as olab
from tests.helpers import assert_close, sample_rows

pytestmark = pytest.mark.gpu

eg = pytest.importorskip("equivariant_gnn_electronic_amd")

TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _setup(batch, shells, masks, dev, shift=None, src=None, row_ptr=None, group=False):
    """Basis, layout and graph; group=True gives the graph its source grouping,
    so the kernels take the blocks one source atom at a time."""
    basis = eg.Basis(shells, masks)
    mol_ptr = _t(batch.mol_ptr.astype(np.int32), dev)
    species = _t(batch.species.astype(np.int32), dev)
    orb, bad = eg.egnn_orbital_layout(basis, mol_ptr, species)
    rp = batch.row_ptr if row_ptr is None else row_ptr
    sr = batch.src if src is None else src
    g = eg.Graph.from_csr(_t(rp.astype(np.int32), dev), _t(sr.astype(np.int32), dev),
                          shift=None if shift is None else _t(shift.astype(np.int8), dev), group=group)
    return basis, orb, bad, g


ORDERS = {"by_dst": False, "by_src": True}


def _check_layout(orb, batch, shells, masks):
    ref = olab.orbital_layout(batch.mol_ptr, batch.species, shells, masks)
    for got, want, what in zip((orb.atom_orb, orb.atom_mol, orb.mol_norb, orb.mat_off), ref,
                               ("atom_orb", "atom_mol", "mol_norb", "mat_off")):
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=what)
    return ref


def _dst(row_ptr):
    return np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))


CASES = {
    # the pages' toy example: water in a minimal basis (O: s p, H: s)
    "water": (lambda: synth.MoleculeBatch(np.array([0, 3], np.int32), np.array([0, 1, 1], np.int32),
                                           np.array([0, 2, 4, 6], np.int32),
                                           np.array([1, 2, 0, 2, 0, 1], np.int32)),
              synth.WATER_SHELLS, synth.WATER_MASKS),
    # def2-SVP-like shells over H, C, N, O, F, S, Cl; fully connected molecules
    "svp": (lambda: synth.make_molecule_batch(21, 40, 1, 24), synth.SVP_SHELLS, synth.SVP_MASKS),
    # a partial graph (each edge kept with probability 0.6)
    "svp_partial": (lambda: synth.make_molecule_batch(22, 30, 2, 20, keep=0.6), synth.SVP_SHELLS, synth.SVP_MASKS),
    # f shells (labels up to L = 6): full list s s p p d f, three elements
    "spdf": (lambda: synth.make_molecule_batch(23, 12, 1, 9, fractions=(0.4, 0.3, 0.3)),
             (0, 0, 1, 1, 2, 3), (0b000101, 0b010111, 0b111111)),
    # g shells (labels up to L = 8): full list s p d f g, three elements
    "spdfg": (lambda: synth.make_molecule_batch(25, 12, 1, 8, fractions=synth.G_FRACTIONS),
              synth.G_SHELLS, synth.G_MASKS),
}


@pytest.mark.parametrize("order", list(ORDERS))
@pytest.mark.parametrize("case", list(CASES))
def test_matrix_to_label_and_back(dev, case, order):
    make, shells, masks = CASES[case]
    batch = make()
    print(f"[labels] case={case} order={order} atoms={batch.n_atoms} edges={batch.n_edges}", flush=True)
    basis, orb, bad, g = _setup(batch, shells, masks, dev, group=ORDERS[order])
    lay = _check_layout(orb, batch, shells, masks)
    assert int(bad.item()) == 0
    n = int(lay[3][-1])
    H = synth.make_matrix_values(31, n)
    he, hn, skipped = eg.egnn_matrix_to_label(basis, orb, g, _t(H, dev))
    src, dst = batch.src.astype(np.int64), batch.dst().astype(np.int64)
    ref_e, ref_n = olab.matrix_to_labels(H, src, dst, None, batch.species, lay, shells, masks)
    assert int(skipped.item()) == 0
    assert he.shape == ref_e.shape and hn.shape == ref_n.shape
    assert_close(he.cpu().numpy(), ref_e, TOL, "h_edge")
    assert_close(hn.cpu().numpy(), ref_n, TOL, "h_node")
    # padding is exactly zero
    assert np.all(he.cpu().numpy()[ref_e == 0] == 0)
    # Label -> Matrix from independent labels into a zeroed matrix
    le = synth.make_label_values(32, batch.n_edges, ref_e.shape[1])
    ln = synth.make_label_values(33, batch.n_atoms, ref_e.shape[1])
    Hg, skipped = eg.egnn_label_to_matrix(basis, orb, g, _t(le, dev), _t(ln, dev))
    Href = olab.labels_to_matrix(le, ln, src, dst, None, batch.species, lay, shells, masks)
    assert int(skipped.item()) == 0
    assert_close(Hg.cpu().numpy(), Href, TOL, "H")
    assert np.all(Hg.cpu().numpy()[Href == 0] == 0)     # entries of missing blocks untouched


def test_nodes_only_and_edges_only(dev):
    batch = synth.make_molecule_batch(24, 10, 2, 12)
    shells, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    basis, orb, _, g = _setup(batch, shells, masks, dev)
    lay = olab.orbital_layout(batch.mol_ptr, batch.species, shells, masks)
    H = synth.make_matrix_values(34, lay[3][-1])
    ref_e, ref_n = olab.matrix_to_labels(H, batch.src, batch.dst(), None, batch.species, lay, shells, masks)
    he, hn, _ = eg.egnn_matrix_to_label(basis, orb, g, _t(H, dev), edges=False)
    assert he.shape[0] == 0
    assert_close(hn.cpu().numpy(), ref_n, TOL, "h_node")
    he, hn, _ = eg.egnn_matrix_to_label(basis, orb, g, _t(H, dev), nodes=False)
    assert hn is None
    assert_close(he.cpu().numpy(), ref_e, TOL, "h_edge")
    # on-site blocks only back into a zero matrix
    Hg, _ = eg.egnn_label_to_matrix(basis, orb, None, None, _t(ref_n.astype(np.float32), dev))
    Href = olab.labels_to_matrix(np.zeros((0, ref_n.shape[1])), ref_n.astype(np.float32), np.zeros(0, np.int64),
                                 np.zeros(0, np.int64), None, batch.species, lay, shells, masks)
    assert_close(Hg.cpu().numpy(), Href, TOL, "H on-site")


@pytest.mark.parametrize("order", list(ORDERS))
def test_skipped_edges(dev, order):
    """Edges across structures and edges with an image shift have no block."""
    batch = synth.make_molecule_batch(25, 6, 2, 8)
    shells, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    # prepend into row 0 an edge from the batch's last atom (another molecule)
    src = np.concatenate([[batch.n_atoms - 1], batch.src]).astype(np.int32)
    row_ptr = batch.row_ptr.copy()
    row_ptr[1:] += 1
    shift = np.zeros((len(src), 3), np.int8)
    shift[2, 0] = -1                                  # and shift an ordinary edge
    basis, orb, _, g = _setup(batch, shells, masks, dev, shift=shift, src=src, row_ptr=row_ptr,
                              group=ORDERS[order])
    lay = olab.orbital_layout(batch.mol_ptr, batch.species, shells, masks)
    H = synth.make_matrix_values(35, lay[3][-1])
    dst = _dst(row_ptr)
    he, hn, skipped = eg.egnn_matrix_to_label(basis, orb, g, _t(H, dev))
    ref_e, ref_n = olab.matrix_to_labels(H, src, dst, shift, batch.species, lay, shells, masks)
    assert int(skipped.item()) == 2
    assert_close(he.cpu().numpy(), ref_e, TOL, "h_edge")
    assert np.all(he[:1].cpu().numpy() == 0) and np.all(he[2].cpu().numpy() == 0)
    Hg, skipped = eg.egnn_label_to_matrix(basis, orb, g, he, hn)
    assert int(skipped.item()) == 2
    Href = olab.labels_to_matrix(ref_e, ref_n, src, dst, shift, batch.species, lay, shells, masks)
    assert_close(Hg.cpu().numpy(), Href, TOL, "H")


def test_degenerate_layouts(dev):
    """Empty structures, an element index outside the table and an empty batch."""
    shells, masks = synth.WATER_SHELLS, synth.WATER_MASKS
    mol_ptr = np.array([0, 0, 3, 3, 5], np.int32)          # two empty molecules
    species = np.array([0, 1, 9, 1, 0], np.int32)          # 9 is not an element
    batch = synth.MoleculeBatch(mol_ptr, species, np.array([0, 0, 0, 0, 0, 0], np.int32), np.zeros(0, np.int32))
    basis, orb, bad, g = _setup(batch, shells, masks, dev)
    lay = _check_layout(orb, batch, shells, masks)
    assert int(bad.item()) == 1
    H = synth.make_matrix_values(36, lay[3][-1])
    he, hn, skipped = eg.egnn_matrix_to_label(basis, orb, g, _t(H, dev))
    _, ref_n = olab.matrix_to_labels(H, np.zeros(0, np.int64), np.zeros(0, np.int64), None, species, lay, shells,
                                     masks)
    assert he.shape[0] == 0 and int(skipped.item()) == 0
    assert_close(hn.cpu().numpy(), ref_n, TOL, "h_node")
    assert np.all(hn[2].cpu().numpy() == 0)
    # no atoms at all
    empty = synth.MoleculeBatch(np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(1, np.int32),
                                np.zeros(0, np.int32))
    basis, orb, bad, g = _setup(empty, shells, masks, dev)
    assert int(orb.mat_off[0].item()) == 0 and int(bad.item()) == 0
    he, hn, skipped = eg.egnn_matrix_to_label(basis, orb, g, torch.zeros(1, device=dev))
    assert he.shape[0] == 0 and hn.shape[0] == 0 and int(skipped.item()) == 0


def test_invalid_structure_range_is_counted(dev):
    shells, masks = synth.WATER_SHELLS, synth.WATER_MASKS
    basis = eg.Basis(shells, masks)
    mol_ptr = _t(np.array([0, 2, 1, 3], np.int32), dev)     # structure 1 runs backwards
    species = _t(np.array([0, 1, 1], np.int32), dev)
    orb, bad = eg.egnn_orbital_layout(basis, mol_ptr, species)
    assert int(bad.item()) == 1
    assert orb.mol_norb.cpu().numpy()[1] == 0


@pytest.mark.parametrize("order", list(ORDERS))
def test_bench_batch_sampled(dev, order):
    """The benchmark's batch (4,096 molecules of 10-50 atoms, fully connected):
    the whole layout exactly, and sampled label rows and matrix entries
    against the oracle run on those rows only."""
    batch = synth.make_molecule_batch(40, 4096, 10, 50)
    shells, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    print(f"[labels] bench batch order={order} atoms={batch.n_atoms} edges={batch.n_edges}", flush=True)
    basis, orb, bad, g = _setup(batch, shells, masks, dev, group=ORDERS[order])
    lay = _check_layout(orb, batch, shells, masks)
    H = synth.make_matrix_values(41, lay[3][-1])
    Hd = _t(H, dev)
    he, hn, skipped = eg.egnn_matrix_to_label(basis, orb, g, Hd)
    assert int(skipped.item()) == 0
    rows_e = sample_rows(batch.n_edges, 3000, 42)
    rows_n = sample_rows(batch.n_atoms, 1000, 43)
    src, dst = batch.src.astype(np.int64), batch.dst().astype(np.int64)
    H64 = H.astype(np.float64)
    ref_e, _ = olab.matrix_to_labels(H64, src[rows_e], dst[rows_e], None, batch.species, lay, shells, masks)
    _, ref_n = olab.matrix_to_labels(H64, np.zeros(0, np.int64), np.zeros(0, np.int64), None, batch.species, lay,
                                     shells, masks)
    del H64
    assert_close(he[torch.from_numpy(rows_e).to(dev)].cpu().numpy(), ref_e, TOL, "h_edge sample")
    assert_close(hn[torch.from_numpy(rows_n).to(dev)].cpu().numpy(), ref_n[rows_n], TOL, "h_node sample")
    # round trip over the whole batch (a fully connected graph covers every
    # entry once; T of Eq. (1) is orthogonal), compared on the GPU
    Hb, _ = eg.egnn_label_to_matrix(basis, orb, g, he, hn)
    d = (Hb - Hd).double()
    nr = float(d.norm() / Hd.double().norm())
    ma = float(d.abs().max() / Hd.abs().max())
    assert nr <= TOL and ma <= TOL, (nr, ma)


def test_group_sources_matches_stable_order(dev):
    """egnn_group_sources: src_ptr counts each source's edges and src_perm lists
    them in ascending edge order (a stable sort by source); sources outside
    [0, n_src) are in no group."""
    rng = np.random.default_rng(44)
    n, E = 300, 5000
    src = rng.integers(0, n, E).astype(np.int32)
    src[rng.choice(E, 7, replace=False)] = n + 3            # out of range: in no group
    src[rng.choice(E, 5, replace=False)] = -2
    row_ptr = np.linspace(0, E, n + 1).round().astype(np.int32)
    g = eg.Graph.from_csr(_t(row_ptr, dev), _t(src, dev), group=True)
    ok = (src >= 0) & (src < n)
    want_ptr = np.concatenate([[0], np.cumsum(np.bincount(src[ok], minlength=n))])
    want_perm = np.nonzero(ok)[0][np.argsort(src[ok], kind="stable")]
    got_ptr = g.src_ptr.cpu().numpy()
    np.testing.assert_array_equal(got_ptr, want_ptr)
    np.testing.assert_array_equal(g.src_perm[:int(got_ptr[-1])].cpu().numpy(), want_perm)


@pytest.mark.parametrize("order", list(ORDERS))
def test_out_of_range_source_is_skipped(dev, order):
    """An edge whose source is no atom has no block: counted once as skipped in
    both orders (in the source order it is in no group); every other block as usual."""
    batch = synth.make_molecule_batch(26, 5, 2, 7)
    shells, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    src = batch.src.astype(np.int32).copy()
    bad_e = len(src) // 2
    src[bad_e] = batch.n_atoms + 5
    basis, orb, _, g = _setup(batch, shells, masks, dev, src=src, group=ORDERS[order])
    lay = olab.orbital_layout(batch.mol_ptr, batch.species, shells, masks)
    H = synth.make_matrix_values(37, lay[3][-1])
    he, hn, skipped = eg.egnn_matrix_to_label(basis, orb, g, _t(H, dev))
    assert int(skipped.item()) == 1
    keep = np.arange(len(src)) != bad_e
    dst = batch.dst()
    ref_e, ref_n = olab.matrix_to_labels(H, src[keep], dst[keep], None, batch.species, lay, shells, masks)
    got = he.cpu().numpy()
    assert np.all(got[bad_e] == 0)
    assert_close(got[keep], ref_e, TOL, "h_edge")
    assert_close(hn.cpu().numpy(), ref_n, TOL, "h_node")
    Hg, skipped = eg.egnn_label_to_matrix(basis, orb, g, he, hn)
    assert int(skipped.item()) == 1
    Href = olab.labels_to_matrix(ref_e, ref_n, src[keep], dst[keep], None, batch.species, lay, shells, masks)
    assert_close(Hg.cpu().numpy(), Href, TOL, "H")
