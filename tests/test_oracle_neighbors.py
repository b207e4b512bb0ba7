"""Pins of the brute-force neighbour oracle: lattice shell counts, KD-tree pair sets, symmetry."""
import json
import os

import numpy as np
import pytest
from scipy.spatial import cKDTree

import synth
from oracle import neighbors

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sum_of_three_squares.json")


def _r3():
    with open(GOLD) as f:
        return {int(k): v for k, v in json.load(f)["r3"].items()}


@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("r2", [2.5, 5.5, 10.5])
def test_simple_cubic_shell_counts(n, r2):
    """Every atom of a periodic simple cubic lattice sees sum_{k < r^2} r_3(k) images.

    With n = 1 or 2 cells per axis the cutoff exceeds half the cell, so several
    images of the same atom (and of the atom itself) are neighbours.
    """
    a = 1.0
    g1 = np.arange(n) * a + 0.25
    pos = np.stack(np.meshgrid(g1, g1, g1, indexing="ij"), -1).reshape(-1, 3)
    box = np.full(3, n * a)
    g = neighbors.build_graph(pos, len(pos), box, 7, np.sqrt(r2))
    expect = sum(v for k, v in _r3().items() if k < r2)
    assert np.all(np.diff(g["row_ptr"]) == expect)
    d2 = (g["dist"].astype(np.float64)) ** 2
    assert set(np.round(d2).astype(int)) <= {k for k in range(1, 11) if k < r2}


def _pairs_from_graph(g):
    dst = neighbors.dst_of_edges(g["row_ptr"])
    return set(zip(g["src"].tolist(), dst.tolist()))


def test_matches_kdtree_periodic():
    rng = np.random.default_rng(0)
    box = np.array([20.0, 23.0, 21.0])
    pos = rng.random((300, 3)) * box
    r = 6.0                                 # < L/2: minimum image is the only image
    g = neighbors.build_graph(pos, len(pos), box, 7, r)
    tree = cKDTree(pos, boxsize=box)
    pairs = tree.query_pairs(r, output_type="ndarray")
    ref = set(map(tuple, pairs.tolist())) | set(map(tuple, pairs[:, ::-1].tolist()))
    assert _pairs_from_graph(g) == ref
    assert len(g["src"]) == len(ref)


def test_matches_kdtree_open_with_ghosts():
    rng = np.random.default_rng(1)
    pos = rng.random((400, 3)) * np.array([30.0, 25.0, 12.0])
    n_dst = 250                              # the rest are ghosts: sources only
    r = 5.0
    g = neighbors.build_graph(pos, n_dst, np.array([30.0, 25.0, 12.0]), 0, r)
    tree = cKDTree(pos)
    pairs = tree.query_pairs(r, output_type="ndarray")
    both = np.concatenate([pairs, pairs[:, ::-1]])
    ref = set(map(tuple, both[both[:, 1] < n_dst].tolist()))
    assert _pairs_from_graph(g) == ref
    assert np.all(g["shift"] == 0)
    assert len(g["src_ptr"]) == len(pos) + 1


def test_reverse_edge_symmetry_and_layout():
    s = synth.make_structure("tiny")
    g = neighbors.build_graph(s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut)
    dst = neighbors.dst_of_edges(g["row_ptr"])
    fwd = {(int(a), int(b), tuple(int(v) for v in S)): i for i, (a, b, S) in enumerate(zip(g["src"], dst, g["shift"]))}
    for (a, b, S), i in fwd.items():
        j = fwd[(b, a, tuple(-v for v in S))]
        np.testing.assert_allclose(g["vec"][i], -g["vec"][j], atol=1e-6)
    # vec = x_d - (x_s + S L)
    ref = s.pos[dst] - (s.pos[g["src"]] + g["shift"] * s.box)
    np.testing.assert_allclose(g["vec"], ref, atol=1e-5)
    np.testing.assert_allclose(g["dist"], np.linalg.norm(ref, axis=1), atol=1e-5)
    # rows sorted by (s, S) and the source grouping is a valid permutation
    for r in range(s.n_dst):
        b, e = g["row_ptr"][r], g["row_ptr"][r + 1]
        keys = [(int(a), *map(int, S)) for a, S in zip(g["src"][b:e], g["shift"][b:e])]
        assert keys == sorted(keys) and len(set(keys)) == len(keys)
    assert sorted(g["src_perm"].tolist()) == list(range(len(g["src"])))
    for sidx in range(s.n_src):
        ids = g["src_perm"][g["src_ptr"][sidx]:g["src_ptr"][sidx + 1]]
        assert np.all(g["src"][ids] == sidx) and np.all(np.diff(ids) > 0)
    # r_c = 5 > L/2 = 4.5: some pairs appear through more than one image
    pairs = list(zip(g["src"].tolist(), dst.tolist()))
    assert len(set(pairs)) < len(pairs)


def test_edge_count_matches_density():
    s = synth.make_structure("tiny")
    g = neighbors.build_graph(s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut)
    rho = s.n_dst / np.prod(s.box)
    expect = rho * 4 / 3 * np.pi * s.r_cut ** 3 * s.n_dst
    assert abs(len(g["src"]) / expect - 1) < 0.1


def test_sampled_rows_equal_full_build():
    s = synth.make_structure("tiny")
    full = neighbors.build_graph(s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut)
    rows = [3, 17, 40, 63]
    sub = neighbors.build_graph(s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut, rows=rows)
    for i, r in enumerate(rows):
        b, e = full["row_ptr"][r], full["row_ptr"][r + 1]
        sb, se = sub["row_ptr"][i], sub["row_ptr"][i + 1]
        for k in ("src", "shift", "vec", "dist"):
            np.testing.assert_array_equal(full[k][b:e], sub[k][sb:se])
