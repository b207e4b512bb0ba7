"""Shared helpers for the parity tests: inputs from synth/, errors, oracle runs."""
from __future__ import annotations

import numpy as np

import synth
from oracle import layer as olayer
from oracle import neighbors as onb


def norm_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def assert_close(got, ref, tol, what=""):
    """Normwise relative error <= tol and max-abs error <= tol * max|ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nr = norm_rel(got, ref)
    ma = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert nr <= tol and ma <= tol * max(scale, 1e-30), f"{what}: normwise {nr:.3e}, max-abs {ma:.3e} (scale {scale:.3e})"
    return nr, ma


def desc_of(cfg):
    return olayer.LayerDesc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut)


def grid_box(struct):
    """(lo, box) handed to the graph builder: the cell for periodic structures,
    the padded extent of all positions for open ones."""
    if struct.periodic_mask == 7:
        return np.zeros(3), np.asarray(struct.box, np.float64)
    lo = struct.pos.min(axis=0)
    hi = struct.pos.max(axis=0)
    return lo, (hi - lo) * (1 + 1e-12) + 1e-9


def oracle_graph(struct, rows=None):
    return onb.build_graph(struct.pos, struct.n_dst, struct.box, struct.periodic_mask, struct.r_cut, rows=rows)


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(k, n), replace=False))
