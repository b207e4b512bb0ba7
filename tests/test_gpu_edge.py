"""Edge-update block on the GPU vs the fp64 oracle, through the C ABI (needs an MI355X).

Tolerances as for the node block: fp32 <= 1e-4 normwise relative and max-abs
<= 1e-4 * max|ref|; bf16 storage <= 2e-2 against the oracle on the
bf16-rounded inputs and weights.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import layer as olayer
from oracle import neighbors as onb
from tests.helpers import assert_close, desc_of, oracle_graph, sample_rows
from tests.test_gpu_parity import gpu_graph, host

pytestmark = pytest.mark.gpu

eg = pytest.importorskip("equivariant_gnn_electronic_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _setup(cfg, dev):
    s = synth.make_structure(cfg)
    x, ws = synth.make_layer_inputs(cfg)
    g = gpu_graph(s, dev)
    storage = eg.EGNN_BF16 if cfg.storage == "bf16" else eg.EGNN_F32
    dt = torch.bfloat16 if storage == eg.EGNN_BF16 else torch.float32
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, storage)
    geom = eg.egnn_edge_geom(desc, g)
    e = synth.make_edge_embeddings(cfg, g.n_edges)
    return dict(s=s, x=x, w=ws[0], g=g, desc=desc, geom=geom, xt=torch.from_numpy(x).to(dev).to(dt),
                wt=torch.from_numpy(ws[0]).to(dev), e=e, et=torch.from_numpy(e).to(dev).to(dt), dt=dt)


def _oracle_edges_in_gpu_order(r):
    """The oracle's graph is destination-sorted in the same canonical order as the GPU's."""
    og = oracle_graph(r["s"])
    gg = host(r["g"])
    np.testing.assert_array_equal(og["src"], gg["src"])
    np.testing.assert_array_equal(og["row_ptr"], gg["row_ptr"])
    return og


EDGE_CASES = {
    "tiny": synth.CONFIGS["tiny"],
    "tiny_l4": synth.CONFIGS["tiny_l4"],
    "tiny_stack": synth.CONFIGS["tiny_stack"],
    "tiny_l6": synth.CONFIGS["tiny_l6"],
    # degree 8 (g-orbital labels), fp32 and bf16 channel pairs
    "tiny_l8": dataclasses.replace(synth.CONFIGS["tiny"], name="tiny_l8", lmax=8, mmax=2, C=16),
    "tiny_l8_bf16": dataclasses.replace(synth.CONFIGS["tiny"], name="tiny_l8_bf16", lmax=8, mmax=1, C=128,
                                        storage="bf16"),
    "tiny_l6_bf16": dataclasses.replace(synth.CONFIGS["tiny"], name="tiny_l6_bf16", lmax=6, mmax=2, C=32,
                                        storage="bf16"),
}


@pytest.mark.parametrize("name,tol", [("tiny", 1e-4), ("tiny_l4", 1e-4), ("tiny_stack", 2e-2), ("tiny_l6", 1e-4),
                                      ("tiny_l8", 1e-4), ("tiny_l8_bf16", 2e-2), ("tiny_l6_bf16", 2e-2)])
def test_edge_update_forward_backward(dev, name, tol):
    cfg = EDGE_CASES[name]
    print(f"[edge] {name}", flush=True)
    r = _setup(cfg, dev)
    eo, buf = eg.egnn_edge_update_fwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["et"])
    Ge = synth.make_edge_cotangent(cfg, r["g"].n_edges)
    gx, gw = eg.egnn_edge_update_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], buf, torch.from_numpy(Ge).to(dev))
    torch.cuda.synchronize()
    og = _oracle_edges_in_gpu_order(r)
    x64, w64, e64 = r["x"].astype(np.float64), r["w"].astype(np.float64), r["e"].astype(np.float64)
    fwd = olayer.edge_update_forward(og, x64, e64, w64, desc_of(cfg))
    assert_close(eo.float().cpu().numpy(), fwd["e_out"], tol, "e_out")
    if cfg.storage == "f32":
        assert_close(eo.cpu().numpy() - e64, fwd["e_out"] - e64, tol, "e_out - e")
    dx, de, dw = olayer.edge_update_backward(og, x64, w64, desc_of(cfg), fwd, Ge.astype(np.float64))
    assert_close(gx.cpu().numpy(), dx, tol, "grad x")
    o = 0
    for bname, shape in synth.layer_weight_sizes(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf):
        n = int(np.prod(shape))
        if bname == "w_att":
            assert np.all(gw.cpu().numpy()[o:o + n] == 0)
        else:
            assert_close(gw.cpu().numpy()[o:o + n], dw[o:o + n], tol, f"grad {bname}")
        o += n
    # in place gives the same result, and the backward is deterministic
    e2 = r["et"].clone()
    eg.egnn_edge_update_fwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], e2, e_out=e2)
    gx2, gw2 = eg.egnn_edge_update_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], buf,
                                       torch.from_numpy(Ge).to(dev))
    torch.cuda.synchronize()
    assert torch.equal(e2, eo)
    assert torch.equal(gx, gx2) and torch.equal(gw, gw2)


def _edge_keys(src, dst, shift):
    sh = np.asarray(shift, np.int64) + 8
    return ((np.asarray(src, np.int64) * (1 << 22) + np.asarray(dst, np.int64)) * 4096
            + sh[:, 0] * 256 + sh[:, 1] * 16 + sh[:, 2])


def test_edge_update_hfo2_sampled(dev):
    """Full-size HfO2 graph (544k edges, the benchmark's launch): e_out of
    sampled edges, and dL/dx of sampled atoms against the oracle run on every
    row that touches them, with each oracle edge's cotangent taken from the
    GPU edge of the same (source, destination, image)."""
    cfg = synth.CONFIGS["train"]
    r = _setup(cfg, dev)
    s = r["s"]
    eo, buf = eg.egnn_edge_update_fwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["et"])
    E = r["g"].n_edges
    Ge = synth.make_edge_cotangent(cfg, E)
    gx, _ = eg.egnn_edge_update_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], buf, torch.from_numpy(Ge).to(dev))
    torch.cuda.synchronize()
    gg = host(r["g"])
    dst = np.repeat(np.arange(s.n_dst), np.diff(gg["row_ptr"]))
    x64, w64 = r["x"].astype(np.float64), r["w"].astype(np.float64)
    W = olayer.unpack_weights(w64, desc_of(cfg))
    # forward: sampled edges
    es = sample_rows(E, 2000, 31)
    sub = dict(src=gg["src"][es], vec=gg["vec"][es].astype(np.float64), dist=gg["dist"][es].astype(np.float64))
    msg = olayer.edge_forward(sub, x64, W, desc_of(cfg), x64[dst[es]])["msg"]
    assert_close(eo.cpu().numpy()[es], r["e"][es] + msg, 1e-4, "e_out of sampled edges")
    # backward: sampled atoms
    nodes = sample_rows(s.n_dst, 2, 32)
    rows = np.unique(np.concatenate([nodes, dst[np.isin(gg["src"], nodes)]]))
    rest = np.setdiff1d(np.arange(s.n_src), rows)
    perm = np.concatenate([rows, rest])
    og = onb.build_graph(s.pos[perm], len(rows), s.box, s.periodic_mask, s.r_cut)
    odst = np.repeat(np.arange(len(rows)), np.diff(og["row_ptr"]))
    keys_gpu = _edge_keys(gg["src"], dst, gg["shift"])
    order = np.argsort(keys_gpu)
    keys_o = _edge_keys(perm[og["src"]], perm[odst], og["shift"])
    pos = np.searchsorted(keys_gpu[order], keys_o)
    assert np.all(keys_gpu[order][pos] == keys_o)
    Ge_o = Ge[order[pos]].astype(np.float64)
    xp = x64[perm]
    fwd = olayer.edge_update_forward(og, xp, np.zeros_like(Ge_o), w64, desc_of(cfg))
    dx, _, _ = olayer.edge_update_backward(og, xp, w64, desc_of(cfg), fwd, Ge_o)
    assert_close(gx.cpu().numpy()[nodes], dx[np.searchsorted(rows, nodes)], 1e-4, "grad x of sampled atoms")
