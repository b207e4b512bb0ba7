"""HIP path vs the fp64 oracle over the layer's shape space (needs an MI355X).

The 64-atom periodic cell (several images per pair) carries every
(lmax, mmax, C, n_rbf, storage) combination below, so each kernel
instantiation the ABI dispatches to is exercised: lmax 1-4, 6 and 8, mmax 0-2, C with
a partial 64-channel chunk (24, 96) and two chunks (128), 3/4/6/8/12/16 radial
functions, bf16 storage on both bf16 GEMM variants and the fallback for
K not a multiple of 32, and the channel-pair kernels (bf16, C = 128: rotate-in,
aggregate, the backward row kernel at every (lmax, mmax), the node gradient with
packed gates); forward and backward for every one.  Also: an open cell with
isolated atoms (rows without incoming edges) and ghosts, in fp32 and on the bf16
channel pairs, and a graph with no edges at all.
Tolerances as in test_gpu_parity.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import layer as olayer
from tests.helpers import assert_close, desc_of, grid_box, oracle_graph

pytestmark = pytest.mark.gpu

eg = pytest.importorskip("equivariant_gnn_electronic_amd")

VARIANTS = [
    # lmax, mmax, C, n_rbf, storage
    (1, 0, 8, 8, "f32"),
    (1, 1, 16, 4, "f32"),
    (2, 1, 96, 8, "f32"),
    (3, 1, 24, 8, "f32"),
    (3, 2, 8, 12, "f32"),
    (2, 2, 8, 16, "f32"),
    (4, 2, 128, 8, "f32"),
    (4, 1, 32, 8, "f32"),
    (4, 0, 16, 8, "f32"),
    (3, 1, 32, 8, "bf16"),
    (4, 2, 8, 8, "bf16"),
    (2, 0, 64, 4, "bf16"),
    (2, 1, 128, 6, "bf16"),   # two channels per lane in rotate-in (C a multiple of 128, n_rbf <= 8)
    (4, 2, 128, 3, "bf16"),   # the same with an odd basis count (last basis pair half zero)
    (4, 2, 128, 8, "bf16"),   # the GeSbTe layer's shape (channel pairs, eight basis functions)
    (1, 0, 128, 8, "bf16"),   # channel pairs (bf16, C = 128) at every (lmax, mmax) of the backward row kernel
    (1, 1, 128, 2, "bf16"),
    (2, 0, 128, 8, "bf16"),
    (2, 2, 128, 4, "bf16"),
    (3, 0, 128, 8, "bf16"),
    (3, 1, 128, 7, "bf16"),
    (3, 2, 128, 8, "bf16"),
    (4, 0, 128, 5, "bf16"),
    (4, 1, 128, 16, "bf16"),  # pairs in the backward row kernel, per-channel rotate-in (16 basis functions)
    (6, 2, 8, 8, "f32"),      # higher degrees: f (lmax 6) and g (lmax 8) orbital labels need them
    (6, 1, 64, 8, "f32"),
    (6, 2, 128, 8, "bf16"),
    (8, 2, 16, 8, "f32"),
    (8, 0, 8, 4, "f32"),
    (8, 1, 32, 8, "bf16"),
    (8, 1, 128, 8, "bf16"),   # bf16 C = 128 at lmax 8: per-channel rotate-in and node gradient, packed bf16 gates both ways
    (6, 2, 16, 16, "f32"),    # three degree parts at lmax 6 (16 radial functions)
    (8, 2, 16, 16, "f32"),    # four degree parts at lmax 8
    (6, 2, 96, 8, "f32"),     # row backward in degree parts with two channel slots per lane
    (8, 1, 80, 8, "bf16"),    # the same at lmax 8 in bf16 (64 < C < 128: no channel pairs)
]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _graph(struct, dev):
    lo, box = grid_box(struct)
    pos = torch.from_numpy(struct.pos).to(dev)
    return eg.egnn_build_graph(pos, struct.n_dst, lo, box, struct.periodic_mask, struct.r_cut)


def _message_scaled(w, cfg, f=4.0):
    """Weights with every block but w_att scaled by f (a power of two, so bf16
    values stay exact).  With f = 4 the aggregated message is about as large as
    the residual x, so comparing x' - x tests the message itself even after the
    bf16 rounding of x' (which is then ~0.2% of the message instead of 5-15%)."""
    w = w.copy()
    o = 0
    for name, shape in synth.layer_weight_sizes(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf):
        n = int(np.prod(shape))
        if name != "w_att":
            w[o:o + n] *= f
        o += n
    return w


def _run(cfg, s, dev, backward):
    x, ws = synth.make_layer_inputs(cfg)
    if cfg.storage == "bf16":
        ws = [_message_scaled(ws[0], cfg)]
    g = _graph(s, dev)
    storage = eg.EGNN_BF16 if cfg.storage == "bf16" else eg.EGNN_F32
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, storage)
    geom = eg.egnn_edge_geom(desc, g)
    xt = torch.from_numpy(x).to(dev)
    if storage == eg.EGNN_BF16:
        xt = xt.to(torch.bfloat16)
    wt = torch.from_numpy(ws[0]).to(dev)
    buf = eg.LayerBuffers(desc, g, train=backward)
    (xo, eo), buf = eg.egnn_layer_fwd(desc, g, geom, wt, xt, edge_out=True, buffers=buf)
    out = dict(g=g, x=x, w=ws[0], xo=xo.float().cpu().numpy(), eo=eo.float().cpu().numpy())
    if backward:
        G = synth.make_cotangent(cfg, s.n_dst)
        gx, gw = eg.egnn_layer_bwd(desc, g, geom, wt, xt, buf, torch.from_numpy(G).to(dev))
        out.update(G=G, gx=gx.cpu().numpy(), gw=gw.cpu().numpy())
    torch.cuda.synchronize()
    return out


def _check(cfg, s, r, backward):
    og = oracle_graph(s)
    x64, w64 = r["x"].astype(np.float64), r["w"].astype(np.float64)
    fwd = olayer.layer_forward(og, x64, w64, desc_of(cfg))
    tol = 2e-2 if cfg.storage == "bf16" else 1e-4
    x_dst = x64[:s.n_dst]
    assert_close(r["xo"], fwd["x_out"], tol, "x_out")
    # the aggregated message and the per-edge messages, without the residual
    assert_close(r["xo"] - x_dst, fwd["x_out"] - x_dst, tol, "x_out - x")
    if len(og["src"]):
        assert_close(r["eo"], fwd["edge_out"], tol, "edge_out")
    if backward:
        dx, dw = olayer.layer_backward(og, x64, w64, desc_of(cfg), fwd, r["G"].astype(np.float64))
        resid = np.zeros_like(dx)
        resid[:s.n_dst] = r["G"]
        assert_close(r["gx"], dx, tol, "grad x")
        assert_close(r["gx"] - resid, dx - resid, tol, "grad x - [G; 0]")
        o = 0
        for name, shape in synth.layer_weight_sizes(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf):
            n = int(np.prod(shape))
            assert_close(r["gw"][o:o + n], dw[o:o + n], tol, f"grad {name}")
            o += n


@pytest.mark.parametrize("lmax,mmax,C,n_rbf,storage", VARIANTS)
def test_layer_shapes(dev, lmax, mmax, C, n_rbf, storage):
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], lmax=lmax, mmax=mmax, C=C, n_rbf=n_rbf, storage=storage)
    s = synth.make_structure(cfg)
    r = _run(cfg, s, dev, True)
    _check(cfg, s, r, True)


OPEN_SPARSE = synth.Config("open_sparse", 12, (40,), (12.0, 12.0, 12.0), False, 3.2, 2, 1, 16, halo=3.2,
                           note="open cell, sparse enough that some atoms have no neighbour; ghost shell")


@pytest.mark.parametrize("variant", ["f32", "bf16_pairs"])
def test_open_cell_isolated_rows(dev, variant):
    cfg = OPEN_SPARSE
    if variant == "bf16_pairs":
        cfg = dataclasses.replace(cfg, C=128, storage="bf16")
    s = synth.make_structure(cfg)
    assert s.n_src > s.n_dst
    r = _run(cfg, s, dev, True)
    indeg = np.diff(r["g"].row_ptr.cpu().numpy())
    assert (indeg == 0).any() and (indeg > 0).any()
    _check(cfg, s, r, True)
    # rows without edges keep x, and their own gradient is G
    empty = np.flatnonzero(indeg == 0)
    kept = r["x"][empty] if cfg.storage == "f32" else synth.bf16_round(r["x"][empty])
    np.testing.assert_array_equal(r["xo"][empty], kept)


def test_no_edges(dev):
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], name="far_apart")
    pos = torch.tensor([[0.0, 0, 0], [40.0, 0, 0], [0, 40.0, 0], [40.0, 40.0, 40.0]], dtype=torch.float64, device=dev)
    g = eg.egnn_build_graph(pos, 3, [0, 0, 0], [50.0, 50.0, 50.0], 0, cfg.r_cut)
    assert g.n_edges == 0
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut)
    x, ws = synth.make_layer_inputs(cfg, n_src=4)
    xt = torch.from_numpy(x).to(dev)
    wt = torch.from_numpy(ws[0]).to(dev)
    geom = eg.egnn_edge_geom(desc, g)
    buf = eg.LayerBuffers(desc, g, train=True)
    (xo, _), buf = eg.egnn_layer_fwd(desc, g, geom, wt, xt, buffers=buf)
    G = torch.from_numpy(synth.make_cotangent(cfg, 3)).to(dev)
    gx, gw = eg.egnn_layer_bwd(desc, g, geom, wt, xt, buf, G)
    torch.cuda.synchronize()
    assert torch.equal(xo, xt[:3])
    assert torch.equal(gx[:3], G) and not gx[3].any()
    assert not gw.any()


def test_hblocks_bf16_irreps(dev):
    """Decode of bf16 irreps (the bf16 path's last layer, C 16, lmax 4) against
    the oracle on the same bf16 values; fp32 arithmetic, so 1e-5."""
    cfg = synth.CONFIGS["tiny_stack"]
    s = synth.make_structure(cfg)
    x, ws = synth.make_layer_inputs(cfg)
    g = _graph(s, dev)
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, eg.EGNN_BF16)
    geom = eg.egnn_edge_geom(desc, g)
    (xo, eo), _ = eg.egnn_layer_fwd(desc, g, geom, torch.from_numpy(ws[0]).to(dev),
                                    torch.from_numpy(x).to(dev).to(torch.bfloat16), edge_out=True)
    we, wn = synth.make_decode_weights(cfg)
    he, hn = eg.egnn_hblocks(cfg.lmax, cfg.C, torch.from_numpy(np.concatenate(we)).to(dev),
                             torch.from_numpy(np.concatenate(wn)).to(dev), eo, xo, storage=eg.EGNN_BF16)
    torch.cuda.synchronize()
    from oracle import decode as odec
    assert_close(he.cpu().numpy(), odec.hblocks(eo.float().cpu().numpy().astype(np.float64), we), 1e-5, "edge blocks")
    assert_close(hn.cpu().numpy(), odec.hblocks(xo.float().cpu().numpy().astype(np.float64), wn), 1e-5, "on-site")
