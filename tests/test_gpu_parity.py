"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Tolerances: integer graph arrays and vec bit-exact, dist within 1 ulp;
Wigner rows and radial basis <= 1e-6 absolute; fp32 layer outputs and
gradients <= 1e-4 normwise relative and max-abs <= 1e-4 * max|ref|;
bf16 storage <= 2e-2 normwise against the oracle on the bf16-rounded inputs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import decode as odec
from oracle import layer as olayer
from oracle import neighbors as onb
from oracle import so3
from tests.helpers import assert_close, desc_of, grid_box, oracle_graph, sample_rows

pytestmark = pytest.mark.gpu

eg = pytest.importorskip("equivariant_gnn_electronic_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def gpu_graph(struct, dev):
    lo, box = grid_box(struct)
    pos = torch.from_numpy(struct.pos).to(dev)
    if struct.periodic_mask == 7:
        return eg.egnn_build_graph(pos, struct.n_dst, lo, box, 7, struct.r_cut)
    return eg.egnn_build_graph(pos, struct.n_dst, lo, box, 0, struct.r_cut)


def host(g):
    return {k: getattr(g, k).cpu().numpy() for k in ("row_ptr", "src", "shift", "vec", "dist", "src_ptr", "src_perm")}


def _check_rows(gg, og, rows):
    for i, r in enumerate(rows):
        b, e = gg["row_ptr"][r], gg["row_ptr"][r + 1]
        ob, oe = og["row_ptr"][i], og["row_ptr"][i + 1]
        assert e - b == oe - ob, f"row {r}: {e - b} vs {oe - ob} edges"
        np.testing.assert_array_equal(gg["src"][b:e], og["src"][ob:oe])
        np.testing.assert_array_equal(gg["shift"][b:e], og["shift"][ob:oe])
        np.testing.assert_array_equal(gg["vec"][b:e], og["vec"][ob:oe])
        ulp = np.abs(gg["dist"][b:e].view(np.int32) - og["dist"][ob:oe].view(np.int32))
        assert ulp.max(initial=0) <= 1


def _check_src_grouping(gg, n_src):
    order = np.argsort(gg["src"], kind="stable")
    np.testing.assert_array_equal(gg["src_perm"], order)
    cnt = np.bincount(gg["src"], minlength=n_src)
    np.testing.assert_array_equal(gg["src_ptr"], np.concatenate([[0], np.cumsum(cnt)]))


@pytest.mark.parametrize("name,nrows", [("tiny", None), ("hfo2", None), ("gst", 400), ("halo", 400)])
def test_graph_bit_exact(dev, name, nrows):
    s = synth.make_structure(name)
    g = gpu_graph(s, dev)
    gg = host(g)
    rows = np.arange(s.n_dst) if nrows is None else sample_rows(s.n_dst, nrows, 11)
    og = oracle_graph(s, rows=None if nrows is None else rows)
    if nrows is None:
        assert g.n_edges == len(og["src"])
        np.testing.assert_array_equal(gg["row_ptr"], og["row_ptr"])
    _check_rows(gg, og, rows)
    _check_src_grouping(gg, s.n_src)
    # deterministic: a second build is bit-identical
    gg2 = host(gpu_graph(s, dev))
    for k in gg:
        np.testing.assert_array_equal(gg[k], gg2[k])


def test_graph_capacity_protocol_and_empty(dev):
    s = synth.make_structure("tiny")
    g = gpu_graph(s, dev)
    assert g.n_edges > 0
    # isolated atoms (open boundary, far apart): zero edges, empty rows
    pos = torch.tensor([[0.0, 0, 0], [50.0, 0, 0], [0, 50.0, 0]], dtype=torch.float64, device=dev)
    g0 = eg.egnn_build_graph(pos, 3, [0, 0, 0], [60.0, 60.0, 60.0], 0, 5.0)
    assert g0.n_edges == 0
    assert g0.row_ptr.cpu().tolist() == [0, 0, 0, 0]
    assert g0.src_ptr.cpu().tolist() == [0, 0, 0, 0]


def _oracle_geom_rows(vec, dist, cfg):
    d = desc_of(cfg)
    D = olayer.edge_wigner(vec.astype(np.float64), cfg.lmax)
    parts = []
    for l in range(cfg.lmax + 1):
        mr = min(l, cfg.mmax)
        parts.append(D[l][:, l - mr:l + mr + 1, :].reshape(len(vec), -1))
    return np.concatenate(parts, axis=1), olayer.radial_basis(dist, d)


GEOM_CASES = {n: synth.CONFIGS[n] for n in ("tiny", "tiny_l4", "tiny_l6", "hfo2", "hfo2_l6", "hfo2_l8")}
GEOM_CASES["tiny_l8"] = dataclasses.replace(synth.CONFIGS["tiny"], name="tiny_l8", lmax=8, mmax=2, C=16)
GEOM_CASES["tiny_l8_m1"] = dataclasses.replace(synth.CONFIGS["tiny"], name="tiny_l8_m1", lmax=8, mmax=1, C=16)


@pytest.mark.parametrize("name", list(GEOM_CASES))
def test_edge_geom(dev, name):
    """Wigner rows |m| <= mmax of every degree (to lmax 8) and the radial basis
    against the oracle's least-squares Wigner-D, 1e-6 absolute."""
    cfg = GEOM_CASES[name]
    s = synth.make_structure(cfg)
    g = gpu_graph(s, dev)
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut)
    geom = eg.egnn_edge_geom(desc, g).cpu().numpy()
    gg = host(g)
    idx = np.arange(g.n_edges) if g.n_edges < 50000 else sample_rows(g.n_edges, 20000, 3)
    Dref, phiref = _oracle_geom_rows(gg["vec"][idx], gg["dist"][idx], cfg)
    nD = Dref.shape[1]
    assert np.max(np.abs(geom[idx, :nD] - Dref)) <= 1e-6
    assert np.max(np.abs(geom[idx, nD:nD + cfg.n_rbf] - phiref)) <= 1e-6
    dst = np.repeat(np.arange(s.n_dst), np.diff(gg["row_ptr"]))
    np.testing.assert_array_equal(geom[:g.n_edges, nD + cfg.n_rbf].view(np.int32), dst)


def _gpu_forward(cfg, dev, edge_out=False, train=False, layer=0):
    s = synth.make_structure(cfg)
    x, ws = synth.make_layer_inputs(cfg)
    g = gpu_graph(s, dev)
    storage = eg.EGNN_BF16 if cfg.storage == "bf16" else eg.EGNN_F32
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, storage)
    geom = eg.egnn_edge_geom(desc, g)
    xt = torch.from_numpy(x).to(dev)
    if storage == eg.EGNN_BF16:
        xt = xt.to(torch.bfloat16)
    wt = torch.from_numpy(ws[layer]).to(dev)
    buf = eg.LayerBuffers(desc, g, train=train) if train else None
    (xo, eo), buf = eg.egnn_layer_fwd(desc, g, geom, wt, xt, edge_out=edge_out, buffers=buf)
    torch.cuda.synchronize()
    return dict(s=s, x=x, w=ws[layer], g=g, desc=desc, geom=geom, xt=xt, wt=wt, buf=buf, xo=xo, eo=eo)


@pytest.mark.parametrize("name", ["tiny", "tiny_l4"])
def test_layer_forward_full(dev, name):
    cfg = synth.CONFIGS[name]
    r = _gpu_forward(cfg, dev, edge_out=True)
    og = oracle_graph(r["s"])
    ref = olayer.layer_forward(og, r["x"].astype(np.float64), r["w"].astype(np.float64), desc_of(cfg))
    xo = r["xo"].float().cpu().numpy()
    assert_close(xo, ref["x_out"], 1e-4, "x_out")
    assert_close(xo - r["x"][:r["s"].n_dst], ref["x_out"] - r["x"][:r["s"].n_dst], 1e-4, "aggregate")
    assert_close(r["eo"].float().cpu().numpy(), ref["edge_out"], 1e-4, "edge_out")


def test_layer_forward_hfo2_sampled_rows(dev):
    cfg = synth.CONFIGS["hfo2"]
    r = _gpu_forward(cfg, dev)
    rows = sample_rows(r["s"].n_dst, 200, 5)
    og = oracle_graph(r["s"], rows=rows)
    xo_ref, _ = olayer.layer_forward_rows(og, r["x"].astype(np.float64), r["w"].astype(np.float64), desc_of(cfg))
    xo = r["xo"].float().cpu().numpy()[rows]
    assert_close(xo, xo_ref, 1e-4, "x_out rows")
    assert_close(xo - r["x"][rows], xo_ref - r["x"][rows], 1e-4, "aggregate rows")


@pytest.mark.parametrize("name", ["tiny", "tiny_l4"])
def test_layer_backward_full(dev, name):
    cfg = synth.CONFIGS[name]
    r = _gpu_forward(cfg, dev, train=True)
    G = synth.make_cotangent(cfg, r["s"].n_dst)
    gx, gw = eg.egnn_layer_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["buf"],
                               torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    og = oracle_graph(r["s"])
    x64, w64 = r["x"].astype(np.float64), r["w"].astype(np.float64)
    fwd = olayer.layer_forward(og, x64, w64, desc_of(cfg))
    dx, dw = olayer.layer_backward(og, x64, w64, desc_of(cfg), fwd, G.astype(np.float64))
    assert_close(gx.cpu().numpy(), dx, 1e-4, "grad x")
    o = 0
    for bname, shape in synth.layer_weight_sizes(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf):
        n = int(np.prod(shape))
        assert_close(gw.cpu().numpy()[o:o + n], dw[o:o + n], 1e-4, f"grad {bname}")
        o += n
    # deterministic
    gx2, gw2 = eg.egnn_layer_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["buf"],
                                 torch.from_numpy(G).to(dev))
    assert torch.equal(gx, gx2) and torch.equal(gw, gw2)


def test_hblocks(dev):
    cfg = synth.CONFIGS["tiny_l4"]
    r = _gpu_forward(cfg, dev, edge_out=True)
    we, wn = synth.make_decode_weights(cfg)
    wet = torch.from_numpy(np.concatenate(we)).to(dev)
    wnt = torch.from_numpy(np.concatenate(wn)).to(dev)
    he, hn = eg.egnn_hblocks(4, cfg.C, wet, wnt, r["eo"], r["xo"])
    torch.cuda.synchronize()
    he_ref = odec.hblocks(r["eo"].cpu().numpy(), we)
    hn_ref = odec.hblocks(r["xo"].cpu().numpy(), wn)
    assert_close(he.cpu().numpy(), he_ref, 1e-5, "edge blocks")
    assert_close(hn.cpu().numpy(), hn_ref, 1e-5, "on-site blocks")


def test_hblocks_f_shells(dev):
    """Decode with f shells (s s p p d f, 20 orbitals, labels up to L = 6) from
    lmax-6 irreps: the layer's edge messages and outputs at lmax 6."""
    cfg = synth.CONFIGS["tiny_l6"]
    r = _gpu_forward(cfg, dev, edge_out=True)
    shells = (0, 0, 1, 1, 2, 3)
    _, n = odec.label_layout(shells)
    rng = np.random.default_rng(61)
    we = [(rng.standard_normal((c, cfg.C)) / np.sqrt(cfg.C)).astype(np.float32) for c in n]
    wn = [(rng.standard_normal((c, cfg.C)) / np.sqrt(cfg.C)).astype(np.float32) for c in n]
    he, hn = eg.egnn_hblocks(6, cfg.C, torch.from_numpy(np.concatenate(we)).to(dev),
                             torch.from_numpy(np.concatenate(wn)).to(dev), r["eo"], r["xo"], shell_l=shells)
    torch.cuda.synchronize()
    assert he.shape[1:] == (20, 20)
    assert_close(he.cpu().numpy(), odec.hblocks(r["eo"].cpu().numpy(), we, shells), 1e-5, "edge blocks")
    assert_close(hn.cpu().numpy(), odec.hblocks(r["xo"].cpu().numpy(), wn, shells), 1e-5, "on-site blocks")


@pytest.mark.parametrize("C,storage", [(16, "f32"), (32, "bf16")])
def test_hblocks_g_shells(dev, C, storage):
    """Decode with g shells (s p d f g, 25 orbitals, labels up to L = 8) from
    lmax-8 irreps: the layer's edge messages and outputs at lmax 8."""
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], name=f"tiny_l8_{storage}", lmax=8, mmax=2, C=C,
                              storage=storage)
    r = _gpu_forward(cfg, dev, edge_out=True)
    shells = synth.G_SHELLS
    _, n = odec.label_layout(shells)
    rng = np.random.default_rng(62)
    we = [(rng.standard_normal((c, C)) / np.sqrt(C)).astype(np.float32) for c in n]
    wn = [(rng.standard_normal((c, C)) / np.sqrt(C)).astype(np.float32) for c in n]
    st = eg.EGNN_BF16 if storage == "bf16" else eg.EGNN_F32
    he, hn = eg.egnn_hblocks(8, C, torch.from_numpy(np.concatenate(we)).to(dev),
                             torch.from_numpy(np.concatenate(wn)).to(dev), r["eo"], r["xo"], shell_l=shells,
                             storage=st)
    torch.cuda.synchronize()
    assert he.shape[1:] == (25, 25)
    eo = r["eo"].float().cpu().numpy().astype(np.float64)
    xo = r["xo"].float().cpu().numpy().astype(np.float64)
    assert_close(he.cpu().numpy(), odec.hblocks(eo, we, shells), 1e-5, "edge blocks")
    assert_close(hn.cpu().numpy(), odec.hblocks(xo, wn, shells), 1e-5, "on-site blocks")


def _rotate_irreps(a, Q, lmax):
    out = np.empty_like(a)
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        out[:, sl, :] = np.einsum("mn,enc->emc", so3.wigner_d(l, Q), a[:, sl, :])
    return out


def _run_stack(cfg, dev, g, geom, x_t, ws):
    """The layers of cfg chained through the ABI (bf16 or fp32 storage)."""
    storage = eg.EGNN_BF16 if cfg.storage == "bf16" else eg.EGNN_F32
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, storage)
    xs = x_t
    for w in ws:
        (xs, _), _ = eg.egnn_layer_fwd(desc, g, geom, torch.from_numpy(w).to(dev), xs)
    torch.cuda.synchronize()
    return xs


def test_layer_stack_bf16_tiny(dev):
    """Three layers with bf16 storage against the oracle on the same bf16 inputs."""
    from tests.test_gpu_variants import _message_scaled
    cfg = synth.CONFIGS["tiny_stack"]
    s = synth.make_structure(cfg)
    x, ws = synth.make_layer_inputs(cfg)
    # weights (but w_att) doubled: the three layers' messages are then ~20% of
    # x', so x' - x is compared well above the bf16 rounding of x' (~1% of it)
    ws = [_message_scaled(w, cfg, 2.0) for w in ws]
    g = gpu_graph(s, dev)
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, eg.EGNN_BF16)
    geom = eg.egnn_edge_geom(desc, g)
    xo = _run_stack(cfg, dev, g, geom, torch.from_numpy(x).to(dev).to(torch.bfloat16), ws).float().cpu().numpy()
    og = oracle_graph(s)
    xr = x.astype(np.float64)
    for w in ws:
        xr = olayer.layer_forward(og, xr, w.astype(np.float64), desc_of(cfg))["x_out"]
    assert_close(xo, xr, 2e-2, "3-layer bf16 x_out")
    x_dst = x[:s.n_dst].astype(np.float64)
    assert_close(xo - x_dst, xr - x_dst, 2e-2, "3-layer bf16 x_out - x")


def test_layer_forward_gst_bf16_sampled_rows(dev):
    """First layer of the 8,064-atom GeSbTe-like cell (bf16 storage, C 128) on sampled rows."""
    cfg = synth.CONFIGS["gst"]
    r = _gpu_forward(cfg, dev, edge_out=True)
    rows = sample_rows(r["s"].n_dst, 120, 7)
    og = oracle_graph(r["s"], rows=rows)
    xo_ref, _ = olayer.layer_forward_rows(og, r["x"].astype(np.float64), r["w"].astype(np.float64), desc_of(cfg))
    xo = r["xo"].float().cpu().numpy()[rows]
    assert_close(xo, xo_ref, 2e-2, "gst x_out rows")
    # the per-edge messages (no residual) of 40 of these rows, element by element
    gg = host(r["g"])
    sub = rows[:40]
    og40 = oracle_graph(r["s"], rows=sub)
    sel = np.concatenate([np.arange(gg["row_ptr"][q], gg["row_ptr"][q + 1]) for q in sub])
    ef = olayer.edge_forward(og40, r["x"].astype(np.float64), olayer.unpack_weights(r["w"].astype(np.float64), desc_of(cfg)),
                             desc_of(cfg), r["x"][np.repeat(sub, np.diff(og40["row_ptr"]))].astype(np.float64))
    eo = r["eo"][torch.from_numpy(sel).to(dev)].float().cpu().numpy()
    assert_close(eo, ef["msg"], 2e-2, "gst edge messages")


def test_layer_forward_halo_sampled_rows(dev):
    """One GPU's share: 30,000 owned rows, 21,133 ghost sources, open boundary, fp32."""
    cfg = synth.CONFIGS["halo"]
    r = _gpu_forward(cfg, dev)
    assert r["g"].n_src > r["g"].n_dst
    rows = sample_rows(r["s"].n_dst, 200, 9)
    og = oracle_graph(r["s"], rows=rows)
    xo_ref, _ = olayer.layer_forward_rows(og, r["x"].astype(np.float64), r["w"].astype(np.float64), desc_of(cfg))
    xo = r["xo"].float().cpu().numpy()[rows]
    assert_close(xo, xo_ref, 1e-4, "halo x_out rows")
    assert_close(xo - r["x"][rows], xo_ref - r["x"][rows], 1e-4, "halo aggregate rows")


def test_gst_stack_equivariance_full_size(dev):
    """Full 8,064-atom, 3-layer bf16 stack: rotating every edge vector and input irrep by Q
    rotates the output by D(Q) (a property that holds at any size)."""
    from scipy.spatial.transform import Rotation as Rot
    cfg = synth.CONFIGS["gst"]
    s = synth.make_structure(cfg)
    x, ws = synth.make_layer_inputs(cfg)
    g = gpu_graph(s, dev)
    desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, eg.EGNN_BF16)
    geom = eg.egnn_edge_geom(desc, g)
    base = _run_stack(cfg, dev, g, geom, torch.from_numpy(x).to(dev).to(torch.bfloat16), ws).float().cpu().numpy()
    Q = Rot.random(random_state=11).as_matrix()
    vec = g.vec.cpu().numpy().astype(np.float64) @ Q.T
    g2 = eg.Graph(g.n_dst, g.n_src, g.n_edges, g.row_ptr, g.src, g.shift,
                  torch.from_numpy(vec.astype(np.float32)).to(dev), g.dist, g.src_ptr, g.src_perm)
    geom2 = eg.egnn_edge_geom(desc, g2)
    xr = synth.bf16_round(_rotate_irreps(x.astype(np.float64), Q, cfg.lmax).astype(np.float32))
    rot = _run_stack(cfg, dev, g2, geom2, torch.from_numpy(xr).to(dev).to(torch.bfloat16), ws).float().cpu().numpy()
    assert_close(rot, _rotate_irreps(base, Q, cfg.lmax), 2e-2, "rotated 3-layer output")


def _relabelled_rows(struct, rows):
    """Positions with `rows` moved to the front (they become destinations
    0..len(rows)-1); every other atom stays a source, ghosts last."""
    rest = np.setdiff1d(np.arange(struct.n_src), rows)
    perm = np.concatenate([rows, rest])
    return perm, onb.build_graph(struct.pos[perm], len(rows), struct.box, struct.periodic_mask, struct.r_cut)


def test_layer_backward_hfo2_sampled_nodes(dev):
    """Full-size training layer (544k edges, the launch the training step times):
    dL/dx of sampled atoms against the oracle's exact gradient.  The oracle runs
    on every row that touches a sampled atom (its own row and the rows of all
    its outgoing edges), which holds every term of that atom's gradient."""
    cfg = synth.CONFIGS["train"]
    r = _gpu_forward(cfg, dev, train=True)
    s = r["s"]
    G = synth.make_cotangent(cfg, s.n_dst)
    gx, _ = eg.egnn_layer_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["buf"], torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    gx = gx.cpu().numpy()
    gg = host(r["g"])
    dst = np.repeat(np.arange(s.n_dst), np.diff(gg["row_ptr"]))
    nodes = sample_rows(s.n_dst, 2, 21)
    rows = np.unique(np.concatenate([nodes, dst[np.isin(gg["src"], nodes)]]))
    perm, og = _relabelled_rows(s, rows)
    x64, w64 = r["x"][perm].astype(np.float64), r["w"].astype(np.float64)
    fwd = olayer.layer_forward(og, x64, w64, desc_of(cfg))
    dx, _ = olayer.layer_backward(og, x64, w64, desc_of(cfg), fwd, G[rows].astype(np.float64))
    where = np.searchsorted(rows, nodes)  # sampled atoms sit at these relabelled positions
    assert_close(gx[nodes], dx[where], 1e-4, "grad x of sampled atoms")
    assert_close(gx[nodes] - G[nodes], dx[where] - G[nodes], 1e-4, "grad x of sampled atoms - G")


def test_weight_gradient_hfo2_directional(dev):
    """Full-size weight gradient: <dL/dW, v> against the central difference of
    L(W) = <G, x'(W)> along a random direction v, both from the GPU forward
    (a property that holds at any size; fp32 forward, so 1e-2)."""
    cfg = synth.CONFIGS["train"]
    r = _gpu_forward(cfg, dev, train=True)
    G = synth.make_cotangent(cfg, r["s"].n_dst)
    Gt = torch.from_numpy(G).to(dev)
    _, gw = eg.egnn_layer_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["buf"], Gt)
    v = torch.from_numpy(np.random.default_rng(3).standard_normal(r["w"].size).astype(np.float32)).to(dev)
    v *= r["wt"].norm() / v.norm()
    eps = 1e-3

    def loss(w):
        (xo, _), _ = eg.egnn_layer_fwd(r["desc"], r["g"], r["geom"], w, r["xt"])
        return float((xo.double() * Gt.double()).sum())

    fd = (loss(r["wt"] + eps * v) - loss(r["wt"] - eps * v)) / (2 * eps)
    an = float((gw.double() * v.double()).sum())
    assert abs(fd - an) <= 1e-2 * abs(an), (fd, an)


def test_hblocks_hfo2_sampled_edges(dev):
    """Decode at full size (544k edges, 13x13 blocks): sampled edges and atoms
    against the oracle's Label->Matrix on the same irreps."""
    cfg = synth.CONFIGS["train"]
    r = _gpu_forward(cfg, dev, edge_out=True)
    we, wn = synth.make_decode_weights(cfg)
    wet = torch.from_numpy(np.concatenate(we)).to(dev)
    wnt = torch.from_numpy(np.concatenate(wn)).to(dev)
    he, hn = eg.egnn_hblocks(cfg.lmax, cfg.C, wet, wnt, r["eo"], r["xo"])
    torch.cuda.synchronize()
    ei = sample_rows(r["g"].n_edges, 3000, 5)
    ni = sample_rows(r["s"].n_dst, 300, 6)
    eo = r["eo"][torch.from_numpy(ei).to(dev)].cpu().numpy().astype(np.float64)
    xo = r["xo"][torch.from_numpy(ni).to(dev)].cpu().numpy().astype(np.float64)
    assert_close(he[torch.from_numpy(ei).to(dev)].cpu().numpy(), odec.hblocks(eo, we), 1e-5, "edge blocks")
    assert_close(hn[torch.from_numpy(ni).to(dev)].cpu().numpy(), odec.hblocks(xo, wn), 1e-5, "on-site blocks")
    # the per-edge messages themselves at the sampled edges' rows
    gg = host(r["g"])
    rows = np.unique(np.searchsorted(gg["row_ptr"], ei, side="right") - 1)[:40]
    og = oracle_graph(r["s"], rows=rows)
    sel = np.concatenate([np.arange(gg["row_ptr"][q], gg["row_ptr"][q + 1]) for q in rows])
    ef = olayer.edge_forward(og, r["x"].astype(np.float64), olayer.unpack_weights(r["w"].astype(np.float64), desc_of(cfg)),
                             desc_of(cfg), r["x"][np.repeat(rows, np.diff(og["row_ptr"]))].astype(np.float64))
    assert_close(r["eo"][torch.from_numpy(sel).to(dev)].cpu().numpy(), ef["msg"], 1e-4, "edge messages")


def _sampled_atom_grads(cfg, r, dev, n_nodes, seed, tol):
    s = r["s"]
    G = synth.make_cotangent(cfg, s.n_dst)
    gx, _ = eg.egnn_layer_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["buf"], torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    gx = gx.cpu().numpy()
    gg = host(r["g"])
    dst = np.repeat(np.arange(s.n_dst), np.diff(gg["row_ptr"]))
    nodes = sample_rows(s.n_dst, n_nodes, seed)
    rows = np.unique(np.concatenate([nodes, dst[np.isin(gg["src"], nodes)]]))
    perm, og = _relabelled_rows(s, rows)
    x64, w64 = r["x"][perm].astype(np.float64), r["w"].astype(np.float64)
    fwd = olayer.layer_forward(og, x64, w64, desc_of(cfg))
    dx, _ = olayer.layer_backward(og, x64, w64, desc_of(cfg), fwd, G[rows].astype(np.float64))
    assert_close(gx[nodes], dx[np.searchsorted(rows, nodes)], tol, "grad x of sampled atoms")
    assert_close(gx[nodes] - G[nodes], dx[np.searchsorted(rows, nodes)] - G[nodes], tol,
                 "grad x of sampled atoms - G")


def test_layer_backward_gst_bf16_sampled_nodes(dev):
    """Backward of the 8,064-atom GeSbTe-like layer with bf16 storage (C 128,
    1.1M edges): exact oracle gradients of sampled atoms, bf16 tolerance."""
    cfg = synth.CONFIGS["gst"]
    r = _gpu_forward(cfg, dev, train=True)
    _sampled_atom_grads(cfg, r, dev, 2, 23, 2e-2)


def test_weight_gradient_gst_bf16_directional(dev):
    """bf16-storage weight gradient at full GST size (1.1M edges, C 128) against
    the central difference of L(W) = <G, x'(W)> along a random direction.  L is
    evaluated by the fp32-storage forward on the same (bf16-exact) inputs: the
    bf16 forward rounds every activation, which makes its own differences too
    rough, and the bf16 backward approximates this smooth L's gradient."""
    cfg = synth.CONFIGS["gst"]
    r = _gpu_forward(cfg, dev, train=True)
    G = synth.make_cotangent(cfg, r["s"].n_dst)
    Gt = torch.from_numpy(G).to(dev)
    _, gw = eg.egnn_layer_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["buf"], Gt)
    d32 = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, eg.EGNN_F32)
    x32 = r["xt"].float()
    v = torch.from_numpy(np.random.default_rng(4).standard_normal(r["w"].size).astype(np.float32)).to(dev)
    v *= r["wt"].norm() / v.norm()
    eps = 1e-3

    def loss(w):
        (xo, _), _ = eg.egnn_layer_fwd(d32, r["g"], r["geom"], w, x32)
        return float((xo.double() * Gt.double()).sum())

    fd = (loss(r["wt"] + eps * v) - loss(r["wt"] - eps * v)) / (2 * eps)
    an = float((gw.double() * v.double()).sum())
    assert abs(fd - an) <= 2e-2 * abs(an), (fd, an)


def _masked_cotangent(cfg, n_dst, rows):
    """The seeded cotangent G kept on `rows` only, zero on every other row."""
    G = synth.make_cotangent(cfg, n_dst)
    Gm = np.zeros_like(G)
    Gm[rows] = G[rows]
    return Gm


def _oracle_backward_on_rows(cfg, s, x, w, rows, G):
    """Exact oracle gradients of <G, x'> when G is zero outside `rows`.

    Every term of the backward starts from G_d of an edge's destination, so
    only the edges of `rows` contribute: the oracle runs the layer on those
    rows alone (relabelled to destinations 0..len(rows)-1, every atom still a
    source) and its gradients are the full-size ones.  Returns dx in the
    original atom order and the packed weight gradient."""
    perm, og = _relabelled_rows(s, rows)
    x64, w64 = x[perm].astype(np.float64), w.astype(np.float64)
    d = desc_of(cfg)
    fwd = olayer.layer_forward(og, x64, w64, d)
    dxp, dw = olayer.layer_backward(og, x64, w64, d, fwd, G[rows].astype(np.float64))
    dx = np.empty_like(dxp)
    dx[perm] = dxp
    return dx, dw


def _compare_full_backward(cfg, r, dev, rows, tol):
    s = r["s"]
    G = _masked_cotangent(cfg, s.n_dst, rows)
    gx, gw = eg.egnn_layer_bwd(r["desc"], r["g"], r["geom"], r["wt"], r["xt"], r["buf"], torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    gx, gw = gx.cpu().numpy(), gw.cpu().numpy()
    dx, dw = _oracle_backward_on_rows(cfg, s, r["x"], r["w"], rows, G)   # x, w already storage-rounded
    # the message part of grad x, without the residual [G; 0] that both carry
    resid = np.zeros_like(dx)
    resid[:s.n_dst] = G
    assert_close(gx - resid, dx - resid, tol, "grad x (message part)")
    assert_close(gx, dx, tol, "grad x")
    o = 0
    for bname, shape in synth.layer_weight_sizes(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf):
        n = int(np.prod(shape))
        assert_close(gw[o:o + n], dw[o:o + n], tol, f"grad {bname}")
        o += n


def test_layer_backward_hfo2_full_size_masked_rows(dev):
    """The training step's backward launch at full size (544k edges: every split-K
    split of the weight-gradient products, two-level column sums of the attention
    and radial-weight gradients) with G kept on 200 rows spread over the row
    range: every weight-gradient block and grad x of every atom against the
    oracle's exact values, element by element at the fp32 bar."""
    cfg = synth.CONFIGS["train"]
    r = _gpu_forward(cfg, dev, train=True)
    rows = np.unique(np.linspace(0, r["s"].n_dst - 1, 200).round().astype(np.int64))
    _compare_full_backward(cfg, r, dev, rows, 1e-4)


def test_layer_backward_gst_bf16_full_size_masked_rows(dev):
    """The same on the 8,064-atom GeSbTe-like layer (bf16 storage, C 128, 1.1M
    edges: the transposed-read bf16 split-K products and their fold), at the
    bf16 bar against the oracle on the bf16-rounded inputs."""
    cfg = synth.CONFIGS["gst"]
    r = _gpu_forward(cfg, dev, train=True)
    rows = np.unique(np.linspace(0, r["s"].n_dst - 1, 128).round().astype(np.int64))
    _compare_full_backward(cfg, r, dev, rows, 2e-2)


@pytest.mark.parametrize("name,n_rows,storage", [("hfo2_l6", 32, "f32"), ("hfo2_l8", 24, "f32"),
                                                  ("gst_l6", 16, "bf16")])
def test_layer_higher_degree_full_size_masked_rows(dev, name, n_rows, storage):
    """The degree-part launches of the backward node kernels (one launch per
    range of degrees at lmax 6 and 8) at full size: the HfO2-like graph (544k
    edges, fp32, C 64) at lmax 6 and 8, and the GeSbTe-like graph (1.1M edges,
    bf16, C 128: channel-pair forward kernels and packed gates) at lmax 6.
    x' of the sampled rows (its message part at the fp32 bar), then, with the
    cotangent on those rows only, every weight block and grad x of every atom
    against the oracle's exact values."""
    if name == "gst_l6":
        cfg = dataclasses.replace(synth.CONFIGS["gst"], name="gst_l6", lmax=6, layers=1)
    else:
        cfg = synth.CONFIGS[name]
    assert cfg.storage == storage
    r = _gpu_forward(cfg, dev, train=True)
    s = r["s"]
    rows = np.unique(np.linspace(0, s.n_dst - 1, n_rows).round().astype(np.int64))
    print(f"[parity] {name} lmax={cfg.lmax} rows={len(rows)} edges={r['g'].n_edges}", flush=True)
    perm, og = _relabelled_rows(s, rows)
    x64 = r["x"][perm].astype(np.float64)
    ref = olayer.layer_forward(og, x64, r["w"].astype(np.float64), desc_of(cfg))
    xo = r["xo"].float().cpu().numpy()[rows]
    tol = 2e-2 if storage == "bf16" else 1e-4
    assert_close(xo, ref["x_out"], tol, "x_out rows")
    if storage == "f32":
        assert_close(xo - r["x"][rows], ref["x_out"] - x64[:len(rows)], tol, "x_out rows - x")
    _compare_full_backward(cfg, r, dev, rows, tol)


def test_hblocks_gst_bf16_c128_sampled(dev):
    """The decode that the 8,064-atom training step runs: bf16 irreps with C 128
    (the GeSbTe-like layer's own edge messages and outputs, 1.1M edges) into
    13 x 13 blocks, on 3,000 sampled edges and 300 atoms against the oracle's
    Label -> Matrix on the same bf16 values (fp32 arithmetic, so 1e-5)."""
    cfg = synth.CONFIGS["gst"]
    r = _gpu_forward(cfg, dev, edge_out=True)
    we, wn = synth.make_decode_weights(cfg)
    wet = torch.from_numpy(np.concatenate(we)).to(dev)
    wnt = torch.from_numpy(np.concatenate(wn)).to(dev)
    he, hn = eg.egnn_hblocks(cfg.lmax, cfg.C, wet, wnt, r["eo"], r["xo"], storage=eg.EGNN_BF16)
    torch.cuda.synchronize()
    ei = torch.from_numpy(sample_rows(r["g"].n_edges, 3000, 15)).to(dev)
    ni = torch.from_numpy(sample_rows(r["s"].n_dst, 300, 16)).to(dev)
    eo = r["eo"][ei].float().cpu().numpy().astype(np.float64)
    xo = r["xo"][ni].float().cpu().numpy().astype(np.float64)
    assert_close(he[ei].cpu().numpy(), odec.hblocks(eo, we), 1e-5, "edge blocks")
    assert_close(hn[ni].cpu().numpy(), odec.hblocks(xo, wn), 1e-5, "on-site blocks")


@pytest.mark.parametrize("C,storage", [(32, "f32"), (32, "bf16"), (256, "f32"), (256, "bf16"), (8, "bf16")])
def test_hblocks_channel_counts(dev, C, storage):
    """Decode instantiations at C 32 and 256 (and bf16 at C 8): seeded irreps on
    the 64-atom cell's edge count, every block against the oracle at 1e-5."""
    rng = np.random.default_rng(C + (storage == "bf16"))
    E, N, lmax = 2836, 64, 4
    K = (lmax + 1) ** 2
    eo = synth.round_storage(rng.standard_normal((E, K, C)), storage)
    xo = synth.round_storage(rng.standard_normal((N, K, C)), storage)
    cfg = dataclasses.replace(synth.CONFIGS["tiny_l4"], C=C)
    we, wn = synth.make_decode_weights(cfg)
    dt = torch.bfloat16 if storage == "bf16" else torch.float32
    st = eg.EGNN_BF16 if storage == "bf16" else eg.EGNN_F32
    he, hn = eg.egnn_hblocks(lmax, C, torch.from_numpy(np.concatenate(we)).to(dev),
                             torch.from_numpy(np.concatenate(wn)).to(dev),
                             torch.from_numpy(eo).to(dev).to(dt), torch.from_numpy(xo).to(dev).to(dt), storage=st)
    torch.cuda.synchronize()
    assert_close(he.cpu().numpy(), odec.hblocks(eo.astype(np.float64), we), 1e-5, "edge blocks")
    assert_close(hn.cpu().numpy(), odec.hblocks(xo.astype(np.float64), wn), 1e-5, "on-site blocks")


@pytest.mark.parametrize("name,onsite", [("tiny", True), ("tiny", False), ("open_ghosts", True), ("hfo2", True)])
def test_assemble_bsr(dev, name, onsite):
    """Periodic Label -> Matrix: seeded 13 x 13 blocks on the graph's edges (and
    on-site blocks) into one block-sparse row structure over all image shifts,
    bit-exact against the oracle's sort of the same blocks (a pure gather)."""
    from tests.test_gpu_variants import OPEN_SPARSE
    s = synth.make_structure(OPEN_SPARSE if name == "open_ghosts" else synth.CONFIGS[name])
    g = gpu_graph(s, dev)
    og = oracle_graph(s)
    gg = host(g)
    np.testing.assert_array_equal(gg["src"], og["src"])
    n = 13
    E = g.n_edges
    he = synth.make_label_values(70, E, n * n).reshape(E, n, n)
    hn = synth.make_label_values(71, s.n_dst, n * n).reshape(s.n_dst, n, n) if onsite else None
    rp, col, sh, val = eg.egnn_assemble_bsr(g, torch.from_numpy(he).to(dev),
                                            torch.from_numpy(hn).to(dev) if onsite else None)
    torch.cuda.synchronize()
    dst = onb.dst_of_edges(og["row_ptr"])
    ref = odec.assemble_bsr(og["src"], dst, og["shift"], he,
                            hn if onsite else np.zeros((0, n, n), np.float32), s.n_src)
    np.testing.assert_array_equal(rp.cpu().numpy(), ref[0])
    np.testing.assert_array_equal(col.cpu().numpy(), ref[1])
    np.testing.assert_array_equal(sh.cpu().numpy(), ref[2])
    np.testing.assert_array_equal(val.cpu().numpy(), ref[3])


def test_layer_backward_halo_full_size_masked_rows(dev):
    """One GPU's share at full size (30,000 owned rows, 21,133 ghost sources,
    open boundary, 3.15M edges, fp32): the backward with the cotangent on 150
    rows spread over the row range, every weight block and grad x of every
    atom (ghosts included: they receive gradient only through their outgoing
    edges) against the oracle's exact values."""
    cfg = synth.CONFIGS["halo"]
    r = _gpu_forward(cfg, dev, train=True)
    assert r["g"].n_src > r["g"].n_dst
    rows = np.unique(np.linspace(0, r["s"].n_dst - 1, 150).round().astype(np.int64))
    _compare_full_backward(cfg, r, dev, rows, 1e-4)
