"""Pins of the edge-update block: the update is the node block's per-edge
message added to the edge embedding, it is equivariant, and its analytic
backward matches finite differences on every input and weight block."""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation as Rot

import synth
from oracle import layer, neighbors, so3


def _setup(name):
    cfg = synth.CONFIGS[name]
    s = synth.make_structure(cfg)
    g = neighbors.build_graph(s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut)
    x, ws = synth.make_layer_inputs(cfg)
    d = layer.LayerDesc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut)
    e = synth.make_edge_embeddings(cfg, len(g["src"])).astype(np.float64)
    return cfg, s, g, x.astype(np.float64), e, ws[0].astype(np.float64), d


def _rot(a, Q, lmax):
    out = np.empty_like(a)
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        out[:, sl, :] = np.einsum("mn,enc->emc", so3.wigner_d(l, Q), a[:, sl, :])
    return out


def test_update_is_the_node_blocks_message():
    cfg, s, g, x, e, w, d = _setup("tiny_l4")
    out = layer.edge_update_forward(g, x, e, w, d)
    node = layer.layer_forward(g, x, w, d)
    np.testing.assert_allclose(out["e_out"] - e, node["edge_out"], atol=1e-12)
    # and the attention weights play no part: changing them leaves e' alone
    W = layer.unpack_weights(w, d)
    W["w_att"] = W["w_att"] + 1.0
    out2 = layer.edge_update_forward(g, x, e, layer.pack_weights(W, d), d)
    np.testing.assert_allclose(out2["e_out"], out["e_out"], atol=1e-13)


@pytest.mark.parametrize("name", ["tiny", "tiny_l4"])
def test_edge_update_equivariance(name):
    cfg, s, g, x, e, w, d = _setup(name)
    base = layer.edge_update_forward(g, x, e, w, d)["e_out"]
    for seed in (4, 5):
        Q = Rot.random(random_state=seed).as_matrix()
        g2 = dict(g, vec=g["vec"].astype(np.float64) @ Q.T)
        out = layer.edge_update_forward(g2, _rot(x, Q, d.lmax), _rot(e, Q, d.lmax), w, d)["e_out"]
        np.testing.assert_allclose(out, _rot(base, Q, d.lmax), atol=1e-9)


def _loss(g, x, e, w, d, Ge):
    return float(np.sum(layer.edge_update_forward(g, x, e, w, d)["e_out"] * Ge))


@pytest.mark.parametrize("name", ["tiny", "tiny_l4"])
def test_edge_backward_matches_finite_differences(name):
    cfg, s, g, x, e, w, d = _setup(name)
    Ge = synth.make_edge_cotangent(cfg, len(g["src"])).astype(np.float64)
    fwd = layer.edge_update_forward(g, x, e, w, d)
    dx, de, dw = layer.edge_update_backward(g, x, w, d, fwd, Ge)
    rng = np.random.default_rng(9)
    o = 0
    for name_b, shape in synth.layer_weight_sizes(d.lmax, d.mmax, d.C, d.n_rbf):
        n = int(np.prod(shape))
        sl = slice(o, o + n)
        o += n
        v = np.zeros_like(w)
        v[sl] = rng.standard_normal(n)
        h = 1e-6 * max(1.0, np.abs(w[sl]).max())
        fd = (_loss(g, x, e, w + h * v, d, Ge) - _loss(g, x, e, w - h * v, d, Ge)) / (2 * h)
        an = float(dw @ v)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name_b, fd, an)
        if name_b == "w_att":
            assert np.all(dw[sl] == 0)
    for _ in range(2):
        v = rng.standard_normal(x.shape)
        h = 1e-6 * max(1.0, np.abs(x).max())
        fd = (_loss(g, x + h * v, e, w, d, Ge) - _loss(g, x - h * v, e, w, d, Ge)) / (2 * h)
        an = float(np.sum(dx * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
    v = rng.standard_normal(e.shape)
    fd = (_loss(g, x, e + 1e-6 * v, w, d, Ge) - _loss(g, x, e - 1e-6 * v, w, d, Ge)) / 2e-6
    assert abs(fd - np.sum(de * v)) <= 1e-6 * max(1.0, abs(fd))
