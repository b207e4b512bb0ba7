"""Pins of the oracle layer: brute-force SO(3) tensor-product convolution, equivariance,
roll independence, permutation invariance, softmax structure and finite differences."""
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
    return cfg, s, g, x.astype(np.float64), ws[0].astype(np.float64), d


def test_so2_conv_equals_bruteforce_so3_tensor_product():
    """eSCN reduction (MALOQ Sec. II-B1): in the edge frame the SO(3) CG tensor
    product of x with the edge's spherical harmonics is an SO(2) convolution.

    Global-frame TP:  y[lo] = sum_{li,lf} w_{li lf lo} Q^{(li,lf,lo)}(x[li], Y^lf(r)).
    In the edge frame Y^lf = delta_{mf,0} sqrt((2lf+1)/4pi); Q[mi, 0, M] couples
    mi = M (even li+lf+lo) and mi = -M (odd), which gives W_m1 and W_m2 of the
    SO(2) map.  The edge-frame path rotated back must equal the global TP.
    """
    L = 2
    d = layer.LayerDesc(lmax=L, mmax=L, C=3, n_rbf=8, r_cut=5.0)
    Cin, Cout = 2 * d.C, d.C
    rng = np.random.default_rng(0)
    E = 40
    vec = rng.standard_normal((E, 3)) * 2.0
    x = rng.standard_normal((E, d.K, Cin))
    paths = [(li, lf, lo) for li in range(L + 1) for lf in range(2 * L + 1) for lo in range(L + 1)
             if abs(li - lf) <= lo <= li + lf]
    w = {p: rng.standard_normal((Cout, Cin)) for p in paths}
    # global-frame tensor product
    r = vec / np.linalg.norm(vec, axis=1, keepdims=True)
    y_tp = np.zeros((E, d.K, Cout))
    for (li, lf, lo) in paths:
        Q = so3.real_coupling(li, lf, lo)
        sh = so3.real_sh(lf, r)
        xi = x[:, li * li:(li + 1) ** 2, :]
        t = np.einsum("ijM,eic,ej->eMc", Q, xi, sh)
        y_tp[:, lo * lo:(lo + 1) ** 2, :] += np.einsum("eMc,oc->eMo", t, w[(li, lf, lo)])
    # SO(2) weights derived from the paths
    W = {"W0": np.zeros(((L + 1) * Cout, (L + 1) * Cin))}
    for m in range(1, L + 1):
        nl = L - m + 1
        W[f"W{m}_1"] = np.zeros((nl * Cout, nl * Cin))
        W[f"W{m}_2"] = np.zeros((nl * Cout, nl * Cin))
    n_even = {}
    for (li, lf, lo) in paths:
        Q = so3.real_coupling(li, lf, lo)
        yf = np.sqrt((2 * lf + 1) / (4 * np.pi))
        even = (li + lf + lo) % 2 == 0
        for m in range(0, min(li, lo) + 1):
            pp, mm = Q[li + m, lf, lo + m], Q[li - m, lf, lo - m]     # mi = M couplings
            pm, mp = Q[li + m, lf, lo - m], Q[li - m, lf, lo + m]     # mi = -M couplings
            if m == 0:
                assert abs(pm) < 1e-12 or even
                if not even:
                    assert abs(pp) < 1e-12
                blk = W["W0"]
                blk[lo * Cout:(lo + 1) * Cout, li * Cin:(li + 1) * Cin] += pp * yf * w[(li, lf, lo)]
                continue
            ro, ci = (lo - m) * Cout, (li - m) * Cin
            if even:
                assert abs(pm) < 1e-12 and abs(mp) < 1e-12
                np.testing.assert_allclose(pp, mm, atol=1e-12)
                W[f"W{m}_1"][ro:ro + Cout, ci:ci + Cin] += pp * yf * w[(li, lf, lo)]
                n_even[(li, lo, m)] = n_even.get((li, lo, m), 0) + 1
            else:
                assert abs(pp) < 1e-12 and abs(mm) < 1e-12
                np.testing.assert_allclose(pm, -mp, atol=1e-12)
                W[f"W{m}_2"][ro:ro + Cout, ci:ci + Cin] += pm * yf * w[(li, lf, lo)]
    # the edge-frame SO(2) path of the oracle, rotated back
    D = layer.edge_wigner(vec, L)
    y_so2 = layer.rotate_out(D, layer.so2_conv(layer.rotate_in(D, x, d), W, d), d)
    np.testing.assert_allclose(y_so2, y_tp, atol=1e-11)
    assert np.abs(y_tp).max() > 0.1


def _rotate_irreps(a, Q, lmax):
    out = np.empty_like(a)
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) ** 2)
        out[:, sl, :] = np.einsum("mn,enc->emc", so3.wigner_d(l, Q), a[:, sl, :])
    return out


@pytest.mark.parametrize("name", ["tiny", "tiny_l4", "tiny_l6"])
def test_layer_equivariance(name):
    cfg, s, g, x, w, d = _setup(name)
    base = layer.layer_forward(g, x, w, d)
    for seed in (1, 2):
        Q = Rot.random(random_state=seed).as_matrix()
        g2 = dict(g, vec=g["vec"].astype(np.float64) @ Q.T)
        out = layer.layer_forward(g2, _rotate_irreps(x, Q, d.lmax), w, d)
        np.testing.assert_allclose(out["x_out"], _rotate_irreps(base["x_out"], Q, d.lmax), atol=1e-9)
        np.testing.assert_allclose(out["edge_out"], _rotate_irreps(base["edge_out"], Q, d.lmax), atol=1e-9)
        np.testing.assert_allclose(out["alpha"], base["alpha"], atol=1e-12)


def test_layer_roll_independent():
    cfg, s, g, x, w, d = _setup("tiny_l4")
    base = layer.layer_forward(g, x, w, d)
    roll = np.random.default_rng(3).uniform(-np.pi, np.pi, len(g["src"]))
    out = layer.layer_forward(g, x, w, d, roll=roll)
    np.testing.assert_allclose(out["x_out"], base["x_out"], atol=1e-12)
    np.testing.assert_allclose(out["edge_out"], base["edge_out"], atol=1e-12)


def test_layer_permutation_invariance():
    cfg, s, g, x, w, d = _setup("tiny")
    base = layer.layer_forward(g, x, w, d)
    perm = np.random.default_rng(5).permutation(s.n_dst)
    g2 = neighbors.build_graph(s.pos[perm], s.n_dst, s.box, s.periodic_mask, s.r_cut)
    out = layer.layer_forward(g2, x[perm], w, d)
    np.testing.assert_allclose(out["x_out"], base["x_out"][perm], atol=1e-13)
    # shuffle edges inside every row: x' unchanged, edge outputs follow the edges
    rp = g["row_ptr"]
    rng = np.random.default_rng(6)
    idx = np.concatenate([rp[r] + rng.permutation(rp[r + 1] - rp[r]) for r in range(s.n_dst)])
    g3 = dict(g, src=g["src"][idx], shift=g["shift"][idx], vec=g["vec"][idx], dist=g["dist"][idx])
    out3 = layer.layer_forward(g3, x, w, d)
    np.testing.assert_allclose(out3["x_out"], base["x_out"], atol=1e-13)
    np.testing.assert_allclose(out3["edge_out"], base["edge_out"][idx], atol=1e-13)


def test_softmax_rows_and_degenerate_rows():
    cfg, s, g, x, w, d = _setup("tiny")
    out = layer.layer_forward(g, x, w, d)
    sums = np.add.reduceat(out["alpha"], g["row_ptr"][:-1])
    np.testing.assert_allclose(sums, 1.0, atol=1e-13)
    # 3 atoms, open boundary: 0 <-> 1 within the cutoff, 2 isolated
    pos = np.array([[0.0, 0.0, 0.0], [1.2, 1.0, -0.7], [20.0, 0.0, 0.0]])
    g2 = neighbors.build_graph(pos, 3, np.array([30.0, 30.0, 30.0]), 0, cfg.r_cut)
    assert list(np.diff(g2["row_ptr"])) == [1, 1, 0]
    out2 = layer.layer_forward(g2, x[:3], w, d)
    np.testing.assert_allclose(out2["alpha"], 1.0)
    np.testing.assert_allclose(out2["x_out"][2], x[2])
    np.testing.assert_allclose(out2["x_out"][0], x[0] + out2["edge_out"][0], atol=1e-14)


def _loss(g, x, w, d, G):
    return float(np.sum(layer.layer_forward(g, x, w, d)["x_out"] * G))


@pytest.mark.parametrize("name", ["tiny", "tiny_l4", "tiny_l6"])
def test_backward_matches_finite_differences(name):
    cfg, s, g, x, w, d = _setup(name)
    G = synth.make_cotangent(cfg, s.n_dst).astype(np.float64)
    fwd = layer.layer_forward(g, x, w, d)
    dx, dw = layer.layer_backward(g, x, w, d, fwd, G)
    rng = np.random.default_rng(7)
    blocks = {}
    o = 0
    for name_b, shape in synth.layer_weight_sizes(d.lmax, d.mmax, d.C, d.n_rbf):
        n = int(np.prod(shape))
        blocks[name_b] = slice(o, o + n)
        o += n
    assert o == w.size
    # directional derivatives, one random direction per weight block and two for x
    for name_b, sl in blocks.items():
        v = np.zeros_like(w)
        v[sl] = rng.standard_normal(sl.stop - sl.start)
        h = 1e-6 * max(1.0, np.abs(w[sl]).max())
        fd = (_loss(g, x, w + h * v, d, G) - _loss(g, x, w - h * v, d, G)) / (2 * h)
        an = float(dw @ v)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name_b, fd, an)
    for _ in range(2):
        v = rng.standard_normal(x.shape)
        h = 1e-6 * max(1.0, np.abs(x).max())
        fd = (_loss(g, x + h * v, w, d, G) - _loss(g, x - h * v, w, d, G)) / (2 * h)
        an = float(np.sum(dx * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
    # a few single coordinates of w and x
    for i in rng.choice(w.size, 4, replace=False):
        e = np.zeros_like(w)
        e[i] = 1.0
        h = 1e-6
        fd = (_loss(g, x, w + h * e, d, G) - _loss(g, x, w - h * e, d, G)) / (2 * h)
        assert abs(fd - dw[i]) <= 1e-6 * max(1.0, abs(dw[i])), (i, fd, dw[i])


def test_backward_with_ghost_sources():
    """Open boundary, ghosts after the owned rows: gradients reach ghost rows only through edges."""
    rng = np.random.default_rng(8)
    pos = rng.random((40, 3)) * np.array([10.0, 10.0, 6.0])
    n_dst = 25
    d = layer.LayerDesc(lmax=2, mmax=1, C=4, n_rbf=8, r_cut=4.0)
    g = neighbors.build_graph(pos, n_dst, np.array([10.0, 10.0, 6.0]), 0, d.r_cut)
    x = rng.standard_normal((40, d.K, d.C))
    n_w = sum(int(np.prod(sh)) for _, sh in synth.layer_weight_sizes(d.lmax, d.mmax, d.C, d.n_rbf))
    w = rng.standard_normal(n_w) * 0.3
    G = rng.standard_normal((n_dst, d.K, d.C))
    fwd = layer.layer_forward(g, x, w, d)
    dx, dw = layer.layer_backward(g, x, w, d, fwd, G)
    assert fwd["x_out"].shape == (n_dst, d.K, d.C)
    for _ in range(2):
        v = rng.standard_normal(x.shape)
        h = 1e-6
        fd = (_loss(g, x + h * v, w, d, G) - _loss(g, x - h * v, w, d, G)) / (2 * h)
        assert abs(fd - np.sum(dx * v)) <= 1e-6 * max(1.0, abs(fd))
        v = rng.standard_normal(w.shape)
        fd = (_loss(g, x, w + h * v, d, G) - _loss(g, x, w - h * v, d, G)) / (2 * h)
        assert abs(fd - dw @ v) <= 1e-6 * max(1.0, abs(fd))


@pytest.mark.parametrize("n_rbf,r_cut", [(8, 5.0), (8, 10.0), (4, 6.0), (16, 8.0)])
def test_radial_basis_closed_forms(n_rbf, r_cut):
    """Reading R11 worked by hand, with no call into the oracle for the expected
    values: n Gaussians with centres k r_c/(n-1) and width r_c/(n-1), times the
    cosine envelope (1 + cos(pi d / r_c))/2.  So at d = 0 the envelope is 1 and
    phi_k = exp(-k^2/2); at its own centre phi_k equals the envelope there; one
    width either side it is exp(-1/2) times the envelope; the envelope is 1/2 at
    r_c/2 and 0 at r_c.  A different width, centre spacing or envelope (e.g.
    sigma = r_c/n, or cos(pi d / 2r_c)) fails one of these."""
    import math
    d = layer.LayerDesc(2, 2, 8, n_rbf, r_cut)
    phi0 = layer.radial_basis(np.array([0.0]), d)[0]
    np.testing.assert_allclose(phi0, [math.exp(-k * k / 2.0) for k in range(n_rbf)], rtol=1e-12, atol=0)
    step = r_cut / (n_rbf - 1)
    for k in range(n_rbf):
        mu = k * step
        env = 0.5 * (1.0 + math.cos(math.pi * mu / r_cut))
        got = layer.radial_basis(np.array([mu]), d)[0]
        assert abs(got[k] - env) <= 1e-14
        # neighbouring centres sit one width away
        if k + 1 < n_rbf:
            assert abs(got[k + 1] - math.exp(-0.5) * env) <= 1e-14
        if k > 0:
            assert abs(got[k - 1] - math.exp(-0.5) * env) <= 1e-14
        for sgn in (-1.0, 1.0):
            r = mu + sgn * step
            if 0.0 <= r <= r_cut:
                e2 = 0.5 * (1.0 + math.cos(math.pi * r / r_cut))
                assert abs(layer.radial_basis(np.array([r]), d)[0][k] - math.exp(-0.5) * e2) <= 1e-14
    half = layer.radial_basis(np.array([r_cut / 2]), d)[0]
    np.testing.assert_allclose(half, [0.5 * math.exp(-((r_cut / 2 - k * step) ** 2) / (2 * step * step))
                                      for k in range(n_rbf)], rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(layer.radial_basis(np.array([r_cut]), d)[0], 0.0, atol=1e-15)


def _open_cell_with_ghosts():
    rng = np.random.default_rng(8)
    pos = rng.random((40, 3)) * np.array([10.0, 10.0, 6.0])
    n_dst = 25
    d = layer.LayerDesc(lmax=2, mmax=1, C=4, n_rbf=8, r_cut=4.0)
    x = rng.standard_normal((40, d.K, d.C))
    n_w = sum(int(np.prod(sh)) for _, sh in synth.layer_weight_sizes(d.lmax, d.mmax, d.C, d.n_rbf))
    w = rng.standard_normal(n_w) * 0.3
    return pos, n_dst, np.array([10.0, 10.0, 6.0]), d, x, w


@pytest.mark.parametrize("case", ["tiny", "tiny_l4", "open_ghosts"])
@pytest.mark.parametrize("chunk_edges", [1, 150, 16384])
def test_forward_rows_equals_forward(case, chunk_edges):
    """The chunked, row-sampled forward used at full size gives the same x' and
    alpha as the whole-graph forward: on all rows, and on a subset of rows built
    alone (as the large-structure parity tests build them)."""
    if case == "open_ghosts":
        pos, n_dst, box, d, x, w = _open_cell_with_ghosts()
        mask, rc = 0, d.r_cut
    else:
        cfg, s, _, x, w, d = _setup(case)
        pos, n_dst, box, mask, rc = s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut
    g = neighbors.build_graph(pos, n_dst, box, mask, rc)
    ref = layer.layer_forward(g, x, w, d)
    xo, alpha = layer.layer_forward_rows(g, x, w, d, chunk_edges=chunk_edges)
    np.testing.assert_allclose(xo, ref["x_out"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(alpha, ref["alpha"], rtol=0, atol=1e-13)
    rows = np.sort(np.random.default_rng(17).choice(n_dst, size=n_dst // 3, replace=False))
    gs = neighbors.build_graph(pos, n_dst, box, mask, rc, rows=rows)
    xs, alpha_s = layer.layer_forward_rows(gs, x, w, d, chunk_edges=chunk_edges)
    np.testing.assert_allclose(xs, ref["x_out"][rows], rtol=0, atol=1e-13)
    sel = np.concatenate([np.arange(g["row_ptr"][r], g["row_ptr"][r + 1]) for r in rows])
    np.testing.assert_allclose(alpha_s, ref["alpha"][sel], rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", ["tiny", "open_ghosts"])
def test_aggregation_equals_dense_adjacency_product(case):
    """Attention and aggregation as dense matrix algebra: each edge's destination is
    found from geometry alone (the atom at x_src + S L + vec), the logits fill an
    [n_dst][E] matrix with -inf off the adjacency, scipy's softmax along each row
    gives alpha, and x' - x is that matrix times the per-edge messages.  This
    checks the CSR segment softmax and segment sum (and empty rows) independently."""
    from scipy.special import softmax
    if case == "open_ghosts":
        pos, n_dst, box, d, x, w = _open_cell_with_ghosts()
        pos = pos.copy()
        pos[3] = [30.0, 30.0, 30.0]                               # an owned atom with no neighbour
        mask, rc = 0, d.r_cut
    else:
        cfg, s, _, x, w, d = _setup(case)
        pos, n_dst, box, mask, rc = s.pos, s.n_dst, s.box, s.periodic_mask, s.r_cut
    g = neighbors.build_graph(pos, n_dst, box, mask, rc)
    out = layer.layer_forward(g, x, w, d)
    E = len(g["src"])
    tip = pos[g["src"]] + g["shift"].astype(np.float64) * box + g["vec"].astype(np.float64)
    d2 = ((tip[:, None, :] - pos[None, :n_dst, :]) ** 2).sum(-1)
    dst = np.argmin(d2, axis=1)
    assert np.sqrt(d2[np.arange(E), dst]).max() < 1e-5          # the tip lands on an owned atom
    A = np.full((n_dst, E), -np.inf)
    A[dst, np.arange(E)] = out["logits"]
    has = np.isfinite(A).any(axis=1)
    alpha = np.zeros_like(A)
    alpha[has] = softmax(A[has], axis=1)
    np.testing.assert_allclose(alpha[dst, np.arange(E)], out["alpha"], rtol=0, atol=1e-14)
    agg = (alpha @ out["msg"].reshape(E, -1)).reshape(n_dst, d.K, d.C)
    np.testing.assert_allclose(out["x_out"] - x[:n_dst], agg, rtol=0, atol=1e-12)
    if case == "open_ghosts":
        assert (~has).any()
        np.testing.assert_array_equal(out["x_out"][~has], x[:n_dst][~has])
