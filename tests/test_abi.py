"""C ABI checks that need no GPU: every declared symbol is exported, host-side
size queries agree with the documented layouts, and invalid arguments are
rejected on the host with a status and a message (nothing is launched)."""
import ctypes as ct
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "egnn.h")


@pytest.fixture(scope="module")
def lib():
    from equivariant_gnn_electronic_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from equivariant_gnn_electronic_amd import build
        build.build(verbose=False)
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(egnn_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    from equivariant_gnn_electronic_amd import _lib
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), f"{n} declared in egnn.h but not exported"
    # and the binding declares a signature for each of them
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_status_strings(lib):
    assert lib.egnn_version() >= 100
    for code in range(6):
        assert lib.egnn_status_string(code)
    assert lib.egnn_status_string(99) == b"unknown status"


def _desc(lmax, mmax, C, n_rbf=8, r_cut=5.0, storage=0):
    from equivariant_gnn_electronic_amd import _lib
    return _lib.EgnnLayerDesc(lmax, mmax, C, n_rbf, r_cut, storage)


@pytest.mark.parametrize("name", ["tiny", "tiny_l4", "hfo2", "gst", "halo"])
def test_weight_count_matches_packed_layout(lib, name):
    cfg = synth.CONFIGS[name]
    d = _desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut)
    n = sum(int(a * b) for _, (a, b) in synth.layer_weight_sizes(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf))
    assert lib.egnn_layer_weight_count(ct.byref(d)) == n


def test_geom_stride(lib):
    # rows |m| <= mmax of D^l for l <= lmax, then n_rbf, then the destination, padded to 16
    for lmax, mmax in [(1, 0), (2, 2), (3, 1), (4, 2), (4, 0), (6, 2), (8, 1)]:
        nd = sum((2 * min(l, mmax) + 1) * (2 * l + 1) for l in range(lmax + 1))
        d = _desc(lmax, mmax, 16)
        assert lib.egnn_geom_stride(ct.byref(d)) == (nd + 8 + 1 + 15) // 16 * 16
    assert lib.egnn_geom_stride(ct.byref(_desc(4, 2, 64))) == 128   # 115 Wigner rows + 8 + 1, padded


@pytest.mark.parametrize("bad", [dict(lmax=5), dict(lmax=7), dict(lmax=9), dict(lmax=0), dict(mmax=3), dict(C=12), dict(C=0),
                                 dict(n_rbf=1), dict(n_rbf=17), dict(storage=7)])
def test_invalid_layer_desc_rejected(lib, bad):
    from equivariant_gnn_electronic_amd import _lib
    kw = dict(lmax=4, mmax=2, C=64, n_rbf=8, r_cut=8.0, storage=0)
    kw.update(bad)
    d = _lib.EgnnLayerDesc(kw["lmax"], kw["mmax"], kw["C"], kw["n_rbf"], kw["r_cut"], kw["storage"])
    assert lib.egnn_layer_weight_count(ct.byref(d)) == 0
    g = _fake_graph(10, 10, 100)
    st = lib.egnn_layer_fwd(ct.byref(d), ct.byref(g), None, None, None, None, None, None, None, 0, None)
    assert st == _lib.EGNN_E_ARG
    assert b"invalid layer description" in lib.egnn_last_error()


def _fake_graph(n_dst, n_src, E):
    """A graph struct with placeholder (never dereferenced) device pointers."""
    from equivariant_gnn_electronic_amd import _lib
    g = _lib.EgnnGraph()
    g.n_dst, g.n_src, g.capacity, g.n_edges = n_dst, n_src, E, E
    for f in ("row_ptr", "src", "shift", "vec", "dist", "src_ptr", "src_perm"):
        setattr(g, f, 0x1000)
    return g


def test_layer_sizes_scale_with_edges(lib):
    d = _desc(4, 2, 64)
    sizes = []
    for E in (1000, 2000):
        s, f, b = ct.c_size_t(), ct.c_size_t(), ct.c_size_t()
        g = _fake_graph(100, 100, E)
        assert lib.egnn_layer_sizes(ct.byref(d), ct.byref(g), ct.byref(s), ct.byref(f), ct.byref(b)) == 0
        sizes.append((s.value, f.value, b.value))
    # saved = A_m + Y_m + alpha per edge: (19*2C + 19*C) * 4 + 4 bytes at C=64 (plus alignment)
    per_edge = (19 * 128 + 19 * 64) * 4 + 4
    assert abs((sizes[1][0] - sizes[0][0]) - 1000 * per_edge) < 8 * 256
    assert sizes[1][1] > sizes[0][1] and sizes[1][2] > sizes[0][2]


def test_graph_argument_checks(lib):
    from equivariant_gnn_electronic_amd import _lib
    lo = (ct.c_double * 3)(0, 0, 0)
    box = (ct.c_double * 3)(10, 10, 10)
    nb = ct.c_size_t()
    assert lib.egnn_build_graph_workspace(10, 20, lo, box, 7, 3.0, 100, ct.byref(nb)) == 0 and nb.value > 0
    nb0 = ct.c_size_t()
    lib.egnn_build_graph_workspace(10, 20, lo, box, 7, 3.0, 0, ct.byref(nb0))
    assert nb.value - nb0.value >= 100 * 8 - 256    # the key buffer grows with capacity (256 B alignment)
    assert lib.egnn_build_graph_workspace(30, 20, lo, box, 7, 3.0, 0, ct.byref(nb)) == _lib.EGNN_E_ARG
    assert lib.egnn_build_graph_workspace(10, 20, lo, box, 8, 3.0, 0, ct.byref(nb)) == _lib.EGNN_E_ARG
    bad_box = (ct.c_double * 3)(10, 0, 10)
    assert lib.egnn_build_graph_workspace(10, 20, lo, bad_box, 7, 3.0, 0, ct.byref(nb)) == _lib.EGNN_E_ARG
    g = _fake_graph(10, 20, 0)
    g.capacity = 50
    g.src = None  # capacity > 0 needs the edge arrays
    st = lib.egnn_build_graph(ct.c_void_p(0x1000), lo, box, 7, 3.0, ct.byref(g), ct.c_void_p(0x1000),
                              1 << 30, None)
    assert st == _lib.EGNN_E_ARG and b"edge arrays" in lib.egnn_last_error()
    g = _fake_graph(10, 20, 0)
    st = lib.egnn_build_graph(ct.c_void_p(0x1000), lo, box, 7, 3.0, ct.byref(g), None, 0, None)
    assert st == _lib.EGNN_E_WORKSPACE


def test_backward_rejects_unsupported_width(lib):
    from equivariant_gnn_electronic_amd import _lib
    d = _desc(4, 2, 256, storage=1)  # the backward handles C <= 128
    g = _fake_graph(10, 10, 100)
    p = ct.c_void_p(0x1000)
    st = lib.egnn_layer_bwd(ct.byref(d), ct.byref(g), p, p, p, p, p, p, p, p, 1 << 30, None)
    assert st == _lib.EGNN_E_UNSUPPORTED


def test_workspace_too_small_rejected(lib):
    from equivariant_gnn_electronic_amd import _lib
    d = _desc(4, 2, 64)
    g = _fake_graph(10, 10, 100)
    p = ct.c_void_p(0x1000)
    st = lib.egnn_layer_fwd(ct.byref(d), ct.byref(g), p, p, p, ct.c_void_p(0x2000), None, None, p, 16, None)
    assert st == _lib.EGNN_E_WORKSPACE
    assert b"workspace" in lib.egnn_last_error()
    st = lib.egnn_layer_fwd(ct.byref(d), ct.byref(g), p, p, p, p, None, None, p, 1 << 40, None)
    assert st == _lib.EGNN_E_ARG   # x_out aliases x_in


def test_misaligned_workspace_rejected(lib):
    """The split-K weight-gradient product reads the saved tensors with 16-byte
    loads, so ws and saved must be 16-byte aligned; the host check says so."""
    from equivariant_gnn_electronic_amd import _lib
    d = _desc(4, 2, 64, storage=1)
    g = _fake_graph(10, 10, 100)
    p = ct.c_void_p(0x1000)
    odd = ct.c_void_p(0x1008)
    st = lib.egnn_layer_fwd(ct.byref(d), ct.byref(g), p, p, p, ct.c_void_p(0x2000), None, None, odd, 1 << 40, None)
    assert st == _lib.EGNN_E_ARG
    assert b"aligned" in lib.egnn_last_error()
    st = lib.egnn_layer_bwd(ct.byref(d), ct.byref(g), p, p, p, odd, p, p, p, p, 1 << 40, None)
    assert st == _lib.EGNN_E_ARG


def test_decode_description_checks(lib):
    from equivariant_gnn_electronic_amd import _lib
    arr = (ct.c_int32 * 5)(0, 0, 1, 1, 2)
    h = _lib.EgnnHDesc(4, 64, 5, arr, 0)
    assert lib.egnn_hblocks_label_rows(ct.byref(h)) == 9 + 17 + 13 + 5 + 1
    h_small = _lib.EgnnHDesc(3, 64, 5, arr, 0)          # lmax must cover 2 * max shell l
    assert lib.egnn_hblocks_label_rows(ct.byref(h_small)) == 0
    assert lib.egnn_hblocks(ct.byref(h_small), 1, 1, None, None, None, None, None, None, None) == _lib.EGNN_E_ARG
    arr3 = (ct.c_int32 * 1)(3)                            # f x f: one label channel for each L = 0..6
    assert lib.egnn_hblocks_label_rows(ct.byref(_lib.EgnnHDesc(8, 64, 1, arr3, 0))) == 7
    assert lib.egnn_hblocks_label_rows(ct.byref(_lib.EgnnHDesc(6, 64, 1, arr3, 0))) == 7
    assert lib.egnn_hblocks_label_rows(ct.byref(_lib.EgnnHDesc(4, 64, 1, arr3, 0))) == 0   # lmax < 6
    arr4 = (ct.c_int32 * 1)(4)                            # g x g: one label channel for each L = 0..8
    assert lib.egnn_hblocks_label_rows(ct.byref(_lib.EgnnHDesc(8, 64, 1, arr4, 0))) == 9
    assert lib.egnn_hblocks_label_rows(ct.byref(_lib.EgnnHDesc(6, 64, 1, arr4, 0))) == 0   # lmax < 8
    arr_g = (ct.c_int32 * 5)(0, 1, 2, 3, 4)               # s p d f g
    assert lib.egnn_hblocks_label_rows(ct.byref(_lib.EgnnHDesc(8, 16, 5, arr_g, 0))) == 85
    arr5 = (ct.c_int32 * 1)(5)                            # h shells are not supported
    assert lib.egnn_hblocks_label_rows(ct.byref(_lib.EgnnHDesc(8, 64, 1, arr5, 0))) == 0
    # nothing to do is fine
    assert lib.egnn_hblocks(ct.byref(h), 0, 0, None, None, None, None, None, None, None) == 0


def test_decode_rejects_misaligned_irreps(lib):
    """The decode reads each lane's channel run with 16-byte loads; the host
    check rejects irreps that are not 16-byte aligned before anything runs."""
    from equivariant_gnn_electronic_amd import _lib
    arr = (ct.c_int32 * 5)(0, 0, 1, 1, 2)
    h = _lib.EgnnHDesc(4, 64, 5, arr, 1)
    p = ct.c_void_p(0x1000)
    odd = ct.c_void_p(0x1008)
    st = lib.egnn_hblocks(ct.byref(h), 10, 0, p, None, odd, None, p, None, None)
    assert st == _lib.EGNN_E_ARG and b"aligned" in lib.egnn_last_error()
    st = lib.egnn_hblocks(ct.byref(h), 0, 4, None, p, None, odd, None, p, None)
    assert st == _lib.EGNN_E_ARG and b"aligned" in lib.egnn_last_error()


def test_timing_collect_without_events(lib):
    from equivariant_gnn_electronic_amd import _lib
    out = (_lib.EgnnTimingEntry * 4)()
    dropped = ct.c_int64(-1)
    lib.egnn_timing_reset()
    assert lib.egnn_timing_collect(out, 4, ct.byref(dropped)) == 0
    assert dropped.value == 0


def test_binding_refuses_host_tensors():
    import torch

    import equivariant_gnn_electronic_amd as eg
    with pytest.raises(ValueError):
        eg._ptr(torch.zeros(3))


def _basis(shells, masks):
    from equivariant_gnn_electronic_amd import _lib
    l = (ct.c_int32 * len(shells))(*shells)
    m = (ct.c_uint32 * len(masks))(*masks)
    b = _lib.EgnnBasis(len(shells), l, len(masks), m)
    b._keep = (l, m)
    return b


def test_label_width_and_basis_checks(lib):
    """Host-side table build: n_full^2 labels; degrees above 3, more than 32
    orbitals or a mask naming a missing shell are refused (width 0)."""
    assert lib.egnn_label_width(ct.byref(_basis(synth.WATER_SHELLS, synth.WATER_MASKS))) == 16
    assert lib.egnn_label_width(ct.byref(_basis(synth.SVP_SHELLS, synth.SVP_MASKS))) == 18 * 18
    assert lib.egnn_label_width(ct.byref(_basis((0, 1, 2, 3), (0b1111,)))) == 16 * 16
    assert lib.egnn_label_width(ct.byref(_basis((0, 4), (0b11,)))) == 10 * 10
    assert lib.egnn_label_width(ct.byref(_basis(synth.G_SHELLS, synth.G_MASKS))) == 25 * 25
    assert lib.egnn_label_width(ct.byref(_basis((0, 5), (0b11,)))) == 0              # h shells
    assert lib.egnn_label_width(ct.byref(_basis((3, 3, 3, 3, 3), (0b1,)))) == 0     # 35 orbitals
    assert lib.egnn_label_width(ct.byref(_basis((0, 1), (0b111,)))) == 0
    assert lib.egnn_label_width(None) == 0


def test_label_calls_reject_bad_arguments(lib):
    from equivariant_gnn_electronic_amd import _lib
    b = _basis(synth.WATER_SHELLS, synth.WATER_MASKS)
    assert lib.egnn_orbital_layout(ct.byref(b), None, None, None) == _lib.EGNN_E_ARG
    o = _lib.EgnnOrbitals()
    o.n_mols, o.n_atoms = 1, 3
    assert lib.egnn_orbital_layout(ct.byref(b), ct.byref(o), None, None) == _lib.EGNN_E_ARG   # null arrays
    assert b"null" in lib.egnn_last_error()
    o.mol_ptr = o.species = o.atom_orb = o.atom_mol = o.mol_norb = o.mat_off = 16
    g = _lib.EgnnGraph()
    g.n_dst, g.n_src, g.n_edges = 4, 4, 0
    # the graph's rows must be the layout's atoms
    assert lib.egnn_matrix_to_label(ct.byref(b), ct.byref(o), ct.byref(g), 16, 9, 16, 16, None,
                                    None) == _lib.EGNN_E_ARG
    g.n_dst = g.n_src = 3
    # an empty matrix with blocks to fill
    assert lib.egnn_label_to_matrix(ct.byref(b), ct.byref(o), None, None, 16, 16, 0, None, None) == _lib.EGNN_E_ARG
    assert lib.egnn_matrix_to_label(ct.byref(b), ct.byref(o), None, None, 9, None, 16, None,
                                    None) == _lib.EGNN_E_ARG


def _cpu_graph(n_dst=6, n_src=8, E=20):
    import torch
    import equivariant_gnn_electronic_amd as eg
    rp = torch.linspace(0, E, n_dst + 1).round().to(torch.int32)
    return eg.Graph(n_dst, n_src, E, rp, torch.zeros(E, dtype=torch.int32), torch.zeros((E, 3), dtype=torch.int8),
                    torch.ones((E, 3)), torch.ones(E), torch.zeros(n_src + 1, dtype=torch.int32),
                    torch.zeros(E, dtype=torch.int32))


def _layer_args(storage=0, lmax=2, mmax=2, C=16):
    import torch
    import equivariant_gnn_electronic_amd as eg
    g = _cpu_graph()
    desc = eg.layer_desc(lmax, mmax, C, 8, 5.0, storage)
    K = (lmax + 1) ** 2
    dt = torch.bfloat16 if storage else torch.float32
    geom = torch.zeros((g.n_edges, eg.egnn_geom_stride(desc)))
    w = torch.zeros(eg.egnn_layer_weight_count(desc))
    x = torch.zeros((g.n_src, K, C), dtype=dt)
    return eg, g, desc, geom, w, x, K, C, dt


def test_binding_rejects_wrong_dtypes_and_shapes(lib):
    """The binding is the only guard against a buffer of the wrong type or size
    (the C ABI sees plain pointers): every wrapper raises before any call."""
    import torch
    eg, g, desc, geom, w, x, K, C, dt = _layer_args()
    buf = eg.LayerBuffers(desc, g, train=True)
    G = torch.zeros((g.n_dst, K, C))
    with pytest.raises(ValueError, match="grad_out"):
        eg.egnn_layer_bwd(desc, g, geom, w, x, buf, G.to(torch.bfloat16))
    with pytest.raises(ValueError, match="grad_out"):
        eg.egnn_layer_bwd(desc, g, geom, w, x, buf, G[:-1].contiguous())
    with pytest.raises(ValueError, match="grad_x"):
        eg.egnn_layer_bwd(desc, g, geom, w, x, buf, G, grad_x=torch.zeros((g.n_dst, K, C)))
    with pytest.raises(ValueError, match="grad_w"):
        eg.egnn_layer_bwd(desc, g, geom, w, x, buf, G, grad_w=torch.zeros(w.numel() - 1))
    with pytest.raises(ValueError, match="train=True"):
        eg.egnn_layer_bwd(desc, g, geom, w, x, eg.LayerBuffers(desc, g, train=False), G)
    with pytest.raises(ValueError, match="weights"):
        eg.egnn_layer_fwd(desc, g, geom, w[:-1].contiguous(), x)
    with pytest.raises(ValueError, match="weights"):
        eg.egnn_layer_fwd(desc, g, geom, w.double(), x)
    with pytest.raises(ValueError, match="x "):
        eg.egnn_layer_fwd(desc, g, geom, w, x[:-1].contiguous())
    with pytest.raises(ValueError, match="x "):
        eg.egnn_layer_fwd(desc, g, geom, w, x.to(torch.bfloat16))
    with pytest.raises(ValueError, match="geom"):
        eg.egnn_layer_fwd(desc, g, geom[:-1].contiguous(), w, x)
    with pytest.raises(ValueError, match="x_out"):
        eg.egnn_layer_fwd(desc, g, geom, w, x, x_out=torch.zeros((g.n_dst, K, C + 1)))
    with pytest.raises(ValueError, match="contiguous"):
        eg.egnn_layer_fwd(desc, g, geom, w, torch.zeros((g.n_src, C, K)).transpose(1, 2))
    # edge-update block: e_in / e_out in the storage type, grad_e_out fp32
    e = torch.zeros((g.n_edges, K, C))
    with pytest.raises(ValueError, match="e_in"):
        eg.egnn_edge_update_fwd(desc, g, geom, w, x, e.to(torch.bfloat16))
    with pytest.raises(ValueError, match="e_out"):
        eg.egnn_edge_update_fwd(desc, g, geom, w, x, e, e_out=e[:-1].contiguous())
    with pytest.raises(ValueError, match="grad_e_out"):
        eg.egnn_edge_update_bwd(desc, g, geom, w, x, buf, e.to(torch.bfloat16))
    # bf16 storage: x must be bf16, grads stay fp32
    eg, g, desc16, geom16, w16, x16, K, C, dt = _layer_args(storage=1)
    with pytest.raises(ValueError, match="x "):
        eg.egnn_layer_fwd(desc16, g, geom16, w16, x16.float())
    buf16 = eg.LayerBuffers(desc16, g, train=True)
    with pytest.raises(ValueError, match="grad_out"):
        eg.egnn_layer_bwd(desc16, g, geom16, w16, x16, buf16, torch.zeros((g.n_dst, K, C), dtype=torch.bfloat16))
    # everything right but on the host: the device check fires last
    with pytest.raises(ValueError, match="GPU"):
        eg.egnn_layer_bwd(desc16, g, geom16, w16, x16, buf16, torch.zeros((g.n_dst, K, C)))


def test_binding_rejects_wrong_decode_and_label_buffers(lib):
    import torch
    import equivariant_gnn_electronic_amd as eg
    lmax, C = 4, 16
    K = (lmax + 1) ** 2
    rows = eg.egnn_hblocks_label_rows(lmax, C)
    assert rows == 9 + 17 + 13 + 5 + 1
    we = torch.zeros(rows * C)
    eo = torch.zeros((10, K, C))
    xo = torch.zeros((4, K, C))
    with pytest.raises(ValueError, match="edge_irreps"):
        eg.egnn_hblocks(lmax, C, we, we, eo.to(torch.bfloat16), xo)
    with pytest.raises(ValueError, match="node_irreps"):
        eg.egnn_hblocks(lmax, C, we, we, eo, xo.to(torch.bfloat16))
    with pytest.raises(ValueError, match="edge_irreps"):
        eg.egnn_hblocks(lmax, C, we, we, eo, xo, storage=eg.EGNN_BF16)
    with pytest.raises(ValueError, match="w_edge"):
        eg.egnn_hblocks(lmax, C, we[:-1].contiguous(), we, eo, xo)
    with pytest.raises(ValueError, match="edge_irreps"):
        eg.egnn_hblocks(lmax, C, we, we, torch.zeros((10, K, C + 8)), xo)
    with pytest.raises(ValueError, match="GPU"):
        eg.egnn_hblocks(lmax, C, we, we, eo, xo)
    basis = eg.Basis((0, 1), (0b11, 0b01))
    with pytest.raises(ValueError, match="species"):
        eg.egnn_orbital_layout(basis, torch.tensor([0, 2], dtype=torch.int32), torch.tensor([0, 1]))
    with pytest.raises(ValueError, match="pos"):
        eg.egnn_build_graph(torch.zeros((4, 3), dtype=torch.float32), 4, [0, 0, 0], [9, 9, 9], 7, 5.0)
    with pytest.raises(ValueError, match="n_dst"):
        eg.egnn_build_graph(torch.zeros((4, 3), dtype=torch.float64), 5, [0, 0, 0], [9, 9, 9], 7, 5.0)


def test_noalloc_graph_rejects_on_the_host(lib):
    """The allocation-free graph build refuses a workspace need above its static
    array before touching the GPU (EGNN_E_WORKSPACE), and the usual argument errors."""
    from equivariant_gnn_electronic_amd import _lib
    box = (ct.c_double * 3)(9.0, 9.0, 9.0)
    lo = (ct.c_double * 3)(0.0, 0.0, 0.0)
    g = _fake_graph(64, 64, 5_000_000)
    st = lib.egnn_build_graph_noalloc(None, lo, box, 7, 5.0, ct.byref(g), None)
    assert st == _lib.EGNN_E_WORKSPACE
    assert b"allocation-free" in lib.egnn_last_error()
    g2 = _fake_graph(64, 32, 0)
    assert lib.egnn_build_graph_noalloc(None, lo, box, 7, 5.0, ct.byref(g2), None) == _lib.EGNN_E_ARG
    assert lib.egnn_build_graph_noalloc(None, lo, box, 7, -1.0, ct.byref(g), None) == _lib.EGNN_E_ARG


def test_edge_geom_rejects_misaligned_output(lib):
    from equivariant_gnn_electronic_amd import _lib
    d = _desc(4, 2, 64)
    g = _fake_graph(10, 10, 100)
    st = lib.egnn_edge_geom(ct.byref(d), ct.byref(g), ct.c_void_p(0x1004), None)
    assert st == _lib.EGNN_E_ARG and b"aligned" in lib.egnn_last_error()


def test_group_sources_host_checks(lib):
    """Source grouping: the workspace query grows with sources and edges, and the
    call refuses bad arguments and a short workspace before any launch."""
    from equivariant_gnn_electronic_amd import _lib
    a, b = ct.c_size_t(), ct.c_size_t()
    assert lib.egnn_group_sources_workspace(100, 1000, ct.byref(a)) == 0
    assert lib.egnn_group_sources_workspace(100, 2000, ct.byref(b)) == 0
    assert b.value >= a.value + 4 * 1000 - 256 and a.value >= 4 * (2 * 101 + 1000)
    assert lib.egnn_group_sources_workspace(-1, 10, ct.byref(a)) == _lib.EGNN_E_ARG
    assert lib.egnn_group_sources_workspace(10, -1, ct.byref(a)) == _lib.EGNN_E_ARG
    assert lib.egnn_group_sources_workspace(10, 2 ** 31, ct.byref(a)) == _lib.EGNN_E_ARG
    assert lib.egnn_group_sources(None, None, 0, None) == _lib.EGNN_E_ARG
    g = _fake_graph(10, 10, 100)
    assert lib.egnn_group_sources_workspace(10, 100, ct.byref(a)) == 0
    st = lib.egnn_group_sources(ct.byref(g), ct.c_void_p(0x1000), a.value - 1, None)
    assert st == _lib.EGNN_E_WORKSPACE and b"workspace" in lib.egnn_last_error()
    g.src_ptr = None
    assert lib.egnn_group_sources(ct.byref(g), ct.c_void_p(0x1000), a.value, None) == _lib.EGNN_E_ARG
    g = _fake_graph(10, 10, 100)
    g.src_perm = None
    assert lib.egnn_group_sources(ct.byref(g), ct.c_void_p(0x1000), a.value, None) == _lib.EGNN_E_ARG


def test_binding_group_rejects_bad_csr():
    import torch
    import equivariant_gnn_electronic_amd as eg
    rp = torch.tensor([0, 1, 2], dtype=torch.int32)
    with pytest.raises(ValueError):
        eg.Graph.from_csr(rp.to(torch.int64), torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        eg.Graph.from_csr(rp, torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError):
        eg.Graph.from_csr(rp, torch.zeros(2, dtype=torch.int32), shift=torch.zeros((3, 3), dtype=torch.int8))
