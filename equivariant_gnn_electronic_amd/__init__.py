"""MI355X-native SO(2) equivariant message-passing layer: Python binding of libegnn.so.

The functions here carry the names of the C ABI (include/egnn.h) and only
marshal arguments: torch supplies device memory and the current HIP stream,
and every step of the computation runs in the library's HIP kernels.  There
is no fallback path: if libegnn.so is missing, or the tensors are not on a
GPU, the calls raise.
"""
from __future__ import annotations

import ctypes as ct
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import EGNN_BF16, EGNN_F32, EgnnError

__all__ = ["Graph", "layer_desc", "egnn_build_graph", "egnn_build_graph_noalloc", "egnn_edge_geom", "egnn_geom_stride",
           "egnn_layer_weight_count", "egnn_layer_sizes", "egnn_layer_fwd", "egnn_layer_bwd",
           "egnn_hblocks", "egnn_hblocks_label_rows", "egnn_timing_enable", "egnn_timing_collect",
           "egnn_timing_reset", "GraphBuilder", "LayerBuffers", "EgnnError", "EGNN_F32", "EGNN_BF16",
           "Basis", "Orbitals", "egnn_label_width", "egnn_orbital_layout", "egnn_matrix_to_label",
           "egnn_label_to_matrix", "egnn_edge_update_fwd", "egnn_edge_update_bwd", "egnn_assemble_bsr"]

_STORAGE = {EGNN_F32: torch.float32, EGNN_BF16: torch.bfloat16}


def _stream():
    return ct.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ct.c_void_p(t.data_ptr())


def _d3(v):
    return (ct.c_double * 3)(*[float(a) for a in v])


def _expect(t, name, dtype, shape, min_rows=None):
    """Reject a tensor whose dtype or shape differs from what the kernels read.

    The C ABI sees plain pointers, so this is the only place a wrong buffer can be
    caught before a kernel reads or writes past it.  `shape` lists the expected
    sizes (None = any); `min_rows`, when given, replaces an exact first size by a
    lower bound.  Runs before the device check, so it needs no GPU.
    """
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != len(shape):
        raise ValueError(f"{name} must have {len(shape)} dimensions, got shape {tuple(t.shape)}")
    for i, (got, want) in enumerate(zip(t.shape, shape)):
        if i == 0 and min_rows is not None:
            if got < min_rows:
                raise ValueError(f"{name} needs at least {min_rows} rows, got {got}")
        elif want is not None and got != want:
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _expect_bytes(t, name, n):
    if n > 0 and (t is None or t.numel() * t.element_size() < n):
        have = 0 if t is None else t.numel() * t.element_size()
        raise ValueError(f"{name} holds {have} bytes, needs {n}")


@dataclass
class Graph:
    """Destination-sorted CSR (incoming-edge layout) held in torch tensors."""
    n_dst: int
    n_src: int
    n_edges: int
    row_ptr: torch.Tensor
    src: torch.Tensor
    shift: torch.Tensor
    vec: torch.Tensor
    dist: torch.Tensor
    src_ptr: torch.Tensor
    src_perm: torch.Tensor

    def c_struct(self):
        g = _lib.EgnnGraph()
        g.n_dst, g.n_src = self.n_dst, self.n_src
        g.capacity = self.src.numel()
        g.n_edges = self.n_edges
        for f in ("row_ptr", "src", "shift", "vec", "dist", "src_ptr", "src_perm"):
            t = self.__dict__[f]
            setattr(g, f, None if t is None else t.data_ptr())
        return g

    @classmethod
    def from_csr(cls, row_ptr, src, n_src=None, shift=None, group=False):
        """A graph given by its CSR (row_ptr, src, optional shift).  With
        group=True its source grouping (src_ptr, src_perm) is made by
        egnn_group_sources, so Matrix <-> Label takes the source-grouped order."""
        n_dst = row_ptr.numel() - 1
        _expect(row_ptr, "row_ptr", torch.int32, (n_dst + 1,))
        _expect(src, "src", torch.int32, (None,))
        if shift is not None:
            _expect(shift, "shift", torch.int8, (src.numel(), 3))
        g = cls(n_dst, n_dst if n_src is None else n_src, src.numel(), row_ptr, src, shift,
                None, None, None, None)
        if group:
            egnn_group_sources(g)
        return g


def egnn_group_sources(graph: Graph):
    """Write graph.src_ptr [n_src + 1] and graph.src_perm [n_edges]: the edge ids
    of each source in ascending order (sources outside [0, n_src) in no group)."""
    lib = _lib.load()
    _expect(graph.src, "src", torch.int32, (graph.n_edges,))
    dev = graph.src.device
    graph.src_ptr = torch.empty(graph.n_src + 1, dtype=torch.int32, device=dev)
    graph.src_perm = torch.empty(max(graph.n_edges, 1), dtype=torch.int32, device=dev)
    nbytes = ct.c_size_t(0)
    _lib.check("egnn_group_sources_workspace",
               lib.egnn_group_sources_workspace(graph.n_src, graph.n_edges, ct.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=dev)
    g = graph.c_struct()
    _lib.check("egnn_group_sources", lib.egnn_group_sources(ct.byref(g), _ptr(ws), nbytes.value, _stream()))
    return graph


def layer_desc(lmax, mmax, C, n_rbf, r_cut, storage=EGNN_F32):
    return _lib.EgnnLayerDesc(lmax, mmax, C, n_rbf, float(r_cut), storage)


def egnn_build_graph(pos, n_dst, lo, box, periodic_mask, r_cut, capacity=None):
    """Build the graph of positions pos [n_src][3] (float64, on the GPU).

    Runs the two-phase protocol of the C call: an edge count (capacity 0
    unless given), then the fill into arrays of exactly that size.
    """
    lib = _lib.load()
    _expect(pos, "pos", torch.float64, (None, 3))
    dev = pos.device
    n_src = pos.shape[0]
    if not 0 <= n_dst <= n_src:
        raise ValueError(f"n_dst ({n_dst}) must lie in [0, n_src = {n_src}]")
    row_ptr = torch.empty(n_dst + 1, dtype=torch.int32, device=dev)
    cap = 0 if capacity is None else int(capacity)

    def arrays(c):
        return dict(src=torch.empty(max(c, 1), dtype=torch.int32, device=dev),
                    shift=torch.empty((max(c, 1), 3), dtype=torch.int8, device=dev),
                    vec=torch.empty((max(c, 1), 3), dtype=torch.float32, device=dev),
                    dist=torch.empty(max(c, 1), dtype=torch.float32, device=dev),
                    src_ptr=torch.empty(n_src + 1, dtype=torch.int32, device=dev),
                    src_perm=torch.empty(max(c, 1), dtype=torch.int32, device=dev))

    lo3, box3 = _d3(lo), _d3(box)
    for _ in range(2):
        a = arrays(cap)
        g = _lib.EgnnGraph()
        g.n_dst, g.n_src, g.capacity = n_dst, n_src, cap
        g.row_ptr = row_ptr.data_ptr()
        g.src_ptr = a["src_ptr"].data_ptr()
        for f in ("src", "shift", "vec", "dist", "src_perm"):
            setattr(g, f, a[f].data_ptr() if cap > 0 else None)
        ws_bytes = ct.c_size_t()
        _lib.check("egnn_build_graph_workspace", lib.egnn_build_graph_workspace(
            n_dst, n_src, lo3, box3, periodic_mask, float(r_cut), cap, ct.byref(ws_bytes)))
        ws = torch.empty(max(ws_bytes.value, 1), dtype=torch.uint8, device=dev)
        st = lib.egnn_build_graph(_ptr(pos), lo3, box3, periodic_mask, float(r_cut), ct.byref(g),
                                  _ptr(ws), ws_bytes.value, _stream())
        if st == _lib.EGNN_E_CAPACITY:
            cap = int(g.n_edges)
            continue
        _lib.check("egnn_build_graph", st)
        E = int(g.n_edges)
        return Graph(n_dst, n_src, E, row_ptr, a["src"][:E], a["shift"][:E], a["vec"][:E], a["dist"][:E],
                     a["src_ptr"], a["src_perm"][:E])
    raise RuntimeError("egnn_build_graph: edge count changed between the two passes")


def egnn_build_graph_noalloc(pos, n_dst, lo, box, periodic_mask, r_cut, capacity=None):
    """egnn_build_graph through the allocation-free entry point (the library's
    static workspace instead of one from torch).  The output arrays are still
    the caller's: they are allocated here, as in egnn_build_graph."""
    lib = _lib.load()
    _expect(pos, "pos", torch.float64, (None, 3))
    dev = pos.device
    n_src = pos.shape[0]
    if not 0 <= n_dst <= n_src:
        raise ValueError(f"n_dst ({n_dst}) must lie in [0, n_src = {n_src}]")
    row_ptr = torch.empty(n_dst + 1, dtype=torch.int32, device=dev)
    src_ptr = torch.empty(n_src + 1, dtype=torch.int32, device=dev)
    cap = 0 if capacity is None else int(capacity)
    lo3, box3 = _d3(lo), _d3(box)
    for _ in range(2):
        a = {f: torch.empty(sh, dtype=dt, device=dev) for f, sh, dt in (
            ("src", (max(cap, 1),), torch.int32), ("shift", (max(cap, 1), 3), torch.int8),
            ("vec", (max(cap, 1), 3), torch.float32), ("dist", (max(cap, 1),), torch.float32),
            ("src_perm", (max(cap, 1),), torch.int32))}
        g = _lib.EgnnGraph()
        g.n_dst, g.n_src, g.capacity = n_dst, n_src, cap
        g.row_ptr, g.src_ptr = row_ptr.data_ptr(), src_ptr.data_ptr()
        for f in a:
            setattr(g, f, a[f].data_ptr() if cap > 0 else None)
        st = lib.egnn_build_graph_noalloc(_ptr(pos), lo3, box3, periodic_mask, float(r_cut), ct.byref(g), _stream())
        if st == _lib.EGNN_E_CAPACITY:
            cap = int(g.n_edges)
            continue
        _lib.check("egnn_build_graph_noalloc", st)
        E = int(g.n_edges)
        return Graph(n_dst, n_src, E, row_ptr, a["src"][:E], a["shift"][:E], a["vec"][:E], a["dist"][:E],
                     src_ptr, a["src_perm"][:E])
    raise RuntimeError("egnn_build_graph_noalloc: edge count changed between the two passes")


class GraphBuilder:
    """Repeated egnn_build_graph calls on one structure size with preallocated arrays.

    The arrays and workspace are sized for `capacity` edges once; each
    build() is a single C call (one edge count + fill).
    """

    def __init__(self, n_dst, n_src, lo, box, periodic_mask, r_cut, capacity, device):
        self.n_dst, self.n_src, self.mask, self.r_cut = n_dst, n_src, periodic_mask, float(r_cut)
        self.lo3, self.box3 = _d3(lo), _d3(box)
        c = max(int(capacity), 1)
        self.cap = int(capacity)
        self.row_ptr = torch.empty(n_dst + 1, dtype=torch.int32, device=device)
        self.src = torch.empty(c, dtype=torch.int32, device=device)
        self.shift = torch.empty((c, 3), dtype=torch.int8, device=device)
        self.vec = torch.empty((c, 3), dtype=torch.float32, device=device)
        self.dist = torch.empty(c, dtype=torch.float32, device=device)
        self.src_ptr = torch.empty(n_src + 1, dtype=torch.int32, device=device)
        self.src_perm = torch.empty(c, dtype=torch.int32, device=device)
        ws_bytes = ct.c_size_t()
        _lib.check("egnn_build_graph_workspace", _lib.load().egnn_build_graph_workspace(
            n_dst, n_src, self.lo3, self.box3, periodic_mask, self.r_cut, self.cap, ct.byref(ws_bytes)))
        self.ws = torch.empty(max(ws_bytes.value, 1), dtype=torch.uint8, device=device)
        self.g = _lib.EgnnGraph()
        g = self.g
        g.n_dst, g.n_src, g.capacity = n_dst, n_src, self.cap
        for f in ("row_ptr", "src", "shift", "vec", "dist", "src_ptr", "src_perm"):
            setattr(g, f, getattr(self, f).data_ptr())

    def build(self, pos):
        _expect(pos, "pos", torch.float64, (self.n_src, 3))
        _lib.check("egnn_build_graph", _lib.load().egnn_build_graph(
            _ptr(pos), self.lo3, self.box3, self.mask, self.r_cut, ct.byref(self.g), _ptr(self.ws),
            self.ws.numel(), _stream()))
        E = int(self.g.n_edges)
        return Graph(self.n_dst, self.n_src, E, self.row_ptr, self.src[:E], self.shift[:E], self.vec[:E],
                     self.dist[:E], self.src_ptr, self.src_perm[:E])


def egnn_timing_enable(on=True):
    _lib.check("egnn_timing_enable", _lib.load().egnn_timing_enable(1 if on else 0))


def egnn_timing_reset():
    _lib.load().egnn_timing_reset()


def egnn_timing_collect():
    """{kernel family: {launches, total_ms, flops, bytes}} accumulated so far (waits for the GPU)."""
    out = (_lib.EgnnTimingEntry * 64)()
    dropped = ct.c_int64()
    n = _lib.load().egnn_timing_collect(out, 64, ct.byref(dropped))
    res = {}
    for i in range(n):
        e = out[i]
        res[e.name.decode()] = dict(launches=int(e.launches), total_ms=float(e.total_ms), flops=float(e.flops),
                                    bytes=float(e.bytes))
    return res, int(dropped.value)


def egnn_geom_stride(desc):
    return int(_lib.load().egnn_geom_stride(ct.byref(desc)))


def egnn_layer_weight_count(desc):
    return int(_lib.load().egnn_layer_weight_count(ct.byref(desc)))


def egnn_edge_geom(desc, graph: Graph, out=None):
    """Per-edge Wigner rows, radial basis and destination row: [E][stride] float32."""
    lib = _lib.load()
    stride = egnn_geom_stride(desc)
    if stride <= 0:
        raise ValueError("invalid layer description")
    if out is None:
        out = torch.empty((max(graph.n_edges, 1), stride), dtype=torch.float32, device=graph.row_ptr.device)
    _expect(out, "out", torch.float32, (None, stride), min_rows=graph.n_edges)
    g = graph.c_struct()
    _lib.check("egnn_edge_geom", lib.egnn_edge_geom(ct.byref(desc), ct.byref(g), _ptr(out), _stream()))
    return out


def egnn_layer_sizes(desc, graph: Graph):
    lib = _lib.load()
    s, f, b = ct.c_size_t(), ct.c_size_t(), ct.c_size_t()
    g = graph.c_struct()
    _lib.check("egnn_layer_sizes", lib.egnn_layer_sizes(ct.byref(desc), ct.byref(g), ct.byref(s), ct.byref(f),
                                                         ct.byref(b)))
    return s.value, f.value, b.value


class LayerBuffers:
    """Saved activations and workspaces for one layer on one graph (allocated by torch)."""

    def __init__(self, desc, graph: Graph, train=True):
        saved, wsf, wsb = egnn_layer_sizes(desc, graph)
        dev = graph.row_ptr.device
        self.saved = torch.empty(max(saved, 1), dtype=torch.uint8, device=dev) if train else None
        self.ws = torch.empty(max(wsf, wsb if train else 0, 1), dtype=torch.uint8, device=dev)


def _check_layer_args(desc, graph: Graph, geom, weights, x):
    """dtype and shape of the inputs every layer call reads; returns (K, storage dtype)."""
    if desc.storage not in _STORAGE:
        raise ValueError(f"unknown storage type {desc.storage}")
    K = (desc.lmax + 1) ** 2
    dt = _STORAGE[desc.storage]
    n_w = egnn_layer_weight_count(desc)
    if n_w == 0:
        raise ValueError("invalid layer description")
    _expect(weights, "weights", torch.float32, (n_w,))
    _expect(geom, "geom", torch.float32, (None, egnn_geom_stride(desc)), min_rows=graph.n_edges)
    _expect(x, "x", dt, (None, K, desc.C), min_rows=graph.n_src)
    return K, dt


def _check_buffers(desc, graph: Graph, buffers, train, bwd):
    saved, wsf, wsb = egnn_layer_sizes(desc, graph)
    if train or bwd:
        if buffers.saved is None:
            raise ValueError("the backward needs buffers made with train=True")
        _expect_bytes(buffers.saved, "buffers.saved", saved)
    _expect_bytes(buffers.ws, "buffers.ws", wsb if bwd else wsf)


def egnn_layer_fwd(desc, graph: Graph, geom, weights, x, x_out=None, edge_out=False, buffers=None):
    """x_out [n_dst][K][C] (and edge_out [E][K][C] if requested) of one layer."""
    lib = _lib.load()
    K, dt = _check_layer_args(desc, graph, geom, weights, x)
    if buffers is None:
        buffers = LayerBuffers(desc, graph, train=False)
    _check_buffers(desc, graph, buffers, train=buffers.saved is not None, bwd=False)
    if x_out is None:
        x_out = torch.empty((graph.n_dst, K, desc.C), dtype=dt, device=x.device)
    _expect(x_out, "x_out", dt, (graph.n_dst, K, desc.C))
    eo = torch.empty((max(graph.n_edges, 1), K, desc.C), dtype=dt, device=x.device) if edge_out else None
    g = graph.c_struct()
    _lib.check("egnn_layer_fwd", lib.egnn_layer_fwd(
        ct.byref(desc), ct.byref(g), _ptr(geom), _ptr(weights), _ptr(x), _ptr(x_out), _ptr(eo),
        _ptr(buffers.saved), _ptr(buffers.ws), buffers.ws.numel(), _stream()))
    return (x_out, eo[:graph.n_edges] if eo is not None else None), buffers


def egnn_layer_bwd(desc, graph: Graph, geom, weights, x, buffers, grad_out, grad_x=None, grad_w=None):
    """(dL/dx [n_src][K][C], dL/dweights) for the loss <grad_out, x_out>."""
    lib = _lib.load()
    K, _ = _check_layer_args(desc, graph, geom, weights, x)
    _check_buffers(desc, graph, buffers, train=True, bwd=True)
    _expect(grad_out, "grad_out", torch.float32, (graph.n_dst, K, desc.C))
    if grad_x is None:
        grad_x = torch.empty((graph.n_src, K, desc.C), dtype=torch.float32, device=x.device)
    if grad_w is None:
        grad_w = torch.empty(egnn_layer_weight_count(desc), dtype=torch.float32, device=x.device)
    _expect(grad_x, "grad_x", torch.float32, (graph.n_src, K, desc.C))
    _expect(grad_w, "grad_w", torch.float32, (egnn_layer_weight_count(desc),))
    g = graph.c_struct()
    _lib.check("egnn_layer_bwd", lib.egnn_layer_bwd(
        ct.byref(desc), ct.byref(g), _ptr(geom), _ptr(weights), _ptr(x), _ptr(buffers.saved), _ptr(grad_out),
        _ptr(grad_x), _ptr(grad_w), _ptr(buffers.ws), buffers.ws.numel(), _stream()))
    return grad_x, grad_w


def egnn_edge_update_fwd(desc, graph: Graph, geom, weights, x, e_in, e_out=None, buffers=None):
    """Edge-update block: e_out = e_in + the per-edge message (in place when e_out is e_in).
    Returns (e_out, buffers); buffers keep the activations the backward reads."""
    lib = _lib.load()
    K, dt = _check_layer_args(desc, graph, geom, weights, x)
    _expect(e_in, "e_in", dt, (graph.n_edges, K, desc.C))
    if buffers is None:
        buffers = LayerBuffers(desc, graph, train=True)
    _check_buffers(desc, graph, buffers, train=buffers.saved is not None, bwd=False)
    if e_out is None:
        e_out = torch.empty_like(e_in)
    _expect(e_out, "e_out", dt, (graph.n_edges, K, desc.C))
    g = graph.c_struct()
    _lib.check("egnn_edge_update_fwd", lib.egnn_edge_update_fwd(
        ct.byref(desc), ct.byref(g), _ptr(geom), _ptr(weights), _ptr(x), _ptr(e_in), _ptr(e_out),
        _ptr(buffers.saved) if buffers.saved is not None else None, _ptr(buffers.ws), buffers.ws.numel(), _stream()))
    return e_out, buffers


def egnn_edge_update_bwd(desc, graph: Graph, geom, weights, x, buffers, grad_e_out, grad_x=None, grad_w=None):
    """Gradients of <grad_e_out, e_out> w.r.t. x and the packed weights (that w.r.t. e_in is grad_e_out)."""
    lib = _lib.load()
    K, _ = _check_layer_args(desc, graph, geom, weights, x)
    _check_buffers(desc, graph, buffers, train=True, bwd=True)
    _expect(grad_e_out, "grad_e_out", torch.float32, (graph.n_edges, K, desc.C))
    if grad_x is None:
        grad_x = torch.empty((graph.n_src, K, desc.C), dtype=torch.float32, device=x.device)
    if grad_w is None:
        grad_w = torch.empty(egnn_layer_weight_count(desc), dtype=torch.float32, device=x.device)
    _expect(grad_x, "grad_x", torch.float32, (graph.n_src, K, desc.C))
    _expect(grad_w, "grad_w", torch.float32, (egnn_layer_weight_count(desc),))
    g = graph.c_struct()
    _lib.check("egnn_edge_update_bwd", lib.egnn_edge_update_bwd(
        ct.byref(desc), ct.byref(g), _ptr(geom), _ptr(weights), _ptr(x), _ptr(buffers.saved), _ptr(grad_e_out),
        _ptr(grad_x), _ptr(grad_w), _ptr(buffers.ws), buffers.ws.numel(), _stream()))
    return grad_x, grad_w


def _hdesc(lmax, C, shell_l, storage):
    arr = (ct.c_int32 * len(shell_l))(*shell_l)
    h = _lib.EgnnHDesc(lmax, C, len(shell_l), arr, storage)
    h._keep = arr
    return h


def egnn_hblocks_label_rows(lmax, C, shell_l=(0, 0, 1, 1, 2), storage=EGNN_F32):
    return int(_lib.load().egnn_hblocks_label_rows(ct.byref(_hdesc(lmax, C, shell_l, storage))))


def egnn_hblocks(lmax, C, w_edge, w_node, edge_irreps, node_irreps, shell_l=(0, 0, 1, 1, 2), storage=EGNN_F32):
    """Orbital blocks [E][n_orb][n_orb] and [N][n_orb][n_orb] from irreps."""
    lib = _lib.load()
    h = _hdesc(lmax, C, shell_l, storage)
    n_orb = sum(2 * l + 1 for l in shell_l)
    if storage not in _STORAGE:
        raise ValueError(f"unknown storage type {storage}")
    rows = egnn_hblocks_label_rows(lmax, C, shell_l, storage)
    if rows <= 0:
        raise ValueError("invalid decode description")
    K = (lmax + 1) ** 2
    if edge_irreps is None and node_irreps is None:
        raise ValueError("edge_irreps or node_irreps is required")
    E = 0 if edge_irreps is None else edge_irreps.shape[0]
    N = 0 if node_irreps is None else node_irreps.shape[0]
    if E:
        _expect(edge_irreps, "edge_irreps", _STORAGE[storage], (E, K, C))
        _expect(w_edge.reshape(-1) if isinstance(w_edge, torch.Tensor) else w_edge, "w_edge", torch.float32,
                (rows * C,))
    if N:
        _expect(node_irreps, "node_irreps", _STORAGE[storage], (N, K, C))
        _expect(w_node.reshape(-1) if isinstance(w_node, torch.Tensor) else w_node, "w_node", torch.float32,
                (rows * C,))
    dev = (edge_irreps if edge_irreps is not None else node_irreps).device
    he = torch.empty((max(E, 1), n_orb, n_orb), dtype=torch.float32, device=dev)
    hn = torch.empty((max(N, 1), n_orb, n_orb), dtype=torch.float32, device=dev)
    _lib.check("egnn_hblocks", lib.egnn_hblocks(
        ct.byref(h), E, N, _ptr(w_edge) if E else None, _ptr(w_node) if N else None,
        _ptr(edge_irreps) if E else None, _ptr(node_irreps) if N else None, _ptr(he) if E else None,
        _ptr(hn) if N else None, _stream()))
    return he[:E], hn[:N]


def egnn_assemble_bsr(graph: Graph, h_edge, h_onsite=None):
    """One block-sparse-row matrix over all image shifts from the decode's blocks:
    (row_ptr [n_src+1], col [nnzb], shift [nnzb][3] int8, val [nnzb][n_orb][n_orb])."""
    lib = _lib.load()
    _expect(h_edge, "h_edge", torch.float32, (graph.n_edges, None, None))
    n_orb = h_edge.shape[1]
    if h_edge.shape[2] != n_orb:
        raise ValueError("h_edge blocks must be square")
    if h_onsite is not None:
        _expect(h_onsite, "h_onsite", torch.float32, (graph.n_dst, n_orb, n_orb))
    dev = graph.row_ptr.device
    nnzb = graph.n_edges + (graph.n_dst if h_onsite is not None else 0)
    rp = torch.empty(graph.n_src + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(nnzb, 1), dtype=torch.int32, device=dev)
    sh = torch.empty((max(nnzb, 1), 3), dtype=torch.int8, device=dev)
    val = torch.empty((max(nnzb, 1), n_orb, n_orb), dtype=torch.float32, device=dev)
    g = graph.c_struct()
    _lib.check("egnn_assemble_bsr", lib.egnn_assemble_bsr(
        ct.byref(g), n_orb, _ptr(h_edge) if graph.n_edges else None,
        _ptr(h_onsite) if h_onsite is not None else None, _ptr(rp), _ptr(col), _ptr(sh), _ptr(val), _stream()))
    return rp, col[:nnzb], sh[:nnzb], val[:nnzb]


class Basis:
    """Full shell list and per-element shell masks (orbital templates)."""

    def __init__(self, shell_l, species_shells):
        self.shell_l = tuple(int(l) for l in shell_l)
        self.species_shells = tuple(int(m) for m in species_shells)
        self._l = (ct.c_int32 * len(self.shell_l))(*self.shell_l)
        self._m = (ct.c_uint32 * len(self.species_shells))(*self.species_shells)
        self.c = _lib.EgnnBasis(len(self.shell_l), self._l, len(self.species_shells), self._m)


@dataclass
class Orbitals:
    """Atom and structure layout of a batch of matrices (egnn_orbital_layout's outputs)."""
    mol_ptr: torch.Tensor
    species: torch.Tensor
    atom_orb: torch.Tensor
    atom_mol: torch.Tensor
    mol_norb: torch.Tensor
    mat_off: torch.Tensor

    @property
    def n_atoms(self):
        return self.species.numel()

    @property
    def n_mols(self):
        return self.mol_ptr.numel() - 1

    def c_struct(self):
        o = _lib.EgnnOrbitals()
        o.n_mols, o.n_atoms = self.n_mols, self.n_atoms
        for f in ("mol_ptr", "species", "atom_orb", "atom_mol", "mol_norb", "mat_off"):
            setattr(o, f, self.__dict__[f].data_ptr())
        return o


def egnn_label_width(basis: Basis):
    return int(_lib.load().egnn_label_width(ct.byref(basis.c)))


def egnn_orbital_layout(basis: Basis, mol_ptr, species):
    """Orbitals of a batch (mol_ptr [n_mols+1], species [n_atoms], int32 on the GPU) and
    the count of invalid structures and element indices (int64 [1] on the GPU)."""
    lib = _lib.load()
    _expect(mol_ptr, "mol_ptr", torch.int32, (None,), min_rows=1)
    _expect(species, "species", torch.int32, (None,))
    dev = species.device
    n_mols, n_atoms = mol_ptr.numel() - 1, species.numel()
    o = Orbitals(mol_ptr, species,
                 torch.empty(max(n_atoms, 1), dtype=torch.int32, device=dev)[:n_atoms],
                 torch.empty(max(n_atoms, 1), dtype=torch.int32, device=dev)[:n_atoms],
                 torch.empty(max(n_mols, 1), dtype=torch.int32, device=dev)[:n_mols],
                 torch.empty(n_mols + 1, dtype=torch.int64, device=dev))
    bad = torch.empty(1, dtype=torch.int64, device=dev)
    for t in (mol_ptr, species):
        _ptr(t)                      # on the GPU and contiguous
    c = o.c_struct()
    _lib.check("egnn_orbital_layout", lib.egnn_orbital_layout(ct.byref(basis.c), ct.byref(c), _ptr(bad), _stream()))
    return o, bad


def egnn_matrix_to_label(basis: Basis, orbitals: Orbitals, graph, H, edges=True, nodes=True):
    """Labels (h_edge [E][n_lab], h_node [n_atoms][n_lab]) of the batch's matrices H
    (fp32, flat, mat_off[-1] entries) and the count of skipped blocks."""
    lib = _lib.load()
    n_lab = egnn_label_width(basis)
    if n_lab <= 0:
        raise ValueError("invalid basis")
    _expect(H, "H", torch.float32, (None,))
    dev = H.device
    E = graph.n_edges if (graph is not None and edges) else 0
    he = torch.empty((max(E, 1), n_lab), dtype=torch.float32, device=dev)
    hn = torch.empty((max(orbitals.n_atoms, 1), n_lab), dtype=torch.float32, device=dev)
    skipped = torch.empty(1, dtype=torch.int64, device=dev)
    g = graph.c_struct() if (graph is not None and edges) else None
    o = orbitals.c_struct()
    _lib.check("egnn_matrix_to_label", lib.egnn_matrix_to_label(
        ct.byref(basis.c), ct.byref(o), ct.byref(g) if g is not None else None, _ptr(H), H.numel(),
        _ptr(he) if g is not None else None, _ptr(hn) if nodes else None, _ptr(skipped), _stream()))
    return he[:E], (hn[:orbitals.n_atoms] if nodes else None), skipped


def egnn_label_to_matrix(basis: Basis, orbitals: Orbitals, graph, h_edge, h_node, H=None, h_elems=None):
    """Writes the blocks of h_edge / h_node (either may be None) into H (zeros of
    h_elems = mat_off[-1] entries when not given); returns (H, skipped count)."""
    lib = _lib.load()
    n_lab = egnn_label_width(basis)
    if n_lab <= 0:
        raise ValueError("invalid basis")
    if h_edge is not None and graph is not None:
        _expect(h_edge, "h_edge", torch.float32, (graph.n_edges, n_lab))
    if h_node is not None:
        _expect(h_node, "h_node", torch.float32, (orbitals.n_atoms, n_lab))
    dev = orbitals.species.device
    if H is None:
        n = int(orbitals.mat_off[-1].item()) if h_elems is None else int(h_elems)
        H = torch.zeros(max(n, 1), dtype=torch.float32, device=dev)[:n]
    _expect(H, "H", torch.float32, (None,))
    skipped = torch.empty(1, dtype=torch.int64, device=dev)
    g = graph.c_struct() if (graph is not None and h_edge is not None) else None
    o = orbitals.c_struct()
    _lib.check("egnn_label_to_matrix", lib.egnn_label_to_matrix(
        ct.byref(basis.c), ct.byref(o), ct.byref(g) if g is not None else None,
        _ptr(h_edge) if g is not None else None, _ptr(h_node) if h_node is not None else None, _ptr(H),
        H.numel(), _ptr(skipped), _stream()))
    return H, skipped
