"""ctypes view of libegnn.so (the C ABI declared in include/egnn.h)."""
from __future__ import annotations

import ctypes as ct
import os

# EGNN_LIBRARY names another build of the same ABI (the host-only sanitizer
# build that the host-code tests load); the default is the in-tree library.
LIB_PATH = os.environ.get("EGNN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libegnn.so")

EGNN_OK, EGNN_E_ARG, EGNN_E_CAPACITY, EGNN_E_HIP, EGNN_E_UNSUPPORTED, EGNN_E_WORKSPACE = range(6)
EGNN_F32, EGNN_BF16 = 0, 1

# every symbol the header declares, with (restype, argtypes)
_vp, _i32, _i64, _u32, _f64, _sz = ct.c_void_p, ct.c_int32, ct.c_int64, ct.c_uint32, ct.c_double, ct.c_size_t


class EgnnGraph(ct.Structure):
    _fields_ = [("n_dst", ct.c_int32), ("n_src", ct.c_int32), ("capacity", ct.c_int64), ("n_edges", ct.c_int64),
                ("row_ptr", _vp), ("src", _vp), ("shift", _vp), ("vec", _vp), ("dist", _vp),
                ("src_ptr", _vp), ("src_perm", _vp)]


class EgnnLayerDesc(ct.Structure):
    _fields_ = [("lmax", ct.c_int32), ("mmax", ct.c_int32), ("C", ct.c_int32), ("n_rbf", ct.c_int32),
                ("r_cut", ct.c_double), ("storage", ct.c_int32)]


class EgnnHDesc(ct.Structure):
    _fields_ = [("lmax", ct.c_int32), ("C", ct.c_int32), ("n_shells", ct.c_int32),
                ("shell_l", ct.POINTER(ct.c_int32)), ("storage", ct.c_int32)]


class EgnnBasis(ct.Structure):
    _fields_ = [("n_shells", ct.c_int32), ("shell_l", ct.POINTER(ct.c_int32)), ("n_species", ct.c_int32),
                ("species_shells", ct.POINTER(ct.c_uint32))]


class EgnnOrbitals(ct.Structure):
    _fields_ = [("n_mols", ct.c_int32), ("n_atoms", ct.c_int32), ("mol_ptr", _vp), ("species", _vp),
                ("atom_orb", _vp), ("atom_mol", _vp), ("mol_norb", _vp), ("mat_off", _vp)]


class EgnnTimingEntry(ct.Structure):
    _fields_ = [("name", ct.c_char * 48), ("launches", ct.c_int64), ("total_ms", ct.c_double),
                ("flops", ct.c_double), ("bytes", ct.c_double)]


_D3 = ct.POINTER(ct.c_double)
_G = ct.POINTER(EgnnGraph)
_L = ct.POINTER(EgnnLayerDesc)
_H = ct.POINTER(EgnnHDesc)
_PSZ = ct.POINTER(ct.c_size_t)
_B = ct.POINTER(EgnnBasis)
_O = ct.POINTER(EgnnOrbitals)

SIGNATURES = {
    "egnn_status_string": (ct.c_char_p, [ct.c_int]),
    "egnn_last_error": (ct.c_char_p, []),
    "egnn_version": (ct.c_int, []),
    "egnn_build_graph_workspace": (ct.c_int, [_i32, _i32, _D3, _D3, _u32, _f64, _i64, _PSZ]),
    "egnn_build_graph": (ct.c_int, [_vp, _D3, _D3, _u32, _f64, _G, _vp, _sz, _vp]),
    "egnn_build_graph_noalloc": (ct.c_int, [_vp, _D3, _D3, _u32, _f64, _G, _vp]),
    "egnn_group_sources_workspace": (ct.c_int, [_i32, _i64, _PSZ]),
    "egnn_group_sources": (ct.c_int, [_G, _vp, _sz, _vp]),
    "egnn_layer_weight_count": (ct.c_size_t, [_L]),
    "egnn_geom_stride": (ct.c_int32, [_L]),
    "egnn_edge_geom": (ct.c_int, [_L, _G, _vp, _vp]),
    "egnn_layer_sizes": (ct.c_int, [_L, _G, _PSZ, _PSZ, _PSZ]),
    "egnn_layer_fwd": (ct.c_int, [_L, _G, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "egnn_layer_bwd": (ct.c_int, [_L, _G, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "egnn_edge_update_fwd": (ct.c_int, [_L, _G, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "egnn_edge_update_bwd": (ct.c_int, [_L, _G, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "egnn_hblocks_label_rows": (ct.c_int32, [_H]),
    "egnn_hblocks": (ct.c_int, [_H, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "egnn_assemble_bsr": (ct.c_int, [_G, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "egnn_label_width": (ct.c_int32, [_B]),
    "egnn_orbital_layout": (ct.c_int, [_B, _O, _vp, _vp]),
    "egnn_matrix_to_label": (ct.c_int, [_B, _O, _G, _vp, _i64, _vp, _vp, _vp, _vp]),
    "egnn_label_to_matrix": (ct.c_int, [_B, _O, _G, _vp, _vp, _vp, _i64, _vp, _vp]),
    "egnn_timing_enable": (ct.c_int, [ct.c_int]),
    "egnn_timing_collect": (ct.c_int, [ct.POINTER(EgnnTimingEntry), ct.c_int, ct.POINTER(ct.c_int64)]),
    "egnn_timing_reset": (None, []),
}

_lib = None


def load():
    """Load libegnn.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m equivariant_gnn_electronic_amd.build`")
        lib = ct.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class EgnnError(RuntimeError):
    def __init__(self, fn, status):
        lib = load()
        self.status = status
        super().__init__(f"{fn}: {lib.egnn_status_string(status).decode()} "
                         f"({lib.egnn_last_error().decode()})")


def check(fn, status):
    if status != EGNN_OK:
        raise EgnnError(fn, status)
    return status
