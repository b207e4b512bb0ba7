"""Seeded synthetic inputs for the SO(2) message-passing layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP path read
what it produces, so the two sides see bit-identical inputs.

The workloads stand in for the DFT structures of the pages (amorphous HfO2
and GeSbTe cells, MALOQ Table II; the 8,064-atom GST cell of the
"Distributed Equivariant GNNs" review, abstract and GST application), whose
data is not available: positions come from random sequential addition (RSA)
with a 1.8 A minimum spacing, node irreps are N(0,1) and weights are
N(0, 1/fan_in).

Streams per config seed s (``numpy.random.default_rng``): ``s`` draws the
positions (RSA proposals, owned atoms then ghosts) and then the species;
``(s, 1)`` the node irreps x; ``(s, 2)`` the layer weights in packed order,
layer by layer; ``(s, 3)`` the decode weights; ``(s, 4)`` the cotangent G.
"""
from __future__ import annotations

import hashlib
import json
import os
from dataclasses import dataclass, field, asdict

import numpy as np

__all__ = ["Config", "CONFIGS", "Structure", "make_structure", "make_layer_inputs",
           "make_decode_weights", "make_cotangent", "layer_weight_sizes",
           "round_storage", "bf16_round", "SVP_SHELLS", "SVP_ELEMENTS", "SVP_MASKS",
           "SVP_FRACTIONS", "G_SHELLS", "G_MASKS", "G_FRACTIONS", "WATER_SHELLS", "WATER_MASKS", "MoleculeBatch", "make_molecule_batch",
           "make_matrix_values", "make_label_values", "make_edge_embeddings", "make_edge_cotangent"]


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    counts: tuple            # atoms per species (owned atoms)
    box: tuple               # periodic cell, or owned slab extent when open
    periodic: bool
    r_cut: float
    lmax: int
    mmax: int
    C: int
    n_rbf: int = 8
    storage: str = "f32"     # "f32" or "bf16"
    layers: int = 1
    min_sep: float = 1.8
    halo: float = 0.0        # ghost shell thickness around an open slab
    geometry_seed: int | None = None   # reuse another config's positions/x/weights
    note: str = ""

    @property
    def n_owned(self):
        return int(sum(self.counts))

    @property
    def K(self):
        return (self.lmax + 1) ** 2


CONFIGS = {
    "tiny": Config("tiny", 1, (32, 32), (9.0, 9.0, 9.0), True, 5.0, 2, 2, 8,
                   note="64 atoms, 2 species Bernoulli(1/2), 9 A periodic cube, r_c 5 A"),
    "tiny_l4": Config("tiny_l4", 1, (32, 32), (9.0, 9.0, 9.0), True, 5.0, 4, 2, 8,
                      note="tiny geometry at lmax 4 / mmax 2 / C 8 (m-truncation, decode)"),
    "tiny_l6": Config("tiny_l6", 1, (32, 32), (9.0, 9.0, 9.0), True, 5.0, 6, 2, 8,
                      note="tiny geometry at lmax 6 / mmax 2 / C 8 (f-orbital degrees)"),
    "tiny_stack": Config("tiny_stack", 1, (32, 32), (9.0, 9.0, 9.0), True, 5.0, 4, 2, 16, storage="bf16",
                         layers=3, note="tiny geometry, 3 stacked layers, bf16 storage"),
    "hfo2": Config("hfo2", 2, (1000, 2000), (32.8, 32.8, 32.8), True, 8.0, 4, 2, 64,
                   note="HfO2-like: 1,000 Hf + 2,000 O in a 32.8 A periodic cube, r_c 8 A"),
    "gst": Config("gst", 3, (1792, 1792, 4480), (62.5, 62.5, 62.5), True, 10.0, 4, 2, 128,
                  storage="bf16", layers=3,
                  note="GeSbTe-like: 8,064 atoms in a 62.5 A periodic cube, r_c 10 A, 3 layers"),
    "halo": Config("halo", 4, (10000, 10000, 10000), (100.0, 100.0, 60.0), False, 8.0, 4, 2, 64,
                   halo=8.0,
                   note="one GPU's share: 30,000 owned atoms in a 100x100x60 A slab, "
                        "ghost sources in the 8 A shell, open boundary"),
    "hfo2_l6": Config("hfo2_l6", 6, (1000, 2000), (32.8, 32.8, 32.8), True, 8.0, 6, 2, 64, geometry_seed=2,
                      note="HfO2-like geometry at lmax 6 (f-orbital degrees)"),
    "hfo2_l8": Config("hfo2_l8", 7, (1000, 2000), (32.8, 32.8, 32.8), True, 8.0, 8, 2, 64, geometry_seed=2,
                      note="HfO2-like geometry at lmax 8 (g-orbital degrees)"),
    "train": Config("train", 5, (1000, 2000), (32.8, 32.8, 32.8), True, 8.0, 4, 2, 64,
                    geometry_seed=2,
                    note="HfO2-like training step: fwd + bwd + Hamiltonian blocks"),
}

# Species are drawn as a random assignment of the fixed counts, except for the
# tiny cell whose two species are Bernoulli(1/2).
_BERNOULLI = {"tiny", "tiny_l4", "tiny_l6", "tiny_stack"}


def bf16_round(a):
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def round_storage(a, storage):
    """Values as the storage type holds them, returned as float32."""
    a = np.asarray(a, dtype=np.float64).astype(np.float32)
    return bf16_round(a) if storage == "bf16" else a


@dataclass
class Structure:
    pos: np.ndarray          # [n_src, 3] float64; owned atoms first, ghosts after
    n_dst: int
    box: np.ndarray          # [3] float64 (periodic cell; for open systems the padded extent)
    periodic_mask: int       # bit a set = axis a periodic
    species: np.ndarray      # [n_src] int32
    r_cut: float

    @property
    def n_src(self):
        return self.pos.shape[0]


def _rsa(rng, n, lo, hi, min_sep, accepted, box, periodic, reject=None, batch=4096):
    """Random sequential addition of n points uniform in [lo, hi).

    A proposal is kept when its distance to every point already accepted is
    at least min_sep (minimum image on periodic axes).  ``reject(p)`` may veto
    proposals (used for the ghost shell around a slab).  Returns the grown
    list of accepted points.
    """
    lo = np.asarray(lo, float)
    hi = np.asarray(hi, float)
    cell = min_sep
    if periodic:
        ncell = np.maximum(1, np.floor(np.asarray(box) / cell).astype(int))
        origin = np.zeros(3)
        csize = np.asarray(box) / ncell
    else:
        origin = lo - cell
        span = (hi - lo) + 2 * cell
        ncell = np.maximum(1, np.ceil(span / cell).astype(int))
        csize = np.full(3, cell)
    grid = {}

    def key(p):
        c = np.floor((p - origin) / csize).astype(int)
        if periodic:
            c %= ncell
        return tuple(int(v) for v in c)

    pts = list(accepted)
    for i, p in enumerate(pts):
        grid.setdefault(key(p), []).append(i)
    ms2 = min_sep * min_sep
    need = n
    while need > 0:
        props = lo + rng.random((batch, 3)) * (hi - lo)
        for p in props:
            if need == 0:
                break
            if reject is not None and reject(p):
                continue
            c = key(p)
            ok = True
            for dx in (-1, 0, 1):
                for dy in (-1, 0, 1):
                    for dz in (-1, 0, 1):
                        cc = [c[0] + dx, c[1] + dy, c[2] + dz]
                        if periodic:
                            cc = [cc[a] % ncell[a] for a in range(3)]
                        lst = grid.get(tuple(cc))
                        if not lst:
                            continue
                        q = np.asarray([pts[j] for j in lst])
                        d = p - q
                        if periodic:
                            d -= np.round(d / box) * box
                        if np.min(np.einsum("ij,ij->i", d, d)) < ms2:
                            ok = False
                            break
                    if not ok:
                        break
                if not ok:
                    break
            if ok:
                grid.setdefault(c, []).append(len(pts))
                pts.append(p.copy())
                need -= 1
    return pts


_CACHE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), ".synth_cache")


def _cache_path(tag):
    h = hashlib.sha1(tag.encode()).hexdigest()[:16]
    return os.path.join(_CACHE_DIR, f"{h}.npz")


def _draw_structure(cfg: Config, rng) -> Structure:
    box = np.asarray(cfg.box, dtype=np.float64)
    n = cfg.n_owned
    if cfg.periodic:
        pts = _rsa(rng, n, np.zeros(3), box, cfg.min_sep, [], box, True)
        pos = np.asarray(pts, dtype=np.float64)
        n_src = n
        mask = 7
        extent = box
    else:
        pts = _rsa(rng, n, np.zeros(3), box, cfg.min_sep, [], box, False)
        h = cfg.halo
        lo, hi = -h * np.ones(3), box + h
        vol_shell = np.prod(hi - lo) - np.prod(box)
        density = n / np.prod(box)
        n_ghost = int(round(density * vol_shell))

        def inside_slab(p):
            return bool(np.all(p >= 0.0) and np.all(p < box))

        pts = _rsa(rng, n_ghost, lo, hi, cfg.min_sep, pts, box, False, reject=inside_slab)
        pos = np.asarray(pts, dtype=np.float64)
        n_src = pos.shape[0]
        mask = 0
        extent = hi - lo
    # species
    if cfg.name in _BERNOULLI:
        sp_owned = (rng.random(n) < 0.5).astype(np.int32)
    else:
        sp_owned = np.repeat(np.arange(len(cfg.counts), dtype=np.int32), cfg.counts)
        rng.shuffle(sp_owned)
    if n_src > n:
        sp_ghost = rng.integers(0, len(cfg.counts), size=n_src - n).astype(np.int32)
        species = np.concatenate([sp_owned, sp_ghost])
    else:
        species = sp_owned
    return Structure(pos=pos, n_dst=n, box=np.asarray(extent, np.float64) if not cfg.periodic else box,
                     periodic_mask=mask, species=species, r_cut=float(cfg.r_cut))


def layer_weight_sizes(lmax, mmax, C, n_rbf):
    """Sizes (out, in) of the packed weight blocks of one layer, in packed order.

    Order: W0, then (W_m1, W_m2) for m = 1..mmax, then W_rad [n_rbf][n_pairs][2C]
    and w_att [C].  n_pairs = number of (m, l) with 0 <= m <= mmax, m <= l <= lmax.
    """
    blocks = [("W0", ((lmax + 1) * C, (lmax + 1) * 2 * C))]
    for m in range(1, mmax + 1):
        nl = lmax - m + 1
        blocks.append((f"W{m}_1", (nl * C, nl * 2 * C)))
        blocks.append((f"W{m}_2", (nl * C, nl * 2 * C)))
    n_pairs = sum(lmax - m + 1 for m in range(mmax + 1))
    blocks.append(("W_rad", (n_rbf, n_pairs * 2 * C)))
    blocks.append(("w_att", (1, C)))
    return blocks


def _fan_in(name, shape):
    if name.startswith("W") and name[1:2].isdigit() and name != "W0":
        return 2 * shape[1]          # W_m1 and W_m2 both feed each output
    if name == "W_rad":
        return shape[0]
    return shape[1]


def _tag(cfg: Config, what):
    return json.dumps({"cfg": asdict(cfg), "what": what, "v": 3}, sort_keys=True)


def make_structure(cfg: Config | str, use_cache=True) -> Structure:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.geometry_seed if cfg.geometry_seed is not None else cfg.seed
    gcfg = cfg
    if cfg.geometry_seed is not None:
        gcfg = next(c for c in CONFIGS.values() if c.seed == seed and c.geometry_seed is None)
    tag = _tag(gcfg, "structure")
    path = _cache_path(tag)
    if use_cache and os.path.exists(path):
        z = np.load(path)
        return Structure(pos=z["pos"], n_dst=int(z["n_dst"]), box=z["box"],
                         periodic_mask=int(z["mask"]), species=z["species"], r_cut=float(z["r_cut"]))
    rng = np.random.default_rng(seed)
    s = _draw_structure(gcfg, rng)
    if use_cache:
        os.makedirs(_CACHE_DIR, exist_ok=True)
        np.savez(path, pos=s.pos, n_dst=s.n_dst, box=s.box, mask=s.periodic_mask,
                 species=s.species, r_cut=s.r_cut)
    return s


def _stream_cfg(cfg: Config):
    """The config whose seed draws positions, x and layer weights."""
    if cfg.geometry_seed is None:
        return cfg
    return next(c for c in CONFIGS.values() if c.seed == cfg.geometry_seed and c.geometry_seed is None)


def make_layer_inputs(cfg: Config | str, n_src=None, use_cache=True):
    """Node irreps x [n_src][K][C] and the packed weights of each layer.

    Returns (x, [w_layer0, w_layer1, ...]) as float32 arrays already rounded
    to the storage type (bf16-representable when storage is bf16).
    For a config that reuses another's geometry, x and the weights are the
    other config's, drawn with its seed, but shaped by this config's
    (lmax, mmax, C) which must match.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    tag = _tag(cfg, "layer_inputs")
    path = _cache_path(tag)
    if use_cache and os.path.exists(path):
        z = np.load(path)
        return z["x"], [z[f"w{i}"] for i in range(cfg.layers)]
    gcfg = _stream_cfg(cfg)
    if n_src is None:
        n_src = make_structure(cfg, use_cache=use_cache).n_src
    rng = np.random.default_rng((gcfg.seed, 1))
    x = rng.standard_normal((n_src, cfg.K, cfg.C))
    x = round_storage(x, cfg.storage)
    rng = np.random.default_rng((gcfg.seed, 2))
    ws = []
    for _ in range(cfg.layers):
        parts = []
        for name, shape in layer_weight_sizes(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf):
            fan = _fan_in(name, shape)
            parts.append(rng.standard_normal(shape).ravel() / np.sqrt(fan))
        ws.append(round_storage(np.concatenate(parts), cfg.storage))
    if use_cache:
        os.makedirs(_CACHE_DIR, exist_ok=True)
        np.savez(path, x=x, **{f"w{i}": w for i, w in enumerate(ws)})
    return x, ws


def make_decode_weights(cfg: Config | str, n_label=(9, 17, 13, 5, 1)):
    """Decode weights W_dec,L [n_L][C] for edges and for nodes (seed of cfg).

    Stream (seed, 3): edge weights for L = 0..4, then node weights, N(0, 1/C).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng((cfg.seed, 3))
    we = [round_storage(rng.standard_normal((n, cfg.C)) / np.sqrt(cfg.C), "f32") for n in n_label]
    wn = [round_storage(rng.standard_normal((n, cfg.C)) / np.sqrt(cfg.C), "f32") for n in n_label]
    return we, wn


def make_cotangent(cfg: Config | str, n_dst):
    """Seeded cotangent G = dL/dx' [n_dst][K][C] (the loss is <G, x'>)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng((cfg.seed, 4))
    return round_storage(rng.standard_normal((n_dst, cfg.K, cfg.C)), "f32")


# --------------------------------------------------------------------------
# Molecule batches for Matrix <-> Label (MALOQ Sec. III-B2, Table II)
#
# Stand-in for a batch of the nabla^2 DFT small-molecule dataset: drug-like
# molecules of up to 50 atoms over H, C, N, O, F, S, Cl, fully connected
# graphs, described in a def2-SVP-like basis whose shell structure per
# element is H [2s1p], C-F [3s2p1d], S, Cl [4s3p1d] (labels up to L = 4).
# The full shell list is the union, 4s3p1d; an element's shells are a bit
# mask over it.  Matrix values are N(0, 1) (no DFT matrices are available).
# --------------------------------------------------------------------------

SVP_SHELLS = (0, 0, 0, 0, 1, 1, 1, 2)
SVP_ELEMENTS = ("H", "C", "N", "O", "F", "S", "Cl")
SVP_MASKS = (0b00010011,                 # H: s s . . p . . .
             0b10110111, 0b10110111,     # C, N: s s s . p p . d
             0b10110111, 0b10110111,     # O, F
             0b11111111, 0b11111111)     # S, Cl: s s s s p p p d
SVP_FRACTIONS = (0.45, 0.33, 0.08, 0.08, 0.02, 0.02, 0.02)

# the pages' toy example (Fig. 2(b)): water in a minimal basis, O [s p], H [s]
# A basis with g shells (labels up to L = 8, the metal-organic case of MALOQ
# Table II): full list s p d f g; light elements s p, second-row s p d, a
# metal all five shells.
G_SHELLS = (0, 1, 2, 3, 4)
G_MASKS = (0b00011, 0b00111, 0b11111)
G_FRACTIONS = (0.5, 0.35, 0.15)

WATER_SHELLS = (0, 1)
WATER_MASKS = (0b11, 0b01)               # O, H


@dataclass
class MoleculeBatch:
    mol_ptr: np.ndarray      # [n_mols + 1] int32, atoms of molecule b are mol_ptr[b]:mol_ptr[b+1]
    species: np.ndarray      # [n_atoms] int32, index into the basis' element list
    row_ptr: np.ndarray      # [n_atoms + 1] int32, destination-sorted CSR of the graph
    src: np.ndarray          # [n_edges] int32, sources of each row in ascending order

    @property
    def n_atoms(self):
        return int(self.species.shape[0])

    @property
    def n_mols(self):
        return int(self.mol_ptr.shape[0] - 1)

    @property
    def n_edges(self):
        return int(self.src.shape[0])

    def dst(self):
        return np.repeat(np.arange(self.n_atoms, dtype=np.int32), np.diff(self.row_ptr))


def make_molecule_batch(seed, n_mols, min_atoms=10, max_atoms=50, fractions=SVP_FRACTIONS, keep=1.0):
    """Seeded batch: sizes uniform in [min_atoms, max_atoms], species drawn by
    `fractions`, and for each atom every other atom of its molecule as a
    source (fully connected), each edge then kept with probability `keep`.

    Stream (seed, 10): sizes, species, then the keep draws.
    """
    rng = np.random.default_rng((seed, 10))
    sizes = rng.integers(min_atoms, max_atoms + 1, size=n_mols)
    mol_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    n_atoms = int(mol_ptr[-1])
    species = rng.choice(len(fractions), size=n_atoms, p=np.asarray(fractions) / np.sum(fractions)).astype(np.int32)
    srcs, degs = [], np.zeros(n_atoms, np.int64)
    for b in range(n_mols):
        p, n = int(mol_ptr[b]), int(sizes[b])
        grid = np.broadcast_to(np.arange(p, p + n, dtype=np.int32), (n, n))
        off = ~np.eye(n, dtype=bool)
        srcs.append(grid[off])                       # row j: every other atom, ascending
        degs[p:p + n] = n - 1
    src = np.concatenate(srcs) if srcs else np.zeros(0, np.int32)
    row_ptr = np.concatenate([[0], np.cumsum(degs)])
    if keep < 1.0:
        kept = rng.random(src.shape[0]) < keep
        dst = np.repeat(np.arange(n_atoms), degs)
        src = src[kept]
        degs = np.bincount(dst[kept], minlength=n_atoms)
        row_ptr = np.concatenate([[0], np.cumsum(degs)])
    return MoleculeBatch(mol_ptr, species, row_ptr.astype(np.int32), src.astype(np.int32))


def make_matrix_values(seed, n_elems):
    """N(0, 1) float32 values for a batch's matrices stored back to back (stream (seed, 11))."""
    rng = np.random.default_rng((seed, 11))
    return rng.standard_normal(int(n_elems), dtype=np.float32)


def make_label_values(seed, n_rows, n_lab):
    """N(0, 1) float32 labels [n_rows][n_lab] (stream (seed, 12))."""
    rng = np.random.default_rng((seed, 12))
    return rng.standard_normal((int(n_rows), int(n_lab)), dtype=np.float32)


def make_edge_embeddings(cfg: Config | str, n_edges):
    """Seeded edge embeddings e [E][K][C] for the edge-update block (stream (seed, 5)),
    N(0, 1), held as the storage type holds them."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng((cfg.seed, 5))
    return round_storage(rng.standard_normal((int(n_edges), cfg.K, cfg.C)), cfg.storage)


def make_edge_cotangent(cfg: Config | str, n_edges):
    """Seeded cotangent Ge = dL/de' [E][K][C] of the edge-update block (stream (seed, 6))."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng((cfg.seed, 6))
    return round_storage(rng.standard_normal((int(n_edges), cfg.K, cfg.C)), "f32")
