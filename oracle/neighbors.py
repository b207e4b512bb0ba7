"""Brute-force cutoff graph in the incoming-edge layout (fp64).

Test infrastructure only (see oracle/__init__.py).

"Distributed Equivariant GNNs" review, "What carries the argument": every node
owns all edges directed into it, so the graph is stored by destination (a CSR
whose rows are destinations).  The graph is the cutoff graph of the structure
(MALOQ Sec. I: orbital interactions need cutoffs up to 12 A, giving node
degrees over 100), periodic on the axes of the DFT cell (MALOQ Sec. III-D2).

Readings taken:
  * an edge (s -> d, image S) exists iff |x_d - (x_s + S*L)| < r_cut (strict),
    for every periodic image within the cutoff (not only the minimum image),
    except s = d with S = 0;
  * the distance is evaluated in fp64 exactly as
      p_a = x_s,a + fl(S_a L_a);  delta_a = x_d,a - p_a;
      d2 = fl(fl(delta_x^2 + delta_y^2) + delta_z^2)
    with no fused multiply-add, and compared with fl(r_cut^2);
  * rows are destinations 0..n_dst-1 (owned atoms); sources 0..n_src-1 are the
    owned atoms followed by ghosts, and ghosts are never rows;
  * within a row, edges are ordered by (s, S_x, S_y, S_z) ascending;
  * vec = f32(delta) points from the source image to the destination and
    dist = f32(sqrt(d2));
  * the source grouping lists, for every source, its edge ids in ascending order.
"""
from __future__ import annotations

import numpy as np


def image_range(box, periodic_mask, r_cut):
    """Image shifts S_a in [-ceil(r/L_a), ceil(r/L_a)] on periodic axes, {0} otherwise."""
    rng = []
    for a in range(3):
        if (periodic_mask >> a) & 1:
            n = int(np.ceil(r_cut / box[a]))
            rng.append(np.arange(-n, n + 1))
        else:
            rng.append(np.zeros(1, dtype=np.int64))
    sx, sy, sz = np.meshgrid(*rng, indexing="ij")
    return np.stack([sx.ravel(), sy.ravel(), sz.ravel()], axis=-1).astype(np.int64)


def row_edges(pos, d, box, periodic_mask, r_cut, shifts=None):
    """All incoming edges of destination d, sorted by (s, S).

    Returns (src [n], shift [n,3] int, vec [n,3] f32, dist [n] f32).
    """
    pos = np.asarray(pos, dtype=np.float64)
    box = np.asarray(box, dtype=np.float64)
    if shifts is None:
        shifts = image_range(box, periodic_mask, r_cut)
    n_src = pos.shape[0]
    rc2 = np.float64(r_cut) * np.float64(r_cut)
    # candidate (s, S) pairs; S outer so the lexicographic order is restored by the sort below
    off = shifts.astype(np.float64) * box[None, :]            # fl(S_a * L_a)
    p = pos[None, :, :] + off[:, None, :]                      # [nS, n_src, 3]
    delta = pos[d][None, None, :] - p
    d2 = (delta[..., 0] * delta[..., 0] + delta[..., 1] * delta[..., 1]) + delta[..., 2] * delta[..., 2]
    keep = d2 < rc2
    zero = np.all(shifts == 0, axis=1)
    if zero.any():
        keep[np.argmax(zero), d] = False
    si, ss = np.nonzero(keep.T)                                # s-major: [n_src, nS] order
    sh = shifts[ss]
    order = np.lexsort((sh[:, 2], sh[:, 1], sh[:, 0], si))
    si, ss, sh = si[order], ss[order], sh[order]
    dl = delta[ss, si]
    return (si.astype(np.int32), sh.astype(np.int8), dl.astype(np.float32),
            np.sqrt(d2[ss, si]).astype(np.float32))


def build_graph(pos, n_dst, box, periodic_mask, r_cut, rows=None):
    """Destination-sorted CSR of the cutoff graph, by brute force.

    With rows=None every destination 0..n_dst-1 is built and the source
    grouping is included; otherwise only the listed rows are built (rows are
    independent), which is how large structures are sampled.
    """
    pos = np.asarray(pos, dtype=np.float64)
    shifts = image_range(np.asarray(box, np.float64), periodic_mask, r_cut)
    which = range(n_dst) if rows is None else rows
    parts = [row_edges(pos, int(d), box, periodic_mask, r_cut, shifts) for d in which]
    counts = np.array([len(p[0]) for p in parts], dtype=np.int64)
    row_ptr = np.zeros(len(parts) + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    cat = (lambda i, shape, dt: np.concatenate([p[i] for p in parts]) if parts
           else np.zeros(shape, dt))
    g = {
        "row_ptr": row_ptr.astype(np.int32),
        "src": cat(0, (0,), np.int32),
        "shift": cat(1, (0, 3), np.int8),
        "vec": cat(2, (0, 3), np.float32),
        "dist": cat(3, (0,), np.float32),
        "n_dst": len(parts),
        "n_src": pos.shape[0],
        "rows": np.arange(n_dst) if rows is None else np.asarray(rows, dtype=np.int64),
    }
    if rows is None:
        E = int(row_ptr[-1])
        src_perm = np.argsort(g["src"], kind="stable").astype(np.int32)
        cnt = np.bincount(g["src"], minlength=pos.shape[0]) if E else np.zeros(pos.shape[0], np.int64)
        src_ptr = np.zeros(pos.shape[0] + 1, dtype=np.int64)
        np.cumsum(cnt, out=src_ptr[1:])
        g["src_ptr"] = src_ptr.astype(np.int32)
        g["src_perm"] = src_perm
    return g


def dst_of_edges(row_ptr):
    """Destination of every edge of a CSR."""
    counts = np.diff(np.asarray(row_ptr, dtype=np.int64))
    return np.repeat(np.arange(len(counts)), counts)
