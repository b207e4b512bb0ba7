"""Label -> Matrix: Hamiltonian orbital blocks from edge and node irreps (fp64).

Test infrastructure only (see oracle/__init__.py).

MALOQ Sec. III-B1, Eq. (1): the sub-block H^{ab}_ij between a shell of degree
l_a on atom i and a shell of degree l_b on atom j is the tensor product
l_a (x) l_b, which the Clebsch-Gordan transform T writes as the direct sum of
degrees L = |l_a - l_b| .. l_a + l_b.  All |L, M> of a block are concatenated
into a label vector h_ij.  Label -> Matrix (Fig. 2(a), the last step of
inference) applies T^-1 = T^T blockwise.  Matrix -> Label (Sec. III-B2) is the
forward transform; it is kept here as the inverse used by the round-trip pin.

Readings:
  R20 the real coupling Q^{(la,lb,L)} of oracle.so3.real_coupling.
  R21 its sign rule (first significant entry positive).
  R22 one basis for every species: shells (s, s, p, p, d), l = [0, 0, 1, 1, 2],
      13 orbitals per atom (the GST structure of the review has 13 orbitals
      per atom), and species-independent decode weights.
  R23 no hermiticity symmetrisation.
  Label channels: for ordered shell pairs (a, b) in lexicographic order and
  L ascending, channel k(a, b, L) counts the earlier pairs that carry L.
  Labels are predicted by a per-degree linear map h_L = W_dec,L f^L (C -> n_L)
  of the edge irreps f (the last layer's per-edge message) or, for on-site
  blocks, of the node irreps x'.
  Rows of an edge block are the source atom's orbitals, columns the
  destination's.
"""
from __future__ import annotations

import numpy as np

from .so3 import real_coupling

SHELL_L = (0, 0, 1, 1, 2)


def orbital_offsets(shell_l=SHELL_L):
    off, o = [], 0
    for l in shell_l:
        off.append(o)
        o += 2 * l + 1
    return off, o


def label_layout(shell_l=SHELL_L):
    """([(a, b, L, k)], n_L list) for the shells, in the order stated in the module docstring."""
    lmax_lab = 2 * max(shell_l)
    n = [0] * (lmax_lab + 1)
    items = []
    for a, la in enumerate(shell_l):
        for b, lb in enumerate(shell_l):
            for L in range(abs(la - lb), la + lb + 1):
                items.append((a, b, L, n[L]))
                n[L] += 1
    return items, n


def labels_from_irreps(f, w_dec):
    """h_L [N][2L+1][n_L] = W_dec,L applied to the degree-L block of f [N][K][C]."""
    f = np.asarray(f, np.float64)
    h = []
    for L, wL in enumerate(w_dec):
        fL = f[:, L * L:(L + 1) * (L + 1), :]
        h.append(np.einsum("emc,kc->emk", fL, np.asarray(wL, np.float64)))
    return h


def label_to_matrix(h, shell_l=SHELL_L):
    """H [N][n_orb][n_orb] from labels h_L [N][2L+1][n_L] (Eq. (1) inverted blockwise)."""
    items, _ = label_layout(shell_l)
    off, n_orb = orbital_offsets(shell_l)
    N = h[0].shape[0]
    H = np.zeros((N, n_orb, n_orb))
    for a, b, L, k in items:
        la, lb = shell_l[a], shell_l[b]
        Q = real_coupling(la, lb, L)                             # [2la+1][2lb+1][2L+1]
        blk = np.einsum("ijM,eM->eij", Q, h[L][:, :, k])
        H[:, off[a]:off[a] + 2 * la + 1, off[b]:off[b] + 2 * lb + 1] += blk
    return H


def matrix_to_label(H, shell_l=SHELL_L):
    """Labels h_L from blocks H (the forward transform T of Eq. (1))."""
    items, n = label_layout(shell_l)
    off, _ = orbital_offsets(shell_l)
    N = H.shape[0]
    h = [np.zeros((N, 2 * L + 1, n[L])) for L in range(len(n))]
    for a, b, L, k in items:
        la, lb = shell_l[a], shell_l[b]
        Q = real_coupling(la, lb, L)
        blk = H[:, off[a]:off[a] + 2 * la + 1, off[b]:off[b] + 2 * lb + 1]
        h[L][:, :, k] = np.einsum("ijM,eij->eM", Q, blk)
    return h


def hblocks(f, w_dec, shell_l=SHELL_L):
    """Hamiltonian blocks [N][13][13] from irreps f [N][K][C] and W_dec,L [n_L][C]."""
    return label_to_matrix(labels_from_irreps(f, w_dec), shell_l)


def assemble_bsr(src, dst, shift, h_edge, h_onsite, n_src):
    """Label -> Matrix for a periodic structure (MALOQ Sec. III, Fig. 2(a): the
    predicted blocks become the Hamiltonian; Sec. III-B2: matrix assembly).

    The periodic Hamiltonian is one matrix H(S) per image shift S; the block
    of edge e (source atom s at image S, destination atom d in the home cell,
    rows = source orbitals, columns = destination orbitals) is H(S)[s, d], and
    the on-site block of owned atom i is H(0)[i, i].

    Reading R32: all images are held in one block-sparse row (BSR) structure:
    block rows are source atoms 0..n_src-1, a row lists its blocks in
    ascending (destination, S_x, S_y, S_z) order, each with its column
    (destination atom) and its shift; owned atoms (i < len(h_onsite)) carry
    their on-site block in that order at (i, 0, 0, 0).

    Returns row_ptr [n_src + 1], col [nnzb], shift [nnzb][3] (int8) and
    val [nnzb][n_orb][n_orb].
    """
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    shift = np.asarray(shift, np.int64).reshape(-1, 3)
    h_edge = np.asarray(h_edge)
    h_onsite = np.asarray(h_onsite)
    n_on = h_onsite.shape[0]
    rows = np.concatenate([src, np.arange(n_on)])
    cols = np.concatenate([dst, np.arange(n_on)])
    sh = np.concatenate([shift, np.zeros((n_on, 3), np.int64)])
    val = np.concatenate([h_edge, h_onsite]) if n_on else h_edge
    order = np.lexsort((sh[:, 2], sh[:, 1], sh[:, 0], cols, rows))
    counts = np.bincount(rows, minlength=n_src) if len(rows) else np.zeros(n_src, np.int64)
    row_ptr = np.concatenate([[0], np.cumsum(counts)])
    return row_ptr, cols[order], sh[order].astype(np.int8), val[order]
