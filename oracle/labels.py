"""Matrix <-> Label over whole Hamiltonian matrices with per-element bases (fp64).

Test infrastructure only (see oracle/__init__.py).

MALOQ Sec. III-B1 and III-B2: a dataset holds one dense Hamiltonian matrix per
structure, of size N_orb = sum over atoms of that atom's orbital count.  The
block H_ij between atoms i and j is cut out of it with an orbital template
T(Z_i, Z_j) (which rows and columns of the block the two elements carry),
moved into a buffer of the common, largest shape, and Eq. (1) turns every
shell-pair sub-block into its |L, M> components.  Labels of shell pairs an
element does not carry are the padding.  Label -> Matrix writes the blocks
back.  The two steps are taken in that order: extract into equally shaped
buffers, then transform (Matrix -> Label); transform back, then place
(Label -> Matrix).

Readings (the pages leave these open):
  R26 basis: one full shell list (the largest element's basis, or the union
       of the per-degree maxima); each element carries a subset of its
       shells, given as a bit mask.  An atom's orbitals are its shells in
       full-list order, each as m = -l..l.
  R27 padding: a label vector always has the layout of the full list (the
       channel k(a, b, L) of decode.label_layout, flattened in (L, M, k)
       order), and labels of shell pairs absent from (Z_i, Z_j) are zero.
  R28 matrices of a batch are stored back to back, each row-major
       N_orb x N_orb; atoms of a structure are contiguous and in order, so
       an atom's first orbital is the sum of the orbital counts before it.
  R29 which blocks: the on-site block of every atom and the block of every
       edge of the graph (rows = source atom's orbitals, columns =
       destination's, as in decode).  Edges with a nonzero periodic image
       shift, or whose ends lie in different structures, have no block in a
       dense molecular matrix: their labels are zero and nothing is written.
"""
from __future__ import annotations

import numpy as np

from .decode import label_layout, orbital_offsets, matrix_to_label, label_to_matrix


def species_templates(shell_l, species_shells):
    """Per element: map full orbital -> own orbital index (-1 if absent), and orbital count.

    One extra last row stands for an element index outside the table: it
    carries no orbitals (see species_rows)."""
    full_off, n_full = orbital_offsets(shell_l)
    omap = np.full((len(species_shells) + 1, n_full), -1, np.int64)
    n_orb = np.zeros(len(species_shells) + 1, np.int64)
    for z, mask in enumerate(species_shells):
        o = 0
        for a, l in enumerate(shell_l):
            if (int(mask) >> a) & 1:
                omap[z, full_off[a]:full_off[a] + 2 * l + 1] = np.arange(o, o + 2 * l + 1)
                o += 2 * l + 1
        n_orb[z] = o
    return omap, n_orb


def species_rows(species, species_shells):
    """Template row of every atom: its element, or the empty last row if out of range."""
    z = np.asarray(species, np.int64)
    return np.where((z >= 0) & (z < len(species_shells)), z, len(species_shells))


def orbital_layout(mol_ptr, species, shell_l, species_shells):
    """(atom_orb, atom_mol, mol_norb, mat_off) of R28."""
    _, n_orb = species_templates(shell_l, species_shells)
    mol_ptr = np.asarray(mol_ptr, np.int64)
    species = species_rows(species, species_shells)
    n_mols = len(mol_ptr) - 1
    atom_orb = np.zeros(len(species), np.int64)
    atom_mol = np.full(len(species), -1, np.int64)
    mol_norb = np.zeros(n_mols, np.int64)
    for b in range(n_mols):
        o = 0
        for a in range(mol_ptr[b], mol_ptr[b + 1]):
            atom_orb[a] = o
            atom_mol[a] = b
            o += n_orb[species[a]]
        mol_norb[b] = o
    mat_off = np.concatenate([[0], np.cumsum(mol_norb * mol_norb)])
    return atom_orb, atom_mol, mol_norb, mat_off


def flat_labels(h):
    """Labels h_L [N][2L+1][n_L] -> [N][n_lab] in (L, M, k) order."""
    return np.concatenate([x.reshape(x.shape[0], x.shape[1] * x.shape[2]) for x in h], axis=1)


def unflat_labels(hf, shell_l):
    _, n = label_layout(shell_l)
    out, q = [], 0
    for L, c in enumerate(n):
        w = (2 * L + 1) * c
        out.append(hf[:, q:q + w].reshape(-1, 2 * L + 1, c))
        q += w
    return out


def _block_index(zi, zj, omap, atom_orb_i, atom_orb_j, ld, base):
    """Flat matrix index of every full-layout entry of blocks (i, j), and its presence mask."""
    ri = omap[zi]                                   # [nb][n_full]
    cj = omap[zj]
    present = (ri[:, :, None] >= 0) & (cj[:, None, :] >= 0)
    idx = (base[:, None, None] + (atom_orb_i[:, None, None] + np.maximum(ri, 0)[:, :, None]) * ld[:, None, None]
           + atom_orb_j[:, None, None] + np.maximum(cj, 0)[:, None, :])
    return idx, present


def _blocks(src, dst, species, lay, shell_l, species_shells):
    """Index and presence of the edge blocks src -> dst, plus which edges have a block."""
    omap, _ = species_templates(shell_l, species_shells)
    atom_orb, atom_mol, mol_norb, mat_off = lay
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    has = (atom_mol[src] >= 0) & (atom_mol[src] == atom_mol[dst])
    mol = np.where(has, atom_mol[dst], 0)
    idx, present = _block_index(species[src], species[dst], omap, atom_orb[src], atom_orb[dst],
                                mol_norb[mol], mat_off[mol])
    present &= has[:, None, None]
    return idx, present, has


def matrix_to_labels(Hflat, src, dst, shift, species, lay, shell_l, species_shells):
    """Edge labels [E][n_lab] and node labels [n_atoms][n_lab] from the batch's matrices."""
    species = species_rows(species, species_shells)
    Hflat = np.asarray(Hflat, np.float64)
    n_atoms = len(species)

    def run(s, d, keep):
        idx, present, has = _blocks(s, d, species, lay, shell_l, species_shells)
        present &= np.asarray(keep, bool)[:, None, None]
        blk = np.where(present, Hflat[np.where(present, idx, 0)], 0.0)   # (1) extract, padded
        return flat_labels(matrix_to_label(blk, shell_l))                  # (2) Eq. (1)

    keep_e = np.ones(len(src), bool) if shift is None else ~np.any(np.asarray(shift) != 0, axis=1)
    h_edge = run(src, dst, keep_e)
    atoms = np.arange(n_atoms)
    h_node = run(atoms, atoms, np.ones(n_atoms, bool))
    return h_edge, h_node


def labels_to_matrix(h_edge, h_node, src, dst, shift, species, lay, shell_l, species_shells, Hflat=None):
    """Write the blocks of the given labels into the batch's matrices (other entries kept)."""
    species = species_rows(species, species_shells)
    atom_orb, atom_mol, mol_norb, mat_off = lay
    H = np.zeros(int(mat_off[-1])) if Hflat is None else np.array(Hflat, np.float64)
    n_atoms = len(species)

    def run(hf, s, d, keep):
        idx, present, has = _blocks(s, d, species, lay, shell_l, species_shells)
        present &= np.asarray(keep, bool)[:, None, None]
        blk = label_to_matrix(unflat_labels(np.asarray(hf, np.float64), shell_l), shell_l)
        H[idx[present]] = blk[present]

    keep_e = np.ones(len(src), bool) if shift is None else ~np.any(np.asarray(shift) != 0, axis=1)
    run(h_edge, src, dst, keep_e)
    atoms = np.arange(n_atoms)
    run(h_node, atoms, atoms, np.ones(n_atoms, bool))
    return H
