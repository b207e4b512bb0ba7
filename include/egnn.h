/*
 * egnn.h -- C ABI of the MI355X (gfx950) SO(2) equivariant message-passing layer.
 *
 * One eSCN-style layer in the incoming-edge layout, its neighbour-list
 * builder, the per-edge Wigner-D generator and the Clebsch-Gordan decode of
 * irreps into orbital Hamiltonian blocks.  Sources the calls follow:
 *
 *   [Review]  "Distributed Equivariant Graph Neural Networks for Large-Scale
 *             Electronic Structure Prediction" (pith.science review of arXiv
 *             2507.03840), "What carries the argument": each node owns every
 *             edge directed into it; attention and aggregation run over
 *             those edges.
 *   [MALOQ]   "MALOQ: Massively Accelerated Learning of Operators for Quantum
 *             Transport" (arXiv 2606.28911v1): Sec. III and Fig. 2(a)
 *             (workflow), Sec. III-B1 Eq. (1) (CG transform of H blocks),
 *             Sec. III-C1 / Fig. 3(b,c) (Wigner-D rotation of each edge to +y),
 *             Sec. III-D (messages n_i (+) n_j, target node owns its edges),
 *             Sec. II-B1 (SO(3) -> SO(2) reduction).
 *
 * Conventions shared by every call
 *   - Every pointer is a DEVICE pointer unless marked "host".  The caller
 *     owns every buffer; the library keeps no pointer after a call returns
 *     and allocates no device memory inside a call.  Workspace sizes come
 *     from the *_sizes / *_workspace queries.  Constant tables (CG
 *     couplings) are built once per device on first use.
 *   - All argument checks run on the host before any launch.  A failing
 *     check returns a status and launches nothing; nothing aborts and no C++
 *     exception crosses the ABI.  HIP failures map to EGNN_E_HIP with the
 *     runtime's text in egnn_last_error() (thread-local).
 *   - Work is enqueued on `stream` (NULL = the default stream) and is
 *     asynchronous, except egnn_build_graph, which synchronises once to read
 *     the edge count.
 *   - Irreps are row-major [row][k][C], k = l*l + l + m, m = -l..l, in the
 *     real spherical-harmonic basis whose polar axis is y (the axis every
 *     edge is rotated onto) and whose degree-1 block is proportional to
 *     (x, y, z).  Storage type is fp32 or bf16 (EGNN_BF16, x/x_out/edge_out
 *     only); arithmetic accumulates in fp32.
 *   - Calls on one stream may be issued from one thread at a time.
 */
#ifndef EGNN_H
#define EGNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum {
  EGNN_OK = 0,
  EGNN_E_ARG = 1,          /* invalid argument (null pointer, bad size, bad flag)     */
  EGNN_E_CAPACITY = 2,     /* graph capacity too small; n_edges holds the need        */
  EGNN_E_HIP = 3,          /* HIP runtime error; see egnn_last_error()                */
  EGNN_E_UNSUPPORTED = 4,  /* valid request the library does not implement            */
  EGNN_E_WORKSPACE = 5     /* workspace or saved buffer smaller than the query said   */
} egnn_status;

typedef enum { EGNN_F32 = 0, EGNN_BF16 = 1 } egnn_dtype;

/* Static text for a status code (never NULL). */
const char *egnn_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *egnn_last_error(void);
/* Library ABI version (major*100 + minor). */
int egnn_version(void);

/* ---------------------------------------------------------------------------
 * Neighbour graph in the incoming-edge layout  [Review; MALOQ Sec. III-D, III-D2]
 *
 * Rows are destinations (owned atoms 0..n_dst-1); sources are atoms
 * 0..n_src-1, the owned atoms first and then ghosts (ghosts are never rows).
 * Edge (s -> d, image S in Z^3) exists iff
 *     |x_d - (x_s + S*box)| < r_cut  and not (s == d and S == 0),
 * evaluated in fp64 as  p_a = x_s,a + S_a*box_a;  delta_a = x_d,a - p_a;
 * d2 = (delta_x^2 + delta_y^2) + delta_z^2  (no fused multiply-add), compared
 * with r_cut*r_cut.  Every periodic image within the cutoff is an edge (not
 * only the minimum image).  Within a row edges are sorted by (s, S_x, S_y, S_z).
 *   vec  = (float)delta  (source image -> destination),
 *   dist = (float)sqrt(d2),
 *   src_ptr/src_perm = the edge ids of each source in ascending order
 *   (a CSR over sources, used by the forward source gather and the backward).
 * The output is deterministic (bit-identical between runs).
 * A graph handed to the layer calls must be consistent: row_ptr[n_dst] ==
 * n_edges, src_ptr[n_src] == n_edges, and src_perm a permutation of
 * 0..n_edges-1 grouped as above.  egnn_build_graph always produces such a
 * graph; a caller that assembles one itself (a prefix of rows, say) must
 * rebuild src_ptr/src_perm for its edges.  The kernels index with these
 * arrays without re-checking them.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t n_dst, n_src;        /* rows; sources (owned first, then ghosts)                  */
  int64_t capacity;            /* in: edges the arrays below can hold                       */
  int64_t n_edges;             /* out: edge count (also set on EGNN_E_CAPACITY)             */
  int32_t *row_ptr;            /* [n_dst+1]                                                 */
  int32_t *src;                /* [capacity]                                                */
  int8_t  *shift;              /* [capacity][3] image shift S in cell lengths               */
  float   *vec;                /* [capacity][3] x_dst - (x_src + S*box)                     */
  float   *dist;               /* [capacity]                                                */
  int32_t *src_ptr;            /* [n_src+1]                                                 */
  int32_t *src_perm;           /* [capacity]                                                */
} egnn_graph;

/* Workspace bytes for egnn_build_graph with the given capacity (host args).
 * The cell grid covers [lo, lo+box) on every axis; periodic axes wrap with
 * period box[a]; on open axes atoms outside the range are still handled
 * (they fall into the border cells). */
egnn_status egnn_build_graph_workspace(int32_t n_dst, int32_t n_src, const double lo[3] /*host*/,
                                       const double box[3] /*host*/, uint32_t periodic_mask,
                                       double r_cut, int64_t capacity, size_t *bytes /*host*/);

/* Build the graph from positions pos [n_src][3] (fp64, device).
 * periodic_mask: bit a set = axis a periodic.  g->n_dst, g->n_src and
 * g->capacity are inputs.  If the graph needs more than g->capacity edges,
 * returns EGNN_E_CAPACITY with g->n_edges = the need and writes only
 * row_ptr; call again with larger arrays and workspace.  Calling with
 * capacity 0 and NULL edge arrays is the way to learn the edge count
 * (row_ptr and src_ptr, whose sizes do not depend on it, are always needed).
 * A row or source with more than 65535 edges returns EGNN_E_UNSUPPORTED. */
egnn_status egnn_build_graph(const double *pos, const double lo[3] /*host*/,
                             const double box[3] /*host*/, uint32_t periodic_mask, double r_cut,
                             egnn_graph *g /*host struct, device arrays*/, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* Allocation-free egnn_build_graph, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as egnn_build_graph (the
 * capacity protocol included), without the workspace: the library's own
 * 32 MiB static device array serves as workspace, one copy per GPU it runs
 * on, held until the process ends.  The need is what
 * egnn_build_graph_workspace reports (about 8 bytes per edge of capacity,
 * 28 per atom and 12 per cell); a larger need returns EGNN_E_WORKSPACE
 * before any launch.  Calls on one GPU share that array, so calls that
 * overlap on one GPU (several streams or threads) race: the caller
 * serialises them.  The call's kernels clear whatever must start at zero.
 * Synchronises once to read the edge count, like egnn_build_graph. */
egnn_status egnn_build_graph_noalloc(const double *pos, const double lo[3] /*host*/,
                                     const double box[3] /*host*/, uint32_t periodic_mask, double r_cut,
                                     egnn_graph *g /*host struct, device arrays*/, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Source grouping of a graph given by its CSR  [review of arXiv 2507.03840,
 * "What carries the argument": the backward's reverse pattern; MALOQ Sec.
 * III-B2: Matrix <-> Label over a source atom's row strip of a matrix]
 *
 * egnn_build_graph writes src_ptr / src_perm itself.  For a graph made
 * elsewhere (row_ptr, src, n_src, n_edges), this writes them from src:
 * src_perm[src_ptr[s] .. src_ptr[s+1]) lists the edge ids of source s in
 * ascending order, s = 0..n_src-1.  Edges whose src lies outside [0, n_src)
 * are in no group: src_ptr[n_src] counts the grouped edges, and src_perm
 * past it is left as it was.  src_ptr [n_src + 1] and src_perm [n_edges] are
 * the caller's; n_edges <= 2^31 - 1.  A group is ordered by counting ranks,
 * quadratic in its size (fine for atom-sized groups).  The workspace (from the query) is the
 * caller's too, needs no clearing, and is not used after the call's kernels
 * end.  Asynchronous on `stream`; EGNN_E_WORKSPACE when ws_bytes is short.
 * ------------------------------------------------------------------------- */
egnn_status egnn_group_sources_workspace(int32_t n_src, int64_t n_edges, size_t *bytes /*host out*/);
egnn_status egnn_group_sources(egnn_graph *g /*host struct, device arrays*/, void *ws, size_t ws_bytes,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Layer description
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t lmax;     /* degrees 0..lmax, K = (lmax+1)^2 coefficients; 1..4, 6 or 8             */
  int32_t mmax;     /* orders kept in the edge frame, 0 <= mmax <= min(lmax, 2)               */
  int32_t C;        /* channels per coefficient; multiple of 8, 8 <= C <= 256                 */
  int32_t n_rbf;    /* Gaussian radial basis size, 2 <= n_rbf <= 16                            */
  double  r_cut;    /* cutoff of the radial envelope (same as the graph's)                    */
  int32_t storage;  /* egnn_dtype of x / x_out / edge_out / saved activations                 */
} egnn_layer_desc;

/* Packed fp32 weight count of one layer.  Order and row-major shapes:
 *   W0      [(lmax+1) C][(lmax+1) 2C]           (m = 0)
 *   W_m1, W_m2 for m = 1..mmax, each [(lmax-m+1) C][(lmax-m+1) 2C]
 *   W_rad   [n_rbf][n_pairs][2C], pairs (m, l): m = 0..mmax, l = m..lmax
 *   w_att   [C]
 * Row index of a W block = (l_out - m) C + c_out, column = (l_in - m) 2C + c_in,
 * input channels 0..C-1 = source, C..2C-1 = destination.  Returns 0 for an
 * invalid description. */
size_t egnn_layer_weight_count(const egnn_layer_desc *d);

/* ---------------------------------------------------------------------------
 * Edge geometry ("Compute Wigners", MALOQ Sec. III and III-C1, Fig. 3(b,c))
 *
 * Per edge: the rotation R_e taking vec/|vec| to +y with zero roll,
 *   r = (x,y,z), s = sqrt(x^2+z^2), (cos a, sin a) = (z/s, x/s) or (1,0),
 *   cos b = y, sin b = s,  R_e = (R_y(a) R_x(b))^T,
 * its Wigner blocks D^l(R_e) (defined by D^l(R) Y^l(r) = Y^l(R r)), of which
 * only the rows |m| <= mmax are stored, and the radial basis
 *   phi_k(d) = exp(-(d - mu_k)^2 / (2 sigma^2)) (cos(pi d / r_cut) + 1) / 2,
 *   mu_k = k r_cut / (n_rbf - 1), sigma = r_cut / (n_rbf - 1).
 * Layout: geom [n_edges][stride] fp32, stride = egnn_geom_stride(d):
 *   for l = 0..lmax, rows m = -min(l,mmax)..min(l,mmax), columns m' = -l..l
 *   (row-major within l, l blocks consecutive), then phi[0..n_rbf), then the
 *   edge's destination row as int32 bits, then zero padding.
 * geom must be 16-byte aligned (EGNN_E_ARG otherwise; hipMalloc and torch
 * allocations are).  The rotation is formed in fp64 and rounded once; the
 * recursion runs in fp32.
 * One geometry serves every layer on the same graph.
 * ------------------------------------------------------------------------- */
int32_t egnn_geom_stride(const egnn_layer_desc *d);     /* floats per edge, 0 if invalid */
egnn_status egnn_edge_geom(const egnn_layer_desc *d, const egnn_graph *g, float *geom,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * One message-passing layer, forward  [Review; MALOQ Sec. III, III-D, II-B1]
 *
 *   Xt_e  = trunc_{|m|<=mmax}( D_e x_src(e) (+) D_e x_dst(e) )      [K'][2C]
 *   X_e   = g_e * Xt_e,  g_e[(|m|,l), c'] = sum_k phi_k(d_e) W_rad[k][(|m|,l)][c']
 *   Y_e   : m = 0:  Y0 = W0 X0;  m >= 1:  Y+ = W_m1 X+ - W_m2 X-,
 *                                         Y- = W_m2 X+ + W_m1 X-        [K'][C]
 *   a_e   = sum_c w_att[c] SiLU(Y_e[l=0,m=0,c]);  alpha = softmax of a over each row
 *   msg_e = D_e^T Yhat_e  (Yhat = Y zero-padded to K)
 *   x_out[d] = x_in[d] + sum_{e in row d} alpha_e msg_e
 *   edge_out[e] = msg_e   (optional; the per-edge message an edge block consumes)
 * x_in [n_src][K][C], x_out [n_dst][K][C], edge_out [n_edges][K][C] or NULL,
 * weights packed fp32 (egnn_layer_weight_count).  `saved` (NULL for
 * inference) receives what egnn_layer_bwd needs; `ws` is scratch.  Both are
 * 16-byte aligned (EGNN_E_ARG otherwise; hipMalloc and torch allocations are).
 * x_out must not alias x_in.
 * ------------------------------------------------------------------------- */
egnn_status egnn_layer_sizes(const egnn_layer_desc *d, const egnn_graph *g,
                             size_t *saved_bytes /*host*/, size_t *ws_fwd_bytes /*host*/,
                             size_t *ws_bwd_bytes /*host*/);
egnn_status egnn_layer_fwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                           const float *weights, const void *x_in, void *x_out, void *edge_out,
                           void *saved, void *ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the same layer for the loss <grad_out, x_out>:
 *   grad_x_in [n_src][K][C] (fp32, overwritten) = dL/dx_in,
 *   grad_weights (fp32, packed like the weights, overwritten) = dL/dweights.
 * `saved` is what egnn_layer_fwd wrote for the same inputs; grad_out
 * [n_dst][K][C] fp32.  Reductions over edges run in a fixed order (no
 * floating-point atomics), so results are bit-identical between runs.
 * fp32 storage: every product in fp32 (MFMA).  bf16 storage: dL/dY is
 * rounded to bf16 and both gradient products (input and weight) run on bf16
 * MFMA with fp32 accumulation; x_in is the bf16 input; all gradients are fp32.
 * C <= 128 (EGNN_E_UNSUPPORTED otherwise). */
egnn_status egnn_layer_bwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                           const float *weights, const void *x_in, const void *saved,
                           const float *grad_out, float *grad_x_in, float *grad_weights,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Edge-update block  [MALOQ Sec. III-D: after the eSCN convolution the
 * messages n_i (+) n_j either aggregate onto node j (the node block above) or
 * update the edge embedding e_ij; Sec. III, Fig. 3(b): edge embeddings are
 * rotated like node embeddings]
 *
 *   e_out[e] = e_in[e] + D_e^T Yhat_e
 *
 * where Yhat_e is the SO(2) convolution of the gated edge-frame message, the
 * same per-edge message as egnn_layer_fwd's edge_out (same packed weights;
 * w_att is not used).  e_in / e_out: [n_edges][K][C] in the storage type,
 * 16-byte aligned; e_out may be e_in.  saved (for the backward) and the
 * workspace take the sizes egnn_layer_sizes returns for the layer.
 *
 * egnn_edge_update_bwd: gradients of <G_e, e_out> for grad_e_out = G_e, fp32
 * [n_edges][K][C]: grad_x_in [n_src][K][C] and grad_weights (packed, w_att
 * part zero) are overwritten.  The gradient with respect to e_in is G_e itself
 * (the update is a residual) and is not written.  C <= 128.
 * ------------------------------------------------------------------------- */
egnn_status egnn_edge_update_fwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                 const float *weights, const void *x_in, const void *e_in, void *e_out,
                                 void *saved, void *ws, size_t ws_bytes, hipStream_t stream);
egnn_status egnn_edge_update_bwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                 const float *weights, const void *x_in, const void *saved,
                                 const float *grad_e_out, float *grad_x_in, float *grad_weights,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Label -> Matrix: Hamiltonian blocks  [MALOQ Sec. III-B1 Eq. (1), Sec. III-B2]
 *
 * Shells (host list shell_l, each l <= 4; n_orb = sum(2l+1) <= 32).  For
 * ordered shell pairs (a, b) in lexicographic order and L = |la-lb|..la+lb
 * ascending, label channel k(a,b,L) counts the earlier pairs carrying L;
 * n_L = number of pairs carrying L.  Labels are h_L = W_L f^L (C -> n_L) and
 *   H[off_a+i][off_b+j] = sum_{L,M} Q^{(la,lb,L)}[i][j][M] h_L[M][k(a,b,L)]
 * with Q the real CG coupling ((D^la (x) D^lb) Q = Q D^L, orthonormal in M,
 * first entry of magnitude > 1e-9 in row-major (i,j,M) order positive).
 * Weights w_edge / w_node: fp32 [sum_L n_L][C], L ascending, rows k.
 * Edge blocks read edge irreps [n_edges][K][C] (rows = source orbitals,
 * columns = destination orbitals); on-site blocks read node irreps
 * [n_nodes][K][C], both 16-byte aligned (EGNN_E_ARG otherwise; hipMalloc and
 * torch allocations are).  Either part may be skipped with n = 0 / NULL.
 * Requires lmax >= 2*max(shell_l).
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t lmax;              /* degree range of the irreps (K = (lmax+1)^2)   */
  int32_t C;                 /* channels: 8, 16, 32, 64, 128 or 256           */
  int32_t n_shells;          /* 1..16                                         */
  const int32_t *shell_l;    /* host [n_shells]                               */
  int32_t storage;           /* egnn_dtype of the irreps                      */
} egnn_hdesc;

/* Label rows sum_L n_L for the shells (0 if invalid). */
int32_t egnn_hblocks_label_rows(const egnn_hdesc *h);
egnn_status egnn_hblocks(const egnn_hdesc *h, int64_t n_edges, int32_t n_nodes,
                         const float *w_edge, const float *w_node, const void *edge_irreps,
                         const void *node_irreps, float *h_edge /*[n_edges][n_orb][n_orb]*/,
                         float *h_onsite /*[n_nodes][n_orb][n_orb]*/, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Periodic Hamiltonian assembly  [MALOQ Sec. III Fig. 2(a), Sec. III-B2]
 *
 * The blocks of egnn_hblocks for a periodic structure form one matrix H(S)
 * per image shift S: the block of edge e (source atom s seen at image S,
 * destination d in the home cell) is H(S)[s, d], rows = source orbitals;
 * the on-site block of owned atom i is H(0)[i, i].  All images are written
 * as one block-sparse-row structure: block rows are the sources
 * 0..n_src-1; a row lists its blocks in ascending (destination, S_x, S_y,
 * S_z) order, each with its column (destination atom) and shift; an owned
 * atom's on-site block sits in that order at (i, 0, 0, 0).
 *   h_edge    [n_edges][n_orb][n_orb] fp32 (graph edge order)
 *   h_onsite  [n_dst][n_orb][n_orb] fp32, or NULL (no on-site blocks)
 *   nnzb    = n_edges (+ n_dst with on-site blocks)
 *   bsr_row_ptr [n_src + 1], bsr_col [nnzb], bsr_shift [nnzb][3] (int8),
 *   bsr_val [nnzb][n_orb][n_orb]: outputs, caller-allocated.
 * Needs the graph's row_ptr, shift, src_ptr and src_perm (as egnn_build_graph
 * makes them).  n_orb 1..32.  Asynchronous; a pure gather, bit-exact.
 * ------------------------------------------------------------------------- */
egnn_status egnn_assemble_bsr(const egnn_graph *g, int32_t n_orb, const float *h_edge, const float *h_onsite,
                              int32_t *bsr_row_ptr, int32_t *bsr_col, int8_t *bsr_shift, float *bsr_val,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Matrix <-> Label over whole matrices  [MALOQ Sec. III-B1 Eq. (1), Sec. III-B2]
 *
 * Basis: one full shell list (each l <= 4, at most 32 orbitals: the largest
 * element's basis, or the union of the per-degree maxima) and, per element,
 * a bit mask of the full shells it carries (its orbital template).  An
 * atom's orbitals are its shells in full-list order, m = -l..l each.
 *
 * Labels: n_lab = n_full^2 floats per node or edge, in the full list's
 * layout: for ordered shell pairs (a, b) in lexicographic order and L =
 * |la-lb|..la+lb ascending, channel k(a,b,L) counts the earlier pairs that
 * carry L, and label q = off(L) + (M+L) * n_L + k with off(L) = sum over
 * L' < L of (2L'+1) n_L'.  For a block between atoms i and j,
 *   h[q(a,b,L,M,k)] = sum_{m_a,m_b} Q^{(la,lb,L)}[m_a][m_b][M] H_ij[a m_a][b m_b]
 * with Q the real coupling of egnn_hblocks.  Labels of shell pairs that
 * element i or j lacks are zero (the padding to the largest element).
 *
 * Matrices: a batch of structures (molecules) with contiguous atoms, atoms
 * of structure s are mol_ptr[s]..mol_ptr[s+1]-1.  Structure s has one dense
 * row-major fp32 matrix of n_s x n_s entries (n_s = its atoms' orbital
 * counts summed), stored at element offset mat_off[s] of one array H of
 * h_elems = mat_off[n_mols] floats; an atom's first orbital is the sum of
 * the counts of the atoms before it in its structure.
 *
 * Blocks: the on-site block of every atom (h_node rows = atoms) and the
 * block of every graph edge (h_edge rows = edges, in the graph's order; rows
 * of H = the source atom's orbitals, columns = the destination's).  The
 * graph is a destination-sorted CSR over the batch's atoms (n_dst = n_src =
 * n_atoms; row_ptr, src, shift and n_edges are read; shift may be NULL).
 * When it also carries src_ptr and src_perm (both non-NULL), they must group
 * its edges by source as egnn_group_sources writes them; the blocks are then
 * taken one source atom at a time, so one wave reads (writes) that atom's
 * rows of the matrix, whole rows for a fully connected structure.  The
 * results are the same either way; edges in no group count as skipped.  An edge whose ends lie in different structures, or with a nonzero
 * image shift, has no block in a dense matrix: its labels are zero and
 * nothing is written.  Each ordered atom pair must appear at most once.
 *
 * All arrays are device memory owned by the caller; the library keeps no
 * pointer after a call.  Structure and atom arrays that the kernels read
 * are bounds-checked against n_atoms, n_mols and h_elems, so inconsistent
 * values cannot make a kernel leave the arrays; blocks that fail the checks
 * count as skipped.  n_invalid / n_skipped (device int64, may be NULL) are
 * overwritten with the count of structures with an invalid atom range plus
 * atoms whose element index is outside the table / of blocks with no place
 * in a matrix.  Asynchronous on `stream`.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t n_shells;                 /* full shell list, 1..16 shells          */
  const int32_t *shell_l;           /* host [n_shells], each 0..4             */
  int32_t n_species;                /* 1..64 elements                         */
  const uint32_t *species_shells;   /* host [n_species]: bit a = carries full shell a */
} egnn_basis;

typedef struct {
  int32_t n_mols, n_atoms;
  const int32_t *mol_ptr;           /* [n_mols+1], non-decreasing, 0 .. n_atoms          */
  const int32_t *species;           /* [n_atoms] element index into the basis            */
  int32_t *atom_orb;                /* [n_atoms] first orbital of the atom in its matrix */
  int32_t *atom_mol;                /* [n_atoms] structure of the atom (-1: none)        */
  int32_t *mol_norb;                /* [n_mols]  orbitals (matrix side) per structure    */
  int64_t *mat_off;                 /* [n_mols+1] element offset of each matrix in H     */
} egnn_orbitals;

/* Labels per node or edge (n_full^2) for the basis, 0 if it is invalid. */
int32_t egnn_label_width(const egnn_basis *b);

/* Fills atom_orb, atom_mol, mol_norb and mat_off from mol_ptr and species. */
egnn_status egnn_orbital_layout(const egnn_basis *b, egnn_orbitals *o, int64_t *n_invalid /*device or NULL*/,
                                hipStream_t stream);

/* Matrix -> Label: h_edge [n_edges][n_lab] (NULL: skip edges, as does g ==
 * NULL) and h_node [n_atoms][n_lab] (NULL: skip on-site blocks), both
 * overwritten, from H [h_elems]. */
egnn_status egnn_matrix_to_label(const egnn_basis *b, const egnn_orbitals *o, const egnn_graph *g,
                                 const float *H, int64_t h_elems, float *h_edge, float *h_node,
                                 int64_t *n_skipped /*device or NULL*/, hipStream_t stream);

/* Label -> Matrix: writes the template entries of every block given by
 * h_edge / h_node into H; entries of blocks not given are left as they are
 * (start from a zeroed H for a matrix with only the graph's blocks). */
egnn_status egnn_label_to_matrix(const egnn_basis *b, const egnn_orbitals *o, const egnn_graph *g,
                                 const float *h_edge, const float *h_node, float *H, int64_t h_elems,
                                 int64_t *n_skipped /*device or NULL*/, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Kernel timing (observability)
 *
 * When enabled, every entry point brackets each kernel launch with a pair of
 * HIP events recorded on the call's stream, tagged with the kernel family
 * and the launch's algorithmic work (FLOPs for the GEMMs, bytes each array is
 * read or written once for the rest).  egnn_timing_collect waits for the
 * recorded events, adds their elapsed times into per-family totals and
 * recycles the events; it returns the number of families written to `out`
 * (at most max_entries).  Events beyond an internal pool of 16384 are not
 * recorded (counted in `dropped`).  Process-wide; thread-safe.
 * ------------------------------------------------------------------------- */
typedef struct {
  char name[48];        /* kernel family, e.g. "gemm_nt_f32", "rotate_in"  */
  int64_t launches;
  double total_ms;
  double flops;         /* algorithmic FLOPs summed over the launches       */
  double bytes;         /* algorithmic HBM bytes summed over the launches   */
} egnn_timing_entry;

egnn_status egnn_timing_enable(int on);
int egnn_timing_collect(egnn_timing_entry *out /*host*/, int max_entries, int64_t *dropped /*host*/);
void egnn_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* EGNN_H */
