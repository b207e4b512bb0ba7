"""One SO(2)-reduced equivariant message-passing layer, forward and analytic backward (fp64).

Test infrastructure only (see oracle/__init__.py).

The layer, step by step, as the pages describe it:
  1. MALOQ Sec. III-D: the message of edge i -> j starts from the concatenated
     node embeddings n_i (+) n_j (source channels first, then destination).
  2. MALOQ Sec. III-C1, Fig. 3(b): both are rotated into the edge frame, where
     the edge points along +y, by the block-diagonal Wigner-D of the edge.
  3. MALOQ Sec. II-B1 and Sec. III (eSCN): in that frame the SO(3) tensor
     product reduces to SO(2) -- "constrained linear layers" acting per order m.
  4. The review of arXiv 2507.03840, "What carries the argument": attention
     over the messages directed into each node, with no communication since
     the node owns those edges.
  5. MALOQ Sec. III: messages are rotated back and aggregated onto their
     target node (node block); the per-edge message is also what an edge
     block consumes.

Readings (the pages leave these open):
  R10 channels 0..C-1 of the message are the source, C..2C-1 the destination.
  R11 radial basis: phi_k(d) = exp(-(d-mu_k)^2 / (2 sigma^2)) * (cos(pi d/r_c)+1)/2
      with mu_k = k r_c/(n_rbf-1), sigma = r_c/(n_rbf-1).
  R12 the radial basis enters as per-(|m|, l, channel) input gates
      g = phi(d) W_rad (a linear map, no bias), shared by +m and -m.
  R13 coefficients with |m| > mmax are dropped in the edge frame.
  R14 per m >= 1 the SO(2) map is
        Y+ = W_m1 X+ - W_m2 X-,   Y- = W_m2 X+ + W_m1 X-
      (a complex multiplication, which commutes with the roll about y); W0
      acts on m = 0.  No bias, no nonlinearity inside.
  R16 one attention head: a_e = sum_c w_att[c] SiLU(Y_e[l=0, m=0, c]),
      alpha = softmax of a over the incoming edges of the destination.
  R17 residual update x'_d = x_d + sum_e alpha_e msg_e, msg_e = D_e^T Yhat_e.
  R18 the per-edge message msg_e (before alpha) is the edge output.
  R19 a destination with no incoming edge keeps x'_d = x_d.
  R24 backward: the loss is <G, x'> for a given cotangent G.
  R25 no gradient with respect to positions.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import so3
from .neighbors import dst_of_edges


@dataclass(frozen=True)
class LayerDesc:
    lmax: int
    mmax: int
    C: int
    n_rbf: int
    r_cut: float

    @property
    def K(self):
        return (self.lmax + 1) ** 2

    def m_pairs(self):
        """(m, l) pairs of the radial gates, m = 0..mmax, l = m..lmax."""
        return [(m, l) for m in range(self.mmax + 1) for l in range(m, self.lmax + 1)]


def unpack_weights(w, d: LayerDesc):
    """Split the packed weight vector.

    Packed order: W0 [(lmax+1)C][(lmax+1)2C], then for m = 1..mmax
    W_m1, W_m2 [(lmax-m+1)C][(lmax-m+1)2C], then W_rad [n_rbf][n_pairs][2C],
    then w_att [C].  Row index of a W block = (l_out - m) C + c_out, column
    index = (l_in - m) 2C + c_in.
    """
    w = np.asarray(w, dtype=np.float64).ravel()
    out, o = {}, 0

    def take(shape):
        nonlocal o
        n = int(np.prod(shape))
        a = w[o:o + n].reshape(shape)
        o += n
        return a
    C, L = d.C, d.lmax
    out["W0"] = take(((L + 1) * C, (L + 1) * 2 * C))
    for m in range(1, d.mmax + 1):
        nl = L - m + 1
        out[f"W{m}_1"] = take((nl * C, nl * 2 * C))
        out[f"W{m}_2"] = take((nl * C, nl * 2 * C))
    out["W_rad"] = take((d.n_rbf, len(d.m_pairs()), 2 * C))
    out["w_att"] = take((C,))
    if o != w.size:
        raise ValueError(f"weight vector has {w.size} entries, layout needs {o}")
    return out


def pack_weights(parts, d: LayerDesc):
    """Inverse of unpack_weights."""
    seq = [parts["W0"]]
    for m in range(1, d.mmax + 1):
        seq += [parts[f"W{m}_1"], parts[f"W{m}_2"]]
    seq += [parts["W_rad"], parts["w_att"]]
    return np.concatenate([np.asarray(a, np.float64).ravel() for a in seq])


def radial_basis(dist, d: LayerDesc):
    """phi [E][n_rbf] (reading R11)."""
    r = np.asarray(dist, dtype=np.float64)[:, None]
    n = d.n_rbf
    mu = np.arange(n) * d.r_cut / (n - 1)
    sigma = d.r_cut / (n - 1)
    env = 0.5 * (np.cos(np.pi * r / d.r_cut) + 1.0)
    return np.exp(-((r - mu[None, :]) ** 2) / (2.0 * sigma * sigma)) * env


def silu(z):
    return z / (1.0 + np.exp(-z))


def dsilu(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def edge_wigner(vec, lmax, roll=None):
    """Per-edge Wigner blocks D^l(R_e), l = 0..lmax, each [E][2l+1][2l+1].

    `roll` (per-edge angle, tests only) replaces R_e by R_y(roll) R_e, another
    rotation taking the edge to +y; the layer must not depend on it.
    """
    R = so3.edge_frame(np.asarray(vec, np.float64))
    if roll is not None:
        c, s = np.cos(roll), np.sin(roll)
        Ry = np.zeros((len(roll), 3, 3))
        Ry[:, 0, 0], Ry[:, 0, 2], Ry[:, 1, 1], Ry[:, 2, 0], Ry[:, 2, 2] = c, s, 1.0, -s, c
        R = Ry @ R
    return so3.wigner_blocks(R, lmax)


def rotate_in(D, x_rows, d: LayerDesc):
    """Edge-frame coefficients D^l x^l for every l, all m: [E][K][ch]."""
    out = np.zeros_like(x_rows)
    for l in range(d.lmax + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        out[:, sl, :] = np.einsum("emn,enc->emc", D[l], x_rows[:, sl, :])
    return out


def rotate_out(D, y, d: LayerDesc):
    """Back to the global frame: D^l^T y^l for every l: [E][K][ch]."""
    out = np.zeros_like(y)
    for l in range(d.lmax + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        out[:, sl, :] = np.einsum("emn,emc->enc", D[l], y[:, sl, :])
    return out


def trunc_mask(d: LayerDesc):
    """Boolean [K]: coefficient kept in the edge frame (|m| <= mmax)."""
    keep = np.zeros(d.K, dtype=bool)
    for l in range(d.lmax + 1):
        for m in range(-l, l + 1):
            keep[so3.coeff_index(l, m)] = abs(m) <= d.mmax
    return keep


def gates(phi, W, d: LayerDesc):
    """g [E][K][2C]: gate of every kept coefficient (shared by +m and -m), 0 elsewhere."""
    gp = np.einsum("ek,kpc->epc", phi, W["W_rad"])           # [E][n_pairs][2C]
    g = np.zeros((phi.shape[0], d.K, 2 * d.C))
    for p, (m, l) in enumerate(d.m_pairs()):
        g[:, so3.coeff_index(l, m), :] = gp[:, p, :]
        if m > 0:
            g[:, so3.coeff_index(l, -m), :] = gp[:, p, :]
    return g


def _m_block(a, m, d: LayerDesc, sign):
    """Gather coefficients (l, sign*m), l = m..lmax, flattened [E][(l - m) ch + c]."""
    idx = [so3.coeff_index(l, sign * m) for l in range(m, d.lmax + 1)]
    return a[:, idx, :].reshape(a.shape[0], -1)


def _m_scatter(out, vals, m, d: LayerDesc, sign, ch):
    idx = [so3.coeff_index(l, sign * m) for l in range(m, d.lmax + 1)]
    out[:, idx, :] = vals.reshape(vals.shape[0], len(idx), ch)


def so2_conv(X, W, d: LayerDesc):
    """Y [E][K][C] from the gated edge-frame input X [E][K][2C] (reading R14)."""
    E, C = X.shape[0], d.C
    Y = np.zeros((E, d.K, C))
    _m_scatter(Y, _m_block(X, 0, d, +1) @ W["W0"].T, 0, d, +1, C)
    for m in range(1, d.mmax + 1):
        xp, xm = _m_block(X, m, d, +1), _m_block(X, m, d, -1)
        w1, w2 = W[f"W{m}_1"], W[f"W{m}_2"]
        _m_scatter(Y, xp @ w1.T - xm @ w2.T, m, d, +1, C)
        _m_scatter(Y, xp @ w2.T + xm @ w1.T, m, d, -1, C)
    return Y


def so2_conv_bwd(X, dY, W, d: LayerDesc):
    """(dX [E][K][2C], dW dict) for Y = so2_conv(X)."""
    E, C = X.shape[0], d.C
    dX = np.zeros((E, d.K, 2 * C))
    dW = {}
    dy0, x0 = _m_block(dY, 0, d, +1), _m_block(X, 0, d, +1)
    _m_scatter(dX, dy0 @ W["W0"], 0, d, +1, 2 * C)
    dW["W0"] = dy0.T @ x0
    for m in range(1, d.mmax + 1):
        xp, xm = _m_block(X, m, d, +1), _m_block(X, m, d, -1)
        gp, gm = _m_block(dY, m, d, +1), _m_block(dY, m, d, -1)
        w1, w2 = W[f"W{m}_1"], W[f"W{m}_2"]
        _m_scatter(dX, gp @ w1 + gm @ w2, m, d, +1, 2 * C)
        _m_scatter(dX, -gp @ w2 + gm @ w1, m, d, -1, 2 * C)
        dW[f"W{m}_1"] = gp.T @ xp + gm.T @ xm
        dW[f"W{m}_2"] = -gp.T @ xm + gm.T @ xp
    return dX, dW


def segment_softmax(a, row_ptr):
    """alpha_e = exp(a_e - max_row) / sum_row exp(. - max_row) over each CSR row."""
    alpha = np.zeros_like(a)
    rp = np.asarray(row_ptr, dtype=np.int64)
    for r in range(len(rp) - 1):
        b, e = rp[r], rp[r + 1]
        if e > b:
            z = np.exp(a[b:e] - a[b:e].max())
            alpha[b:e] = z / z.sum()
    return alpha


def segment_sum(vals, row_ptr):
    """out[r] = sum of vals over the edges of row r (zero for an empty row)."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    out = np.zeros((len(rp) - 1,) + vals.shape[1:])
    for r in range(len(rp) - 1):
        if rp[r + 1] > rp[r]:
            out[r] = vals[rp[r]:rp[r + 1]].sum(axis=0)
    return out


def edge_forward(graph, x, W, d: LayerDesc, x_dst_rows, roll=None):
    """Per-edge quantities of the forward pass for the edges of `graph`.

    x holds the source rows (indexed by graph['src']); x_dst_rows[e] is the
    destination row of edge e.  Returns a dict of edge arrays.
    """
    D = edge_wigner(graph["vec"], d.lmax, roll)
    phi = radial_basis(graph["dist"], d)
    keep = trunc_mask(d)
    xs = np.asarray(x, np.float64)[graph["src"]]
    xt = np.concatenate([xs, x_dst_rows], axis=2)             # n_i (+) n_j  [E][K][2C]
    Xt = rotate_in(D, xt, d) * keep[None, :, None]             # edge frame, m-truncated
    g = gates(phi, W, d)
    X = g * Xt
    Y = so2_conv(X, W, d)
    a = silu(Y[:, 0, :]) @ W["w_att"]
    msg = rotate_out(D, Y, d)
    return dict(D=D, phi=phi, Xt=Xt, g=g, X=X, Y=Y, a=a, msg=msg)


def layer_forward(graph, x, w, d: LayerDesc, roll=None):
    """Forward of one layer over every row of `graph`.

    graph: CSR from oracle.neighbors (rows = destinations 0..n_dst-1)
    x: [n_src][K][C] node irreps (owned first), w: packed weights.
    Returns dict with x_out [n_dst][K][C], edge_out (= msg) [E][K][C],
    alpha [E], logits [E] and the per-edge intermediates.
    """
    W = unpack_weights(w, d)
    x = np.asarray(x, np.float64)
    n_dst = len(graph["row_ptr"]) - 1
    dst = dst_of_edges(graph["row_ptr"])
    ef = edge_forward(graph, x, W, d, x[dst], roll)
    alpha = segment_softmax(ef["a"], graph["row_ptr"])
    agg = segment_sum(alpha[:, None, None] * ef["msg"], graph["row_ptr"])
    ef.update(alpha=alpha, logits=ef["a"], x_out=x[:n_dst] + agg, edge_out=ef["msg"])
    return ef


def layer_forward_rows(graph, x, w, d: LayerDesc, chunk_edges=16384):
    """Same x_out / alpha as layer_forward, in row-aligned chunks (bounded memory).

    Returns (x_out [n_rows][K][C], alpha [E]).  Only the rows present in
    `graph` are computed; their destination atoms are given by graph['rows']
    when the graph was built for a subset of rows, else 0..n_rows-1.
    """
    W = unpack_weights(w, d)
    x = np.asarray(x, np.float64)
    rp = np.asarray(graph["row_ptr"], np.int64)
    n_rows = len(rp) - 1
    rows = np.asarray(graph.get("rows", np.arange(n_rows)))
    out = np.empty((n_rows, d.K, d.C))
    alpha_all = np.empty(int(rp[-1]))
    r0 = 0
    while r0 < n_rows:
        r1 = r0 + 1
        while r1 < n_rows and rp[r1 + 1] - rp[r0] <= chunk_edges:
            r1 += 1
        b, e = rp[r0], rp[r1]
        sub = {k: graph[k][b:e] for k in ("src", "vec", "dist")}
        sub_rp = rp[r0:r1 + 1] - b
        dst_local = dst_of_edges(sub_rp)
        ef = edge_forward(sub, x, W, d, x[rows[r0:r1]][dst_local])
        alpha = segment_softmax(ef["a"], sub_rp)
        agg = segment_sum(alpha[:, None, None] * ef["msg"], sub_rp)
        out[r0:r1] = x[rows[r0:r1]] + agg
        alpha_all[b:e] = alpha
        r0 = r1
    return out, alpha_all


def layer_backward(graph, x, w, d: LayerDesc, fwd, G):
    """Analytic gradients of <G, x'> with respect to x [n_src][K][C] and the packed weights.

    Reverse of layer_forward, step by step:
      dmsg_e = alpha_e G_d,  dalpha_e = <msg_e, G_d>,
      da_e = alpha_e (dalpha_e - sum_row alpha dalpha),
      dY = D_e dmsg_e (truncated) + logit term on Y[l=0, m=0],
      (dX, dW) = SO(2) backward,  dXt = g * dX,  dg = sum_{+-m} dX * Xt,
      dx_src += D_e^T dXt[:, :C],  dx_dst += D_e^T dXt[:, C:],  dx_dst += G.
    """
    W = unpack_weights(w, d)
    x = np.asarray(x, np.float64)
    G = np.asarray(G, np.float64)
    C, n_src = d.C, x.shape[0]
    n_dst = len(graph["row_ptr"]) - 1
    dst = dst_of_edges(graph["row_ptr"])
    D, alpha, Y = fwd["D"], fwd["alpha"], fwd["Y"]
    keep = trunc_mask(d)
    Gd = G[dst]
    dmsg = alpha[:, None, None] * Gd
    dalpha = np.einsum("ekc,ekc->e", fwd["msg"], Gd)
    s = segment_sum(alpha * dalpha, graph["row_ptr"])
    da = alpha * (dalpha - s[dst])
    dY = rotate_in(D, dmsg, d) * keep[None, :, None]
    y00 = Y[:, 0, :]
    dY[:, 0, :] += da[:, None] * W["w_att"][None, :] * dsilu(y00)
    dw_att = silu(y00).T @ da
    dx, dW = _backward_from_dY(graph, x, W, d, fwd, dY)
    dW["w_att"] = dw_att
    dx[:n_dst] += G
    return dx, pack_weights(dW, d)


def _backward_from_dY(graph, x, W, d: LayerDesc, fwd, dY):
    """The steps shared by the node and edge blocks, from the edge-frame output
    gradient dY: (dX, dW) = SO(2) backward, dXt = g * dX, dg = sum_{+-m} dX * Xt,
    dx_src += D_e^T dXt[:, :C], dx_dst += D_e^T dXt[:, C:].  Returns dx and the
    weight gradients (w_att zero)."""
    C = d.C
    n_dst = len(graph["row_ptr"]) - 1
    D = fwd["D"]
    dX, dW = so2_conv_bwd(fwd["X"], dY, W, d)
    dXt = fwd["g"] * dX
    dgfull = dX * fwd["Xt"]                                     # [E][K][2C]
    dgp = np.zeros((D[0].shape[0], len(d.m_pairs()), 2 * C))
    for p, (m, l) in enumerate(d.m_pairs()):
        dgp[:, p, :] = dgfull[:, so3.coeff_index(l, m), :]
        if m > 0:
            dgp[:, p, :] += dgfull[:, so3.coeff_index(l, -m), :]
    dW["W_rad"] = np.einsum("ek,epc->kpc", fwd["phi"], dgp)
    dW["w_att"] = np.zeros_like(W["w_att"])
    back = rotate_out(D, dXt, d)                                # [E][K][2C]
    dx = np.zeros_like(x)
    np.add.at(dx, graph["src"], back[:, :, :C])
    dx[:n_dst] += segment_sum(back[:, :, C:], graph["row_ptr"])
    return dx, dW


def edge_update_forward(graph, x, e, w, d: LayerDesc, roll=None):
    """Edge-update block (MALOQ Sec. III-D: after the eSCN convolution the
    messages n_i (+) n_j either aggregate onto node j or update the edge
    embedding e_ij; Sec. III / Fig. 3(b) rotate edge embeddings like node
    embeddings).

    Reading R30: e'_e = e_e + D_e^T Yhat_e, with Yhat_e the SO(2) convolution
    of the gated edge-frame message of the node block (same weights, no
    attention).  e: [E][K][C].  Returns the forward dict with e_out.
    """
    W = unpack_weights(w, d)
    x = np.asarray(x, np.float64)
    dst = dst_of_edges(graph["row_ptr"])
    ef = edge_forward(graph, x, W, d, x[dst], roll)
    ef["e_out"] = np.asarray(e, np.float64) + ef["msg"]
    return ef


def edge_update_backward(graph, x, w, d: LayerDesc, fwd, Ge):
    """Gradients of <Ge, e'> with respect to x [n_src][K][C], e and the packed
    weights: de = Ge; dY = D_e Ge (truncated); the rest as the node block."""
    W = unpack_weights(w, d)
    x = np.asarray(x, np.float64)
    Ge = np.asarray(Ge, np.float64)
    dY = rotate_in(fwd["D"], Ge, d) * trunc_mask(d)[None, :, None]
    dx, dW = _backward_from_dY(graph, x, W, d, fwd, dY)
    return dx, Ge.copy(), pack_weights(dW, d)
