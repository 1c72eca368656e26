"""Equivariant message-passing attention potential: layers, energy, forces (oracle).

What is computed follows "Ab Initio Accuracy Beyond the Cutoff" (Abstract):
an equivariant message-passing Transformer whose stacked layers pass
information beyond one cutoff, with forces from back-propagating the energy.
The layer is the plainest form consistent with that description and with the
equivariant tensor-product networks of "Unlocking Tensor Core Performance"
(section "Why MLIPs Need Dedicated Performance Optimization"):

For atom i, features h_i^l in R^{C x (2l+1)}, l = 0..lmax.  Layer input at
t = 1: h^0 = E_emb[species], h^{l>0} = 0.  Heads split the channels into H
contiguous groups of d_h = C/H; k(c) = c // d_h.  For every edge e = (i <- j)
with r_ij = x_j - x_i (minimum image), r = |r_ij|, unit vector rhat:

  1  ht_i^l = W_v^l h_i^l           q_i = W_q h_i^0
  2  w_e[p, c] = u(r) * (W_2 SiLU(W_1 B(r)))[p*C + c]        (radial MLP, no biases)
  3  v_e^{l3}[c, m3] = sum_{p=(l1,l2,l3)} w_e[p,c] sum_{m1,m2} CG_p[m1,m2,m3] ht_j^{l1}[c,m1] Y_{l2 m2}(rhat)
  4  a_e^k = d_h^{-1/2} sum_{c in head k} q_i[c] v_e^0[c]
  5  alpha_e^k = u(r_e) exp(a_e^k - M_i^k) / Z_i^k,  Z_i^k = sum_{e' in row i} u(r_e') exp(a_e'^k - M_i^k)
     (M_i^k: max over the row's edges with r < r_cut; alpha = 0 when Z = 0)
  6  m_i^l[c, :] = sum_{e in row i} alpha_e^{k(c)} v_e^l[c, :]
  7  h_i^0 += SiLU(W_o^0 m_i^0);  gamma_i = sigmoid(W_g m_i^0);
     h_i^l[c, :] += gamma_i[(l-1)C + c] * (W_o^l m_i^l)[c, :]   (l >= 1)

Energy: E_i = sum_c w_out[c] SiLU((W_r h_i^0)[c]), E = sum_i E_i ("Choosing a
Precision Strategy": the energy sum is kept in high precision).  Forces:
F = -dE/dx by reverse-mode differentiation (one backward pass, as in the
"Fused Gradient Inference Pipeline" of "Exascale Multi-Task Graph Foundation
Models", Fig. 5).

The weight blob is row-major [out][in] float32, in this order: E_emb [S][C];
per layer: W_1 [64][NB], W_2 [P*C][64], W_q [C][C], W_v^0..lmax, W_o^0..lmax
(each [C][C]), W_g [lmax*C][C]; then W_r [C][C], w_out [1][C].

Edges with r >= r_cut have u = 0, so they add exactly zero to every sum above
and to every derivative (u, u' and u'' vanish at r_cut); they are dropped.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

from . import basis
from .cg import cg_table, paths


class Params:
    """fp64 views of the float32 weight blob."""

    def __init__(self, cfg, flat):
        C, Hr, NB, L = cfg.channels, cfg.radial_hidden, cfg.n_bessel, cfg.lmax
        P = len(paths(L))
        t = torch.tensor(np.asarray(flat, np.float32).astype(np.float64))
        off = 0

        def take(r, c):
            nonlocal off
            m = t[off:off + r * c].view(r, c)
            off += r * c
            return m

        self.emb = take(cfg.n_species, C)
        self.layers = []
        for _ in range(cfg.layers):
            d = {"w1": take(Hr, NB), "w2": take(P * C, Hr), "wq": take(C, C)}
            d["wv"] = [take(C, C) for _ in range(L + 1)]
            d["wo"] = [take(C, C) for _ in range(L + 1)]
            d["wg"] = take(L * C, C)
            self.layers.append(d)
        self.wr = take(C, C)
        self.wout = take(1, C)
        assert off == t.numel(), "weight blob size does not match the configuration"


def _as_f64(pos):
    """float32 positions are widened exactly; float64 positions are used as given."""
    a = np.asarray(pos)
    return a.astype(np.float64) if a.dtype != np.float64 else a.copy()


def edge_geometry(P, L, row, col):
    """P [N,3] float64; returns r [E], rhat [E,3] for edges (row <- col)."""
    d = P[col] - P[row]
    if L is not None:
        d = d - L * torch.round(d / L)
    r = torch.linalg.norm(d, dim=1)
    return r, d / r[:, None]


def csr_rows(row_ptr):
    rp = np.asarray(row_ptr, np.int64)
    return torch.tensor(np.repeat(np.arange(rp.size - 1), np.diff(rp)))


def _messages(cfg, lw, ht, q, r, rhat, row, col, n_atoms, cgs):
    """Steps 2-6 for the edges given (receivers row < n_atoms): m as a list over l of
    [n_atoms, C, 2l+1].  ht: list over l of [*, C, 2l+1] indexed by col; q: [n_atoms, C]."""
    C, Hh, L = cfg.channels, cfg.heads, cfg.lmax
    dh = C // Hh
    head = torch.arange(C) // dh
    B = basis.bessel(r, cfg.cutoff, cfg.n_bessel)
    u = basis.envelope(r, cfg.cutoff)
    Y = basis.real_sh(rhat, L)
    w = (F.silu(B @ lw["w1"].T) @ lw["w2"].T) * u[:, None]
    E = r.shape[0]
    w = w.view(E, len(paths(L)), C)
    htj = [ht[l][col] for l in range(L + 1)]
    v = [torch.zeros(E, C, 2 * l + 1, dtype=torch.float64) for l in range(L + 1)]
    for p, (l1, l2, l3) in enumerate(paths(L)):
        Mp = torch.einsum("abc,eb->eac", cgs[(l1, l2, l3)], Y[l2])
        G = torch.einsum("eca,eab->ecb", htj[l1], Mp)
        v[l3] = v[l3] + w[:, p, :, None] * G
    a = (q[row] * v[0][:, :, 0]).view(E, Hh, dh).sum(-1) / math.sqrt(dh)
    with torch.no_grad():
        M = torch.full((n_atoms, Hh), -math.inf, dtype=torch.float64)
        M = M.scatter_reduce(0, row[:, None].expand(E, Hh), a, reduce="amax", include_self=True)
        M = torch.where(torch.isfinite(M), M, torch.zeros_like(M))
    ue = u[:, None] * torch.exp(a - M[row])
    Z = torch.zeros(n_atoms, Hh, dtype=torch.float64).index_add(0, row, ue)
    Zr = Z[row]
    alpha = torch.where(Zr > 0, ue / torch.where(Zr > 0, Zr, torch.ones_like(Zr)), torch.zeros_like(ue))
    ac = alpha[:, head]
    return [torch.zeros(n_atoms, C, 2 * l + 1, dtype=torch.float64).index_add(0, row, ac[:, :, None] * v[l])
            for l in range(L + 1)]


def _update(cfg, lw, h, m):
    """Step 7: gated residual update."""
    C, L = cfg.channels, cfg.lmax
    out = [h[0] + F.silu(torch.einsum("oc,ncm->nom", lw["wo"][0], m[0]))]
    if L >= 1:
        gamma = torch.sigmoid(m[0][:, :, 0] @ lw["wg"].T)
        for l in range(1, L + 1):
            g = gamma[:, (l - 1) * C:l * C]
            out.append(h[l] + g[:, :, None] * torch.einsum("oc,ncm->nom", lw["wo"][l], m[l]))
    return out


def layer(cfg, lw, h, r, rhat, row, col, n_atoms, cgs):
    """One attention layer.  h: list over l of [N, C, 2l+1]; returns new list."""
    ht = [torch.einsum("oc,ncm->nom", lw["wv"][l], h[l]) for l in range(cfg.lmax + 1)]
    q = h[0][:, :, 0] @ lw["wq"].T
    return _update(cfg, lw, h, _messages(cfg, lw, ht, q, r, rhat, row, col, n_atoms, cgs))


def _row_chunks(row, n_atoms, max_edges):
    """(a0, a1, e0, e1): receivers a0..a1-1 own edges e0..e1-1 of the ascending row
    array; whole rows, about max_edges edges per chunk (a longer row is one chunk)."""
    starts = np.searchsorted(np.asarray(row), np.arange(n_atoms + 1))
    a0 = 0
    while a0 < n_atoms:
        a1 = int(np.searchsorted(starts, starts[a0] + max_edges, side="right")) - 1
        a1 = min(max(a1, a0 + 1), n_atoms)
        yield a0, a1, int(starts[a0]), int(starts[a1])
        a0 = a1


def _chunk_messages(cfg, lw, htj, q_rows, d, rr, n_rows, cgs):
    """Messages of one chunk of whole rows from its gathered inputs: htj (sender
    features per edge), q_rows (the rows' queries), d (edge vectors), rr (row - a0)."""
    r = torch.linalg.norm(d, dim=1)
    return _messages(cfg, lw, htj, q_rows, r, d / r[:, None], rr, torch.arange(d.shape[0]), n_rows, cgs)


def _edge_vectors(X, L, row, col):
    d = X[col] - X[row]
    if L is not None:
        d = d - L * torch.round(d / L)
    return d


def _messages_chunked(cfg, lw, ht, q, X, L, row, col, n_atoms, cgs, chunks):
    """m for every atom, chunk by chunk (no gradients)."""
    parts = []
    for a0, a1, e0, e1 in chunks:
        if e1 == e0:
            parts.append([torch.zeros(a1 - a0, cfg.channels, 2 * l + 1, dtype=torch.float64)
                          for l in range(cfg.lmax + 1)])
            continue
        rr, cc = row[e0:e1], col[e0:e1]
        d = _edge_vectors(X, L, rr, cc)
        parts.append(_chunk_messages(cfg, lw, [x[cc] for x in ht], q[a0:a1], d, rr - a0, a1 - a0, cgs))
    return [torch.cat([p[l] for p in parts]) for l in range(cfg.lmax + 1)]


def layer_chunked(cfg, lw, h, X, L, row, col, n_atoms, cgs, max_edges=1024, with_messages=False):
    """`layer` without gradients, evaluated over chunks of whole receiver rows (the
    softmax of a row reads only that row's edges, so each chunk computes its rows
    exactly as the whole layer does).  row must be ascending.  with_messages: also
    return the messages m."""
    with torch.no_grad():
        ht = [torch.einsum("oc,ncm->nom", lw["wv"][l], h[l]) for l in range(cfg.lmax + 1)]
        q = h[0][:, :, 0] @ lw["wq"].T
        parts = []
        m = _messages_chunked(cfg, lw, ht, q, X, L, row, col, n_atoms, cgs, _row_chunks(row, n_atoms, max_edges))
        out = _update(cfg, lw, h, m)
        return (out, m) if with_messages else out


def _layer_vjp(cfg, lw, h, m, X, L, row, col, n_atoms, cgs, g_out, max_edges=1024):
    """Reverse step of one layer with input h and messages m: g_out = dE/d(layer
    output) -> (dE/dh, dE/dX).  The
    chain rule taken in three local pieces, each by autograd: the gated update (all
    atoms), the messages of each chunk of whole rows with respect to that chunk's
    own gathered inputs (sender features, queries, edge vectors; their gradients are
    scattered back with index_add), and the per-atom products W_v h, W_q h^0."""
    Lm = cfg.lmax
    h = [x.detach().requires_grad_() for x in h]
    ht = [torch.einsum("oc,ncm->nom", lw["wv"][l], h[l]) for l in range(Lm + 1)]
    q = h[0][:, :, 0] @ lw["wq"].T
    htd, qd = [x.detach() for x in ht], q.detach()
    chunks = list(_row_chunks(row, n_atoms, max_edges))
    m = [x.detach().requires_grad_() for x in m]
    out = _update(cfg, lw, h, m)
    g = torch.autograd.grad(out, h + m, grad_outputs=g_out)
    g_h, g_m = list(g[:Lm + 1]), g[Lm + 1:]
    g_ht = [torch.zeros_like(x) for x in htd]
    g_q = torch.zeros_like(qd)
    g_X = torch.zeros_like(X)
    for a0, a1, e0, e1 in chunks:
        if e1 == e0:
            continue  # rows without edges: their messages are zero
        rr, cc = row[e0:e1], col[e0:e1]
        d = _edge_vectors(X, L, rr, cc).requires_grad_()
        htj = [x[cc].requires_grad_() for x in htd]
        qr = qd[a0:a1].requires_grad_()
        mc = _chunk_messages(cfg, lw, htj, qr, d, rr - a0, a1 - a0, cgs)
        gs = torch.autograd.grad(mc, [d, qr] + htj, grad_outputs=[x[a0:a1] for x in g_m], allow_unused=True)
        g_X.index_add_(0, cc, gs[0])
        g_X.index_add_(0, rr, -gs[0])
        g_q[a0:a1] += gs[1]
        for l in range(Lm + 1):
            if gs[2 + l] is not None:
                g_ht[l].index_add_(0, cc, gs[2 + l])
    g2 = torch.autograd.grad(ht + [q], h, grad_outputs=g_ht + [g_q])
    return [a + b for a, b in zip(g_h, g2)], g_X


def energy_forces_chunked(cfg, prm, cgs, X, species, L, row, col, keep=None, read=None, max_edges=1024):
    """E = sum of E_i over the atoms listed in `read` (all if None) after T layers,
    layer t applied to the edges whose receiver is marked in keep[t] (all if None),
    and F = -dE/dX: the layers forward over chunks of rows (`layer_chunked`), then one
    reverse sweep layer by layer (`_layer_vjp`).  The same definition as `energy`
    (pinned against it), with memory bounded by a chunk.  row ascending."""
    T = cfg.layers
    n = X.shape[0]
    X = X.detach()
    h = embed(cfg, prm, species)
    ins, msgs, rows = [], [], []
    for t in range(T):
        e = torch.ones_like(row, dtype=torch.bool) if keep is None else keep[t][row]
        rows.append((row[e], col[e]))
        ins.append(h)
        h, m = layer_chunked(cfg, prm.layers[t], h, X, L, row[e], col[e], n, cgs, max_edges, with_messages=True)
        msgs.append(m)
    h0 = h[0].detach().requires_grad_()
    Ea = readout(prm, h0)
    Es = Ea.sum() if read is None else Ea[torch.as_tensor(read)].sum()
    (g0,) = torch.autograd.grad(Es, h0)
    g = [g0] + [torch.zeros_like(x) for x in h[1:]]
    F = torch.zeros_like(X)
    for t in range(T - 1, -1, -1):
        g, gX = _layer_vjp(cfg, prm.layers[t], ins[t], msgs[t], X, L, rows[t][0], rows[t][1], n, cgs, g, max_edges)
        F -= gX
    return float(Es.detach()), F.numpy()


def embed(cfg, prm, species):
    sp = torch.as_tensor(np.asarray(species, np.int64))
    n = sp.shape[0]
    h = [prm.emb[sp][:, :, None].clone()]
    for l in range(1, cfg.lmax + 1):
        h.append(torch.zeros(n, cfg.channels, 2 * l + 1, dtype=torch.float64))
    return h


def readout(prm, h0):
    return (F.silu(h0[:, :, 0] @ prm.wr.T) * prm.wout[0]).sum(1)


def _active_edges(P, L, row_ptr, col, r_cut):
    row = csr_rows(row_ptr)
    colt = torch.as_tensor(np.asarray(col, np.int64))
    r, _ = edge_geometry(P.detach(), L, row, colt)
    keep = r < r_cut
    return row[keep], colt[keep]


def energy(cfg, weights, pos, species, L, row_ptr, col, forces=True, keep_features=False):
    """Returns dict(E, E_atoms, F?, h?).  pos: [N,3] (float32 or float64) in the CSR's slot order."""
    prm = Params(cfg, weights)
    cgs = cg_table(cfg.lmax)
    Ld = None if L is None else float(np.float32(L))
    P = torch.tensor(_as_f64(pos), requires_grad=forces)
    n = P.shape[0]
    row, colt = _active_edges(P, Ld, row_ptr, col, cfg.cutoff)
    r, rhat = edge_geometry(P, Ld, row, colt)
    h = embed(cfg, prm, species)
    feats = []
    for t in range(cfg.layers):
        h = layer(cfg, prm.layers[t], h, r, rhat, row, colt, n, cgs)
        if keep_features:
            feats.append([x.detach().clone() for x in h])
    Ea = readout(prm, h[0])
    E = Ea.sum()
    out = {"E": float(E.detach()), "E_atoms": Ea.detach().numpy(), "n_active": int(row.numel())}
    if forces:
        (g,) = torch.autograd.grad(E, P)
        out["F"] = (-g).numpy()
    if keep_features:
        out["h"] = [to_flat(x) for x in feats]
    return out


def energy_heads(cfg, weights, head_wr, head_wout, lam, pos, species, L, row_ptr, col, forces=True):
    """Several readout heads on one encoder ("Exascale Multi-Task Graph Foundation Models",
    Fig. 5: the encoder runs once, every head reads its output, the heads' energies form a
    weighted sum and one backward pass gives the forces).  Head k replaces the readout
    (W_r, w_out) of the blob by head_wr[k] [C][C] (out, in) and head_wout[k] [C]:

      E_k = sum_i sum_c w_out^k[c] SiLU((W_r^k h_i^0)[c]),   E = sum_k lam_k E_k,   F = -dE/dx

    Returns dict(E_heads [R], E, E_atoms [R][N], F?).  The blob's own readout is unused."""
    prm = Params(cfg, weights)
    cgs = cg_table(cfg.lmax)
    Ld = None if L is None else float(np.float32(L))
    P = torch.tensor(_as_f64(pos), requires_grad=forces)
    n = P.shape[0]
    row, colt = _active_edges(P, Ld, row_ptr, col, cfg.cutoff)
    r, rhat = edge_geometry(P, Ld, row, colt)
    h = embed(cfg, prm, species)
    for t in range(cfg.layers):
        h = layer(cfg, prm.layers[t], h, r, rhat, row, colt, n, cgs)
    wr = torch.as_tensor(np.asarray(head_wr, np.float32).astype(np.float64))
    wo = torch.as_tensor(np.asarray(head_wout, np.float32).astype(np.float64))
    lam_d = [float(np.float32(x)) for x in np.asarray(lam).ravel()]
    Ea = torch.stack([(F.silu(h[0][:, :, 0] @ wr[k].T) * wo[k]).sum(1) for k in range(len(lam_d))])
    Ek = Ea.sum(1)
    E = sum(lam_d[k] * Ek[k] for k in range(len(lam_d)))
    out = {"E_heads": Ek.detach().numpy(), "E": float(E.detach()), "E_atoms": Ea.detach().numpy()}
    if forces:
        (g,) = torch.autograd.grad(E, P)
        out["F"] = (-g).numpy()
    return out


def to_flat(h):
    """list over l of [N, C, 2l+1] -> numpy [N, K, C] with k = l^2 + m + l."""
    return torch.cat([x.permute(0, 2, 1) for x in h], dim=1).numpy()


def from_flat(hf, lmax):
    hf = torch.as_tensor(np.asarray(hf, np.float64))
    out, k = [], 0
    for l in range(lmax + 1):
        out.append(hf[:, k:k + 2 * l + 1, :].permute(0, 2, 1).contiguous())
        k += 2 * l + 1
    return out


def layer_forward(cfg, weights, t, h_in_flat, pos, L, row_ptr, col):
    """One layer t (0-based) on given input features [N, K, C] -> [N, K, C]."""
    prm = Params(cfg, weights)
    cgs = cg_table(cfg.lmax)
    Ld = None if L is None else float(np.float32(L))
    with torch.no_grad():
        P = torch.tensor(_as_f64(pos))
        row, colt = _active_edges(P, Ld, row_ptr, col, cfg.cutoff)
        r, rhat = edge_geometry(P, Ld, row, colt)
        h = from_flat(h_in_flat, cfg.lmax)
        return to_flat(layer(cfg, prm.layers[t], h, r, rhat, row, colt, P.shape[0], cgs))


def embed_flat(cfg, weights, species):
    prm = Params(cfg, weights)
    with torch.no_grad():
        return to_flat(embed(cfg, prm, species))


def atom_energy_local(cfg, weights, pos, species, L, k, margin=0.5):
    """E_k of atom k in the periodic box, evaluated on k's receptive field only.

    By the locality of message passing ("Ab Initio Accuracy Beyond the Cutoff",
    Abstract: T stacked layers carry information T cutoffs far), E_k depends only
    on atoms joined to k by chains of at most T edges with r < r_cut, all within
    T * r_cut of k.  The atoms within T * r_cut + margin of k are taken as an open
    cluster (minimum-image displacements about k; requires T * r_cut + margin <
    L / 2).  Layer t (0-based) is applied only to receivers within
    (T - 1 - t) * r_cut + margin of k, whose inputs (neighbours within one more
    cutoff) were all produced by layer t - 1 or by the embedding; the features of
    other atoms are never read afterwards.  The arithmetic is that of `layer`.
    Pinned against energy()["E_atoms"] on boxes where both apply.
    """
    T, rc = cfg.layers, cfg.cutoff
    Ld = float(np.float32(L))
    P = _as_f64(pos)
    d = P - P[k]
    d = d - Ld * np.round(d / Ld)
    dist = np.linalg.norm(d, axis=1)
    R = T * rc + margin
    if not R < Ld / 2:
        raise ValueError("receptive field does not fit in the box")
    sel = np.nonzero(dist < R)[0]
    X = d[sel]
    dc = dist[sel]
    n = sel.size
    # every ordered pair (a <- b), a != b, with |x_b - x_a| < r_cut (brute force)
    rows, cols = [], []
    for a0 in range(0, n, 1024):
        blk = X[a0:a0 + 1024]
        r2 = ((X[None, :, :] - blk[:, None, :]) ** 2).sum(-1)
        a, b = np.nonzero(r2 < rc * rc)
        a = a + a0
        keep = a != b
        rows.append(a[keep])
        cols.append(b[keep])
    row = torch.as_tensor(np.concatenate(rows).astype(np.int64))
    col = torch.as_tensor(np.concatenate(cols).astype(np.int64))
    prm = Params(cfg, weights)
    cgs = cg_table(cfg.lmax)
    with torch.no_grad():
        Xt = torch.tensor(X)
        r, rhat = edge_geometry(Xt, None, row, col)
        act = r < rc
        row, col, r, rhat = row[act], col[act], r[act], rhat[act]
        h = embed(cfg, prm, np.asarray(species)[sel])
        dct = torch.tensor(dc)
        for t in range(T):
            need = dct < (T - 1 - t) * rc + margin
            e = need[row]
            h = layer(cfg, prm.layers[t], h, r[e], rhat[e], row[e], col[e], n, cgs)
        kk = int(np.nonzero(sel == k)[0][0])
        return float(readout(prm, h[0][kk:kk + 1])[0])


def forces_local(cfg, weights, pos, species, L, center, delta=2.0, max_edges=1024):
    """Exact forces on the atoms within delta of atom `center` of the periodic box,
    from an open cluster around it.

    By locality ("Ab Initio Accuracy Beyond the Cutoff", Abstract: T stacked layers
    reach T cutoffs, and forces back-propagate through the same layers), the force
    on atom k, F_k = -d/dx_k sum_i E_i, involves only the E_i of atoms within
    T * r_cut of k, and each of those only atoms within T * r_cut of i.  For the
    atoms k within delta of the centre it is therefore the gradient of
    sum_{i: |x_i - x_c| < T r_cut + delta} E_i over the open cluster of radius
    2 T r_cut + delta about the centre (minimum-image displacements), with layer t
    (0-based) applied to receivers within (2T - 1 - t) r_cut + delta -- whose inputs
    are all exact -- evaluated over chunks of whole rows (`energy_forces_chunked`).  Pair candidates come
    from a k-d tree (a library radius search); the pair is kept when the float64
    distance is < r_cut.  Requires 2 (2 T r_cut + delta) < L - r_cut, so that no
    two cluster atoms meet through another image.  Pinned against the forces of
    `energy` on whole boxes.

    Returns (idx int64 [m]: indices into pos of the atoms within delta of the
    centre, ascending; F float64 [m][3])."""
    from scipy.spatial import cKDTree
    T, rc = cfg.layers, cfg.cutoff
    Ld = float(np.float32(L))
    P = _as_f64(pos)
    d = P - P[center]
    d = d - Ld * np.round(d / Ld)
    dist = np.linalg.norm(d, axis=1)
    R = 2 * T * rc + delta
    if not (R < Ld / 2 and 2 * R < Ld - rc):
        raise ValueError("force cluster does not fit in the box")
    sel = np.nonzero(dist < R)[0]
    X0 = d[sel]
    dc = dist[sel]
    n = sel.size
    pr = cKDTree(X0).query_pairs(rc * (1 + 1e-9), output_type="ndarray").astype(np.int64)
    a = np.concatenate([pr[:, 0], pr[:, 1]])
    b = np.concatenate([pr[:, 1], pr[:, 0]])
    order = np.lexsort((b, a))
    a, b = a[order], b[order]
    r = np.linalg.norm(X0[b] - X0[a], axis=1)
    keep = r < rc
    row = torch.as_tensor(a[keep])
    col = torch.as_tensor(b[keep])
    prm = Params(cfg, weights)
    cgs = cg_table(cfg.lmax)
    dct = torch.tensor(dc)
    keep = [dct < (2 * T - 1 - t) * rc + delta for t in range(T)]
    _, Fc = energy_forces_chunked(cfg, prm, cgs, torch.tensor(X0), np.asarray(species)[sel], None, row, col,
                                  keep=keep, read=np.nonzero(dc < T * rc + delta)[0], max_edges=max_edges)
    k = np.nonzero(dc < delta)[0]
    return sel[k].astype(np.int64), Fc[k]
