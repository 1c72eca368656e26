"""Wrap, Hilbert sort and the skin-padded radius graph (oracle).

"Ab Initio Accuracy Beyond the Cutoff" (Abstract): atoms are sorted along a
space-filling curve, and a conservative neighbour skin keeps the graph's
topology valid between rebuilds.  The list therefore holds every ordered pair
closer than R = r_cut + skin.  To make the list reproducible bit for bit on
CPU and GPU, the whole decision is stated in float64 with a fixed operation
order (no fused multiply-add):

  wrap      w = x - L*floor(x/L), then one conditional +L / -L fix-up each way;
            stored as float32, and a float32 value equal to L becomes 0.
  order     stable sort by (Hilbert key, input index); slot s holds input atom perm[s].
            For the curve comparison of the abstract, the Morton key or no sort at all
            (input order) may replace the Hilbert key; the rest is unchanged.
  pair test d_a = P_t,a - P_s,a, shifted once by -L or +L when |d_a| > L/2;
            D = (dx*dx + dy*dy) + dz*dz; pair iff D < (r_cut + skin)^2.
  CSR       full directed list without self pairs; each row ascending; int32.
  rev[e]    position of the reverse pair (t -> s) of e = (s -> t).

The cell list below only proposes candidates; brute force gives the same list.
"""
import numpy as np

from . import hilbert


def wrap_positions(x, L):
    """float32 [N,3] -> float32 [N,3] in [0, L)."""
    Lf = np.float32(L)
    Ld = float(Lf)
    xd = np.asarray(x, np.float32).astype(np.float64)
    w = xd - Ld * np.floor(xd / Ld)
    w = np.where(w < 0.0, w + Ld, w)
    w = np.where(w >= Ld, w - Ld, w)
    xf = w.astype(np.float32)
    xf = np.where(xf >= Lf, np.float32(0.0), xf)
    return xf.astype(np.float32)


def hilbert_keys(xf, L, bits=hilbert.BITS):
    g = hilbert.quantize(xf, L, bits)
    return hilbert.hilbert_index(g[:, 0], g[:, 1], g[:, 2], bits)


def sort_order(xf, L, bits=hilbert.BITS, order="hilbert"):
    """perm[s] = input index of slot s: stable by (key, input index)."""
    if order == "hilbert":
        keys = hilbert_keys(xf, L, bits)
    elif order == "morton":
        g = hilbert.quantize(xf, L, bits)
        keys = hilbert.morton_index(g[:, 0], g[:, 1], g[:, 2], bits)
    elif order == "input":
        keys = np.zeros(xf.shape[0], np.uint32)
    else:
        raise ValueError(order)
    return np.argsort(keys, kind="stable").astype(np.int32), keys


def _radius2(r_cut, skin):
    R = float(np.float32(r_cut)) + float(np.float32(skin))
    return R * R


def _pair_d2(Pi, Pj, L):
    """float64 squared minimum-image distance with the fixed operation order."""
    d = Pj - Pi
    if L is not None:
        Ld = float(np.float32(L))
        h = 0.5 * Ld
        d = np.where(d > h, d - Ld, np.where(d < -h, d + Ld, d))
    return (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]


def rows_bruteforce(P, L, r_cut, skin, rows):
    """Neighbour rows for the given slots by testing every atom: list of int32 arrays."""
    Pd = np.asarray(P, np.float32).astype(np.float64)
    R2 = _radius2(r_cut, skin)
    out = []
    for s in rows:
        d2 = _pair_d2(Pd[s][None, :], Pd, L)
        m = d2 < R2
        m[s] = False
        out.append(np.nonzero(m)[0].astype(np.int32))
    return out


def _to_csr(n, src, dst):
    order = np.lexsort((dst, src))
    src, dst = src[order], dst[order]
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(src, minlength=n))])
    return row_ptr.astype(np.int32), dst.astype(np.int32)


def csr_bruteforce(P, L, r_cut, skin, chunk=2048):
    """All pairs tested: O(N^2).  Small boxes only."""
    Pd = np.asarray(P, np.float32).astype(np.float64)
    n = Pd.shape[0]
    R2 = _radius2(r_cut, skin)
    src, dst = [], []
    for a in range(0, n, chunk):
        d2 = _pair_d2(Pd[a:a + chunk, None, :], Pd[None, :, :], L)
        m = d2 < R2
        idx = np.arange(a, min(n, a + chunk))
        m[idx - a, idx] = False
        s, t = np.nonzero(m)
        src.append(s + a)
        dst.append(t)
    return _to_csr(n, np.concatenate(src), np.concatenate(dst))


def csr_cells(P, L, r_cut, skin, chunk=16384):
    """Cell list of side >= R proposes candidates from the 27 surrounding cells."""
    Pd = np.asarray(P, np.float32).astype(np.float64)
    n = Pd.shape[0]
    Ld = float(np.float32(L))
    R = float(np.float32(r_cut)) + float(np.float32(skin))
    nc = int(np.floor(Ld / R))
    if nc < 3:
        return csr_bruteforce(P, L, r_cut, skin)
    R2 = _radius2(r_cut, skin)
    c3 = np.minimum((Pd * (nc / Ld)).astype(np.int64), nc - 1)
    cid = (c3[:, 0] * nc + c3[:, 1]) * nc + c3[:, 2]
    order = np.argsort(cid, kind="stable")
    cstart = np.searchsorted(cid[order], np.arange(nc ** 3 + 1))
    offs = np.array([(a, b, c) for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)])
    src, dst = [], []
    for a in range(0, n, chunk):
        s_idx = np.arange(a, min(n, a + chunk))
        for o in offs:
            nb = (c3[s_idx] + o) % nc
            nid = (nb[:, 0] * nc + nb[:, 1]) * nc + nb[:, 2]
            lo, hi = cstart[nid], cstart[nid + 1]
            cnt = hi - lo
            rep_s = np.repeat(s_idx, cnt)
            base = np.repeat(lo - np.concatenate([[0], np.cumsum(cnt)[:-1]]), cnt)
            cand = order[base + np.arange(cnt.sum())]
            d2 = _pair_d2(Pd[rep_s], Pd[cand], L)
            m = (d2 < R2) & (cand != rep_s)
            src.append(rep_s[m])
            dst.append(cand[m])
    return _to_csr(n, np.concatenate(src), np.concatenate(dst))


def reverse_index(row_ptr, col):
    """rev[e] for e = (s -> t): index of (t -> s).  Requires a symmetric list."""
    n = row_ptr.shape[0] - 1
    row = np.repeat(np.arange(n, dtype=np.int64), np.diff(row_ptr))
    key = row * n + col.astype(np.int64)
    rk = col.astype(np.int64) * n + row
    rev = np.searchsorted(key, rk)
    assert np.all(key[rev] == rk), "neighbour list is not symmetric"
    return rev.astype(np.int32)


def build_neighbors(x, L, r_cut, skin, method="auto", order="hilbert"):
    """Full neighbour build: wrap -> Hilbert sort (or `order`) -> CSR -> rev.

    Returns dict(perm, pos_sorted (float32), row_ptr, col, rev, keys)."""
    xf = wrap_positions(x, L)
    perm, keys = sort_order(xf, L, order=order)
    P = xf[perm]
    if method == "brute" or (method == "auto" and P.shape[0] <= 8192):
        row_ptr, col = csr_bruteforce(P, L, r_cut, skin)
    else:
        row_ptr, col = csr_cells(P, L, r_cut, skin)
    rev = reverse_index(row_ptr, col)
    return {"perm": perm, "pos_sorted": P, "row_ptr": row_ptr, "col": col, "rev": rev,
            "keys": keys}


def csr_open_batched(P, struct_ptr, r_cut, skin):
    """Many open structures (no periodic images) concatenated: atom s's neighbours are the atoms
    t != s of its own structure with D = (dx*dx + dy*dy) + dz*dz < (r_cut + skin)^2 in float64
    (the pair test above without the image shift); rows ascending.  Brute force per structure."""
    P = np.asarray(P, np.float32).astype(np.float64)
    R2 = _radius2(r_cut, skin)
    rows = []
    for b in range(len(struct_ptr) - 1):
        a0, a1 = int(struct_ptr[b]), int(struct_ptr[b + 1])
        Q = P[a0:a1]
        d = Q[None, :, :] - Q[:, None, :]
        D = (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]
        for i in range(a1 - a0):
            nb = np.nonzero(D[i] < R2)[0]
            rows.append(a0 + nb[nb != i])
    row_ptr = np.zeros(P.shape[0] + 1, np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return row_ptr.astype(np.int32), col

