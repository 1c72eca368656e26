"""Writes attention_layer_5atom.json: one attention layer on a five-atom open
cluster, evaluated here from the layer's definition without oracle/ or the
library:  python tests/golden/make_attention_golden.py

Independent routes to every ingredient:
  * Clebsch-Gordan: sympy's complex coefficients <l1 m1 l2 m2 | l3 m3>
    (Condon-Shortley), turned into the real basis by the unitary change of
    basis of the real harmonics, then scaled to sum_{m1 m2} C C' = delta and
    signed so the first nonzero entry in (m1, m2, m3) order is positive.  Each
    tensor is checked for equivariance (a rotation-invariant triple product).
  * Real harmonics: scipy's complex ones through the real-form relation
    Y_{l,m} = sqrt2 (-1)^m Re Y_l^m (m > 0), Y_l^0 (m = 0),
    sqrt2 (-1)^|m| Im Y_l^|m| (m < 0); order m = -l..l.
  * Radial basis and envelope: closed forms (the envelope in its expanded
    polynomial 1 - 28 d^6 + 48 d^7 - 21 d^8).
  * The layer: plain scalar loops over atoms, edges, channels and components.

The layer (equivariant message-passing attention: "Ab Initio Accuracy Beyond
the Cutoff", Abstract; tensor-product coupling through Clebsch-Gordan
coefficients: "Unlocking Tensor Core Performance", section "Why MLIPs Need
Dedicated Performance Optimization"), with the conventions this fixture pins:
  ht_j^l = W_v^l h_j^l,  q_i = W_q h_i^0
  w_e[p, c] = u(r) sum_k W_2[p C + c][k] SiLU(sum_n W_1[k][n] B_n(r))
  v_e^{l3}[c, m3] = sum_{p = (l1, l2, l3)} w_e[p, c] sum_{m1, m2} CG_p[m1, m2, m3]
                    ht_j^{l1}[c, m1] Y_{l2 m2}(rhat)      (first CG index: the
                    sender's features; second: the harmonic of the edge)
  a_e^k = (sum over the contiguous head k = {k d_h .. (k+1) d_h - 1} of
           q_i[c] v_e^0[c]) / sqrt(d_h)
  alpha_e^k = u(r_e) exp(a_e^k) / sum_{e' in row i} u(r_e') exp(a_e'^k)
  m_i^l[c] = sum_e alpha_e^{c // d_h} v_e^l[c]
  h_i^0 += SiLU(W_o^0 m_i^0);  h_i^l += sigmoid(W_g m_i^0)[(l-1) C + c] (W_o^l m_i^l)[c]
with edge e = (i <- j) for |x_j - x_i| < r_c, rhat = (x_j - x_i) / r.
"""
import json
import math
import os

import numpy as np
from scipy.special import sph_harm_y
from sympy import S
from sympy.physics.wigner import clebsch_gordan

HERE = os.path.dirname(os.path.abspath(__file__))

LMAX, C, H, NB, HR, RC = 2, 4, 2, 8, 6, 4.0
POS = [[0.0, 0.0, 0.0], [1.9, 0.4, -0.7], [-0.6, 2.1, 1.3], [2.8, 2.9, 0.5], [-3.5, -3.0, 2.0]]


def paths():
    return [(a, b, c) for a in range(LMAX + 1) for b in range(LMAX + 1) for c in range(LMAX + 1)
            if abs(a - b) <= c <= a + b]


def complex_sh(l, v):
    x, y, z = v
    theta, phi = math.acos(max(-1.0, min(1.0, z))), math.atan2(y, x)
    return np.array([complex(sph_harm_y(l, m, theta, phi)) for m in range(-l, l + 1)])


def real_sh(l, v):
    x, y, z = v
    theta, phi = math.acos(max(-1.0, min(1.0, z))), math.atan2(y, x)
    out = []
    for m in range(-l, l + 1):
        c = complex(sph_harm_y(l, abs(m), theta, phi))
        if m > 0:
            out.append(math.sqrt(2) * (-1) ** m * c.real)
        elif m == 0:
            out.append(c.real)
        else:
            out.append(math.sqrt(2) * (-1) ** abs(m) * c.imag)
    return np.array(out)


def real_basis_matrix(l):
    """U with real_sh(l) = U complex_sh(l) (rows m = -l..l, columns mu = -l..l)."""
    U = np.zeros((2 * l + 1, 2 * l + 1), complex)
    U[l, l] = 1.0
    for a in range(1, l + 1):
        s = (-1) ** a
        U[l + a, l + a] = s / math.sqrt(2)     # m = +a
        U[l + a, l - a] = 1 / math.sqrt(2)
        U[l - a, l + a] = -1j * s / math.sqrt(2)  # m = -a
        U[l - a, l - a] = 1j / math.sqrt(2)
    return U


def real_cg(l1, l2, l3):
    T = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                T[m1 + l1, m2 + l2, m3 + l3] = float(clebsch_gordan(S(l1), S(l2), S(l3), S(m1), S(m2), S(m3)))
    U1, U2, U3 = real_basis_matrix(l1), real_basis_matrix(l2), real_basis_matrix(l3)
    Cr = np.einsum("ai,bj,ck,ijk->abc", U1.conj(), U2.conj(), U3, T)
    big = Cr.ravel()[np.argmax(np.abs(Cr.ravel()))]
    Cr = Cr / (big / abs(big))
    assert np.abs(Cr.imag).max() < 1e-12
    Cr = Cr.real
    Cr = Cr / math.sqrt((Cr * Cr).sum()) * math.sqrt(2 * l3 + 1)
    flat = Cr.ravel()
    Cr = Cr * np.sign(flat[np.nonzero(np.abs(flat) > 1e-9)[0][0]])
    Cr[np.abs(Cr) < 1e-14] = 0.0
    return Cr


def _rot(rng):
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
                     [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
                     [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)]])


def check_tables(cgs):
    rng = np.random.default_rng(11)
    for l in range(LMAX + 1):
        v = rng.standard_normal(3)
        v /= np.linalg.norm(v)
        assert np.abs(real_basis_matrix(l) @ complex_sh(l, v) - real_sh(l, v)).max() < 1e-12
    for (l1, l2, l3), Cp in cgs.items():
        for _ in range(3):
            vs = [x / np.linalg.norm(x) for x in rng.standard_normal((3, 3))]
            Q = _rot(rng)
            inv = lambda a, b, c: np.einsum("abc,a,b,c->", Cp, real_sh(l1, a), real_sh(l2, b), real_sh(l3, c))
            assert abs(inv(*vs) - inv(*(Q @ x for x in vs))) < 1e-12, (l1, l2, l3)


def silu(x):
    return x / (1.0 + math.exp(-x))


def sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


def layer(pos, h, W, cgs):
    """h[i][l] [C][2l+1] lists; returns (h_out, alphas) with alphas[(i, j)] = [H]."""
    n, dh = len(pos), C // H
    P = paths()
    ht = [[[[sum(W["wv%d" % l][c][cc] * h[i][l][cc][m] for cc in range(C)) for m in range(2 * l + 1)]
            for c in range(C)] for l in range(LMAX + 1)] for i in range(n)]
    q = [[sum(W["wq"][c][cc] * h[i][0][cc][0] for cc in range(C)) for c in range(C)] for i in range(n)]
    h_out, alphas = [], {}
    for i in range(n):
        edges = []
        for j in range(n):
            if j == i:
                continue
            d = [pos[j][a] - pos[i][a] for a in range(3)]
            r = math.sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2])
            if not r < RC:
                continue
            rhat = [x / r for x in d]
            x = r / RC
            u = 1 - 28 * x ** 6 + 48 * x ** 7 - 21 * x ** 8
            B = [math.sqrt(2 / RC) * math.sin(k * math.pi * r / RC) / r for k in range(1, NB + 1)]
            hid = [silu(sum(W["w1"][k][nn] * B[nn] for nn in range(NB))) for k in range(HR)]
            w = [[u * sum(W["w2"][p * C + c][k] * hid[k] for k in range(HR)) for c in range(C)]
                 for p in range(len(P))]
            Y = [real_sh(l, rhat) for l in range(LMAX + 1)]
            v = [[[0.0] * (2 * l + 1) for _ in range(C)] for l in range(LMAX + 1)]
            for p, (l1, l2, l3) in enumerate(P):
                Cp = cgs[(l1, l2, l3)]
                for c in range(C):
                    for m3 in range(2 * l3 + 1):
                        s = 0.0
                        for m1 in range(2 * l1 + 1):
                            for m2 in range(2 * l2 + 1):
                                s += Cp[m1, m2, m3] * ht[j][l1][c][m1] * Y[l2][m2]
                        v[l3][c][m3] += w[p][c] * s
            a = [sum(q[i][c] * v[0][c][0] for c in range(k * dh, (k + 1) * dh)) / math.sqrt(dh) for k in range(H)]
            edges.append((j, u, a, v))
        msg = [[[0.0] * (2 * l + 1) for _ in range(C)] for l in range(LMAX + 1)]
        if edges:
            for k in range(H):
                top = max(e[2][k] for e in edges)
                Z = sum(e[1] * math.exp(e[2][k] - top) for e in edges)
                for j, u, a, v in edges:
                    alpha = u * math.exp(a[k] - top) / Z
                    alphas.setdefault((i, j), [0.0] * H)[k] = alpha
                    for c in range(k * dh, (k + 1) * dh):
                        for l in range(LMAX + 1):
                            for m in range(2 * l + 1):
                                msg[l][c][m] += alpha * v[l][c][m]
        out = [[[h[i][0][c][0] + silu(sum(W["wo0"][c][cc] * msg[0][cc][0] for cc in range(C)))]
                for c in range(C)]]
        gam = [sigmoid(sum(W["wg"][g][cc] * msg[0][cc][0] for cc in range(C))) for g in range(LMAX * C)]
        for l in range(1, LMAX + 1):
            out.append([[h[i][l][c][m] + gam[(l - 1) * C + c] *
                         sum(W["wo%d" % l][c][cc] * msg[l][cc][m] for cc in range(C))
                         for m in range(2 * l + 1)] for c in range(C)])
        h_out.append(out)
    return h_out, alphas


def main():
    cgs = {p: real_cg(*p) for p in paths()}
    check_tables(cgs)
    rng = np.random.default_rng(20261203)
    f32 = lambda a: np.asarray(a, np.float32).astype(np.float64)
    W = {"w1": f32(rng.standard_normal((HR, NB)) / math.sqrt(NB)),
         "w2": f32(rng.standard_normal((len(paths()) * C, HR)) / math.sqrt(HR)),
         # a larger query scale, so that the attention logits of a row differ by O(1)
         "wq": f32(25.0 * rng.standard_normal((C, C)) / math.sqrt(C))}
    for l in range(LMAX + 1):
        W["wv%d" % l] = f32(rng.standard_normal((C, C)) / math.sqrt(C))
    for l in range(LMAX + 1):
        W["wo%d" % l] = f32(rng.standard_normal((C, C)) / math.sqrt(C))
    W["wg"] = f32(rng.standard_normal((LMAX * C, C)) / math.sqrt(C))
    n = len(POS)
    h = [[rng.standard_normal((C, 2 * l + 1)) for l in range(LMAX + 1)] for _ in range(n)]
    h_out, alphas = layer(POS, [[x.tolist() for x in hi] for hi in h], {k: v.tolist() for k, v in W.items()}, cgs)
    # [atom][k = l^2 + m + l][channel]
    flat = lambda hh: [[[hh[i][l][c][m] for c in range(C)] for l in range(LMAX + 1) for m in range(2 * l + 1)]
                       for i in range(n)]
    doc = {
        "what": "one attention layer on a five-atom open cluster, evaluated by make_attention_golden.py from the "
                "layer definition in its header (sympy Clebsch-Gordan, scipy harmonics, scalar loops); "
                "no oracle or library code",
        "config": {"lmax": LMAX, "channels": C, "heads": H, "n_bessel": NB, "radial_hidden": HR, "cutoff": RC},
        "pos": POS,
        "weights": {k: v.tolist() for k, v in W.items()},
        "h_in": flat([[x.tolist() for x in hi] for hi in h]),
        "h_out": flat(h_out),
        "alpha": [[i, j, *a] for (i, j), a in sorted(alphas.items())],
    }
    with open(os.path.join(HERE, "attention_layer_5atom.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
