"""Real Clebsch-Gordan intertwiners (oracle).

"Unlocking Tensor Core Performance" (section "Why MLIPs Need Dedicated
Performance Optimization", on equivariant networks) couples angular-momentum
channels through Clebsch-Gordan coefficients.  For the real harmonics of
``basis.real_sh`` the coupling l1 x l2 -> l3 is the (one-dimensional) space of
real tensors C[m1, m2, m3] left unchanged by D^l1(Q) x D^l2(Q) x D^l3(Q) for
every rotation Q, where D^l(Q) is the real Wigner matrix with
Y_l(Q r) = D^l(Q) Y_l(r).

Construction here (no Racah formula): D^l(Q) is recovered from the harmonics
themselves by least squares on sample directions; the invariant tensor is the
null vector of the stacked (D1 x D2 x D3 - I) for a few rotations.

Conventions: paths are all triples (l1, l2, l3), 0 <= l <= lmax, with
|l1 - l2| <= l3 <= l1 + l2, in lexicographic order (no parity filter).  Each
tensor is scaled so that sum_{m1,m2} C[m1,m2,m3] C[m1,m2,m3'] = delta, and its
first nonzero entry in lexicographic (m1, m2, m3) order is positive.
"""
import functools

import numpy as np
import torch

from .basis import real_sh


def paths(lmax):
    return [(a, b, c) for a in range(lmax + 1) for b in range(lmax + 1) for c in range(lmax + 1)
            if abs(a - b) <= c <= a + b]


def _rotation(rng):
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
                     [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
                     [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)]])


def wigner_real(l, Q, n_pts=64, seed=0):
    """Real D^l(Q) with Y_l(Q r) = D^l(Q) Y_l(r), by least squares over sample directions."""
    rng = np.random.default_rng(seed)
    p = rng.standard_normal((n_pts, 3))
    p /= np.linalg.norm(p, axis=1, keepdims=True)
    P = torch.tensor(p, dtype=torch.float64)
    Qp = P @ torch.tensor(Q, dtype=torch.float64).T
    Yp = real_sh(P, l)[l].numpy()
    Yq = real_sh(Qp, l)[l].numpy()
    DT, *_ = np.linalg.lstsq(Yp, Yq, rcond=None)
    return DT.T


def _fix(c):
    c = c / np.sqrt((c * c).sum()) * np.sqrt(c.shape[2])
    flat = c.ravel()
    first = flat[np.nonzero(np.abs(flat) > 1e-9)[0][0]]
    c = c * np.sign(first)
    c[np.abs(c) < 1e-13] = 0.0
    return c


@functools.lru_cache(maxsize=None)
def real_cg(l1, l2, l3):
    """C [2l1+1, 2l2+1, 2l3+1] float64."""
    rng = np.random.default_rng(1234 + 100 * l1 + 10 * l2 + l3)
    n1, n2, n3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
    rows = []
    for _ in range(3):
        Q = _rotation(rng)
        D = np.kron(np.kron(wigner_real(l1, Q), wigner_real(l2, Q)), wigner_real(l3, Q))
        rows.append(D - np.eye(n1 * n2 * n3))
    A = np.concatenate(rows)
    _, s, vt = np.linalg.svd(A)
    if not (s[-1] < 1e-9 and (s.size < 2 or s[-2] > 1e-3)):
        raise RuntimeError(f"no unique intertwiner for {(l1, l2, l3)}: {s[-3:]}")
    return _fix(vt[-1].reshape(n1, n2, n3))


def cg_table(lmax):
    """dict path -> torch float64 tensor, in path order."""
    return {p: torch.tensor(real_cg(*p)) for p in paths(lmax)}
