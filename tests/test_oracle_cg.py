"""Pins for the oracle's real Clebsch-Gordan tensors (oracle/cg.py).

Checked against what the definition fixes: orthonormality over (m1, m2);
equivariance under a rotation not used in the construction (with D^l taken
from the harmonics); the closed forms 0 x l -> l = I, l x 0 -> l = I,
1 x 1 -> 0 = delta/sqrt(3), 1 x 1 -> 1 = epsilon/sqrt(2) (with the (y, z, x)
order of the l = 1 harmonics the cyclic order is preserved); the sign rule;
and, for even l1 + l2 + l3, proportionality to the real Gaunt integral
int Y_l1m1 Y_l2m2 Y_l3m3 dOmega computed by quadrature, an independent route
to the same invariant tensor.
"""
import numpy as np
import pytest
import torch

from oracle import basis, cg


def test_path_counts():
    assert len(cg.paths(1)) == 5 and len(cg.paths(2)) == 15
    assert cg.paths(1) == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 1, 1)]


@pytest.mark.parametrize("p", cg.paths(2))
def test_orthonormal_and_sign(p):
    c = cg.real_cg(*p)
    n3 = c.shape[2]
    G = np.einsum("abk,abj->kj", c, c)
    assert np.allclose(G, np.eye(n3), atol=1e-12)
    flat = c.ravel()
    assert flat[np.nonzero(np.abs(flat) > 1e-12)[0][0]] > 0


@pytest.mark.parametrize("p", cg.paths(2))
def test_equivariance_fresh_rotation(p):
    l1, l2, l3 = p
    rng = np.random.default_rng(99)
    Q = cg._rotation(rng)
    D = [cg.wigner_real(l, Q, n_pts=40, seed=5) for l in range(3)]
    c = cg.real_cg(*p)
    a = rng.standard_normal(2 * l1 + 1)
    b = rng.standard_normal(2 * l2 + 1)
    lhs = np.einsum("abk,a,b->k", c, D[l1] @ a, D[l2] @ b)
    rhs = D[l3] @ np.einsum("abk,a,b->k", c, a, b)
    assert np.allclose(lhs, rhs, atol=1e-11)


def test_wigner_from_harmonics_is_orthogonal_and_l1_is_rotation():
    Q = cg._rotation(np.random.default_rng(3))
    D1 = cg.wigner_real(1, Q)
    # l=1 harmonics are (y, z, x): D^1 is Q conjugated by that permutation
    Pm = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], float)
    assert np.allclose(D1, Pm @ Q @ Pm.T, atol=1e-12)
    D2 = cg.wigner_real(2, Q)
    assert np.allclose(D2 @ D2.T, np.eye(5), atol=1e-12)


def test_closed_forms():
    for l in range(3):
        assert np.allclose(cg.real_cg(0, l, l)[0], np.eye(2 * l + 1), atol=1e-12)
        assert np.allclose(cg.real_cg(l, 0, l)[:, 0, :], np.eye(2 * l + 1), atol=1e-12)
    assert np.allclose(cg.real_cg(1, 1, 0)[:, :, 0], np.eye(3) / np.sqrt(3), atol=1e-12)
    eps = np.zeros((3, 3, 3))
    for i, j, k in [(0, 1, 2), (1, 2, 0), (2, 0, 1)]:
        eps[i, j, k], eps[j, i, k] = 1, -1
    assert np.allclose(cg.real_cg(1, 1, 1), eps / np.sqrt(2), atol=1e-12)


def test_even_paths_match_gaunt_integrals():
    n = 16
    x, wx = np.polynomial.legendre.leggauss(n)
    phi = np.arange(2 * n) * (np.pi / n)
    ct, ph = np.meshgrid(x, phi, indexing="ij")
    st = np.sqrt(1 - ct ** 2)
    pts = torch.tensor(np.stack([st * np.cos(ph), st * np.sin(ph), ct], -1).reshape(-1, 3))
    w = (wx[:, None] * np.full(2 * n, np.pi / n)[None, :]).ravel()
    Y = [y.numpy() for y in basis.real_sh(pts, 2)]
    for (l1, l2, l3) in cg.paths(2):
        if (l1 + l2 + l3) % 2:
            continue
        g = np.einsum("s,sa,sb,sc->abc", w, Y[l1], Y[l2], Y[l3])
        c = cg.real_cg(l1, l2, l3)
        scale = (g * c).sum() / (c * c).sum()
        assert abs(scale) > 1e-3
        assert np.allclose(g, scale * c, atol=1e-12), (l1, l2, l3)
