"""Pins for the oracle's edge descriptors (oracle/basis.py).

Real spherical harmonics: orthonormality on the sphere (Gauss-Legendre in
cos(theta) x uniform phi quadrature, exact for these polynomial degrees), the
addition theorem sum_m Y_lm(a) Y_lm(b) = (2l+1)/(4 pi) P_l(a.b) with the
textbook Legendre polynomials, and values on the z axis.  Bessel basis:
orthonormality of r*B_n on [0, r_c].  Envelope: equals its expanded form
1 - 28 d^6 + 48 d^7 - 21 d^8, u(0) = 1, and u, u', u'' vanish at r_c.
"""
import math

import numpy as np
import torch

from oracle import basis


def _sphere_quad(n=12):
    x, wx = np.polynomial.legendre.leggauss(n)
    phi = np.arange(2 * n) * (2 * np.pi / (2 * n))
    ct, ph = np.meshgrid(x, phi, indexing="ij")
    st = np.sqrt(1 - ct ** 2)
    pts = np.stack([st * np.cos(ph), st * np.sin(ph), ct], -1).reshape(-1, 3)
    w = (wx[:, None] * np.full(2 * n, 2 * np.pi / (2 * n))[None, :]).ravel()
    return torch.tensor(pts), torch.tensor(w)


def test_sh_orthonormal():
    pts, w = _sphere_quad()
    Y = torch.cat(basis.real_sh(pts, 2), dim=1)
    G = (Y * w[:, None]).T @ Y
    assert torch.allclose(G, torch.eye(9, dtype=torch.float64), atol=1e-12)


def test_sh_addition_theorem():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((50, 3)); a /= np.linalg.norm(a, axis=1, keepdims=True)
    b = rng.standard_normal((50, 3)); b /= np.linalg.norm(b, axis=1, keepdims=True)
    Ya = basis.real_sh(torch.tensor(a), 2)
    Yb = basis.real_sh(torch.tensor(b), 2)
    c = torch.tensor((a * b).sum(1))
    legendre = [torch.ones_like(c), c, 1.5 * c ** 2 - 0.5]
    for l in range(3):
        lhs = (Ya[l] * Yb[l]).sum(1)
        assert torch.allclose(lhs, (2 * l + 1) / (4 * math.pi) * legendre[l], atol=1e-13)


def test_sh_on_axes():
    z = torch.tensor([[0.0, 0.0, 1.0]], dtype=torch.float64)
    Y = basis.real_sh(z, 2)
    for l in range(3):
        expect = torch.zeros(2 * l + 1, dtype=torch.float64)
        expect[l] = math.sqrt((2 * l + 1) / (4 * math.pi))
        assert torch.allclose(Y[l][0], expect, atol=1e-15)
    x = torch.tensor([[1.0, 0.0, 0.0]], dtype=torch.float64)
    Y = basis.real_sh(x, 2)
    assert abs(Y[1][0, 2] - math.sqrt(3 / (4 * math.pi))) < 1e-15      # m=+1 is x
    assert abs(Y[2][0, 4] - 0.25 * math.sqrt(15 / math.pi)) < 1e-15   # x^2 - y^2


def test_bessel_orthonormal():
    rc = 5.0
    x, wx = np.polynomial.legendre.leggauss(200)
    r = torch.tensor(0.5 * rc * (x + 1))
    w = torch.tensor(0.5 * rc * wx)
    B = basis.bessel(r, rc, 8)
    G = (B * (r ** 2 * w)[:, None]).T @ B
    assert torch.allclose(G, torch.eye(8, dtype=torch.float64), atol=1e-10)


def test_envelope_closed_forms():
    rc = 6.0
    r = torch.linspace(0.0, 7.0, 701, dtype=torch.float64)
    u = basis.envelope(r, rc)
    d = r / rc
    expanded = torch.where(d < 1, 1 - 28 * d ** 6 + 48 * d ** 7 - 21 * d ** 8, torch.zeros_like(d))
    assert torch.allclose(u, expanded, atol=1e-13)
    assert float(u[0]) == 1.0
    assert torch.all(u[r >= rc] == 0)
    rr = torch.tensor([rc * (1 - 1e-7)], dtype=torch.float64, requires_grad=True)
    (g1,) = torch.autograd.grad(basis.envelope(rr, rc).sum(), rr, create_graph=True)
    (g2,) = torch.autograd.grad(g1.sum(), rr)
    assert abs(float(g1.detach())) < 1e-10 and abs(float(g2)) < 1e-5
    assert torch.all(torch.diff(u[r < rc]) <= 0), "monotone decreasing on [0, r_c)"
