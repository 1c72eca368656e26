"""Edge descriptors (oracle): real spherical harmonics, Bessel radial basis, envelope.

"Unlocking Tensor Core Performance" (section "Why MLIPs Need Dedicated
Performance Optimization") describes descriptors built from pairwise distances
and combinations of spherical harmonics, evaluated in high precision ("Choosing
a Precision Strategy").  The radial part follows the Bessel basis and the
polynomial envelope named among the hyper-parameters of "Exascale Multi-Task
Graph Foundation Models" (Table IV: Bessel radial basis for MACE, envelope
exponent 4-6 for DimeNet); the exponent used is p = 6.

  Y_lm   orthonormal real spherical harmonics, m = -l..l, flattened k = l^2 + m + l:
         Y00 = 1/(2 sqrt(pi));  (Y1-1, Y10, Y11) = sqrt(3/4pi) (y, z, x);
         Y2-2 = (1/2)sqrt(15/pi) xy, Y2-1 = (1/2)sqrt(15/pi) yz,
         Y20 = (1/4)sqrt(5/pi)(3z^2 - 1), Y21 = (1/2)sqrt(15/pi) xz,
         Y22 = (1/4)sqrt(15/pi)(x^2 - y^2)            (unit vector (x, y, z))
  B_n(r) sqrt(2/r_c) sin(n pi r / r_c) / r,  n = 1..NB
  u(r)   (1-d)^3 (1 + 3d + 6d^2 + 10d^3 + 15d^4 + 21d^5),  d = r/r_c < 1;  0 beyond
"""
import math

import torch


def real_sh(rhat, lmax):
    """rhat [E,3] unit vectors -> list over l of [E, 2l+1] (float64)."""
    x, y, z = rhat[:, 0], rhat[:, 1], rhat[:, 2]
    out = [torch.full_like(x, 0.5 / math.sqrt(math.pi))[:, None]]
    if lmax >= 1:
        c1 = math.sqrt(3.0 / (4.0 * math.pi))
        out.append(torch.stack([c1 * y, c1 * z, c1 * x], dim=1))
    if lmax >= 2:
        a = 0.5 * math.sqrt(15.0 / math.pi)
        b = 0.25 * math.sqrt(5.0 / math.pi)
        c = 0.25 * math.sqrt(15.0 / math.pi)
        out.append(torch.stack([a * x * y, a * y * z, b * (3 * z * z - 1), a * x * z,
                                c * (x * x - y * y)], dim=1))
    if lmax > 2:
        raise ValueError("lmax <= 2 only")
    return out


def bessel(r, r_cut, n_basis):
    """[E] -> [E, NB]."""
    n = torch.arange(1, n_basis + 1, dtype=r.dtype)
    return math.sqrt(2.0 / r_cut) * torch.sin(n[None, :] * math.pi * r[:, None] / r_cut) / r[:, None]


def envelope(r, r_cut):
    """Smooth cutoff, C2 at r_cut, equal to 1 at r = 0."""
    d = r / r_cut
    poly = (1 - d) ** 3 * (1 + 3 * d + 6 * d ** 2 + 10 * d ** 3 + 15 * d ** 4 + 21 * d ** 5)
    return torch.where(d < 1, poly, torch.zeros_like(d))
