"""Oracle pins against fixed values from outside the oracle: the text fixtures under
tests/golden/ (each with its derivation in its header) and a library routine
(scipy's complex spherical harmonics).  The pages print no worked example of the
computation, so these fixtures come from the closed forms and the published
algorithms the model is built from."""
import math
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def _rows(name):
    return np.loadtxt(os.path.join(HERE, "golden", name), comments="#", ndmin=2)


def test_envelope_and_bessel_closed_form():
    from oracle import basis
    t = _rows("bessel_envelope_closed_form.txt")
    r = torch.tensor(t[:, 0], dtype=torch.float64)
    u = basis.envelope(r, 5.0).numpy()
    assert np.abs(u - t[:, 1]).max() < 1e-14
    inside = t[:, 0] < 5.0
    b = basis.bessel(r[inside], 5.0, 8).numpy()
    assert np.abs(b - t[inside, 2:]).max() < 1e-14
    # r = r_c / 2: sin(n pi / 2) is 1, 0, -1, 0, ...
    half = t[t[:, 0] == 2.5][0, 2:]
    ref = math.sqrt(2 / 5.0) / 2.5 * np.array([1, 0, -1, 0, 1, 0, -1, 0], dtype=float)
    assert np.abs(half - ref).max() < 1e-15


def test_hilbert_one_bit_is_gray_code():
    from oracle import hilbert
    t = _rows("hilbert_one_bit.txt").astype(np.int64)
    keys = hilbert.hilbert_index(t[:, 0], t[:, 1], t[:, 2], bits=1)
    assert keys.tolist() == t[:, 3].tolist()


def _real_sh_scipy(x, y, z, lmax):
    """Orthonormal real harmonics from scipy's complex ones (Condon-Shortley phase):
    Y_{l,m} = sqrt2 (-1)^m Re Y_l^m (m > 0), Y_{l,0} = Y_l^0, Y_{l,-m} = sqrt2 (-1)^m Im Y_l^m."""
    from scipy.special import sph_harm_y
    theta = np.arccos(np.clip(z, -1, 1))
    phi = np.arctan2(y, x)
    out = []
    for l in range(lmax + 1):
        cols = []
        for m in range(-l, l + 1):
            c = sph_harm_y(l, abs(m), theta, phi)
            if m > 0:
                cols.append(math.sqrt(2) * (-1) ** m * c.real)
            elif m == 0:
                cols.append(c.real)
            else:
                cols.append(math.sqrt(2) * (-1) ** abs(m) * c.imag)
        out.append(np.stack(cols, axis=1))
    return out


def test_real_sh_matches_library_routine():
    from oracle import basis
    rng = np.random.default_rng(7)
    v = rng.normal(size=(200, 3))
    v = np.concatenate([v, np.eye(3), -np.eye(3), [[0.6, 0.0, -0.8], [1 / 3, 2 / 3, 2 / 3]]])
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    got = basis.real_sh(torch.tensor(v), 2)
    ref = _real_sh_scipy(v[:, 0], v[:, 1], v[:, 2], 2)
    for l in range(3):
        assert np.abs(got[l].numpy() - ref[l]).max() < 1e-12, l
