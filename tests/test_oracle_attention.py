"""Pins of the oracle's attention layer (oracle/model.py, `layer`) that a
one-neighbour case cannot see: the logit scale d_h^{-1/2}, the contiguous head
split c // d_h, the u-weighting of the softmax, and which Clebsch-Gordan index
takes the sender's features and which the edge harmonic on l1 = l2 paths.

  * attention_layer_5atom.json (tests/golden/make_attention_golden.py): a layer
    evaluated without oracle code -- sympy Clebsch-Gordan coefficients turned
    real, scipy harmonics, scalar loops -- on five atoms with rows of 0, 2 and 3
    neighbours, two heads and unequal logits;
  * a path-(1,1,1) product written out by hand: the sender's l = 1 feature along
    x and the edge along y give a message along +z (the real coupling 1 x 1 -> 1
    is the cross product / sqrt 2, its sign fixed by the first-nonzero-entry
    rule);
  * smoothness: a third neighbour crossing r_cut changes the energy by O(eps^3)
    (the envelope u vanishes to third order and weights both the message and
    the softmax; without u in the softmax the other neighbours' weights jump).
Equations: "Ab Initio Accuracy Beyond the Cutoff", Abstract (equivariant
message-passing Transformer); "Unlocking Tensor Core Performance", section "Why
MLIPs Need Dedicated Performance Optimization" (Clebsch-Gordan coupling).
"""
import json
import math
import os

import numpy as np
import torch

from molecular_dynamics_amd.inputs import ModelConfig, make_weights, weight_layout
from oracle import basis, model

HERE = os.path.dirname(os.path.abspath(__file__))


def _blob(cfg, named):
    """Weight blob in the documented order; matrices not given are zero."""
    parts = []
    for name, r, c in weight_layout(cfg):
        key = name.split(".", 1)[1] if name.startswith("l0.") else name
        m = np.asarray(named[key], np.float32) if key in named else np.zeros((r, c), np.float32)
        assert m.shape == (r, c), (name, m.shape)
        parts.append(m.ravel())
    return np.concatenate(parts)


def _complete_csr(n):
    col = np.array([j for i in range(n) for j in range(n) if j != i], np.int32)
    return np.arange(0, n * (n - 1) + 1, n - 1, dtype=np.int32), col


def test_layer_matches_independent_fixture():
    doc = json.load(open(os.path.join(HERE, "golden", "attention_layer_5atom.json")))
    k = doc["config"]
    cfg = ModelConfig(n_species=1, channels=k["channels"], lmax=k["lmax"], n_bessel=k["n_bessel"],
                      heads=k["heads"], layers=1, cutoff=k["cutoff"], radial_hidden=k["radial_hidden"])
    blob = _blob(cfg, doc["weights"])
    pos = np.array(doc["pos"], np.float64)
    rp, col = _complete_csr(pos.shape[0])  # the layer keeps only r < r_cut itself
    got = model.layer_forward(cfg, blob, 0, np.array(doc["h_in"]), pos, None, rp, col)
    ref = np.array(doc["h_out"])
    assert got.shape == ref.shape
    # the fixture must exercise the softmax: per-head weights differ within a row
    alpha = np.array(doc["alpha"])
    assert np.abs(alpha[:, 2] - alpha[:, 3]).max() > 0.05
    assert np.abs(got - ref).max() < 1e-12 * np.abs(ref).max()


def test_path_111_product_written_out():
    """Sender j directly along +y of receiver i; only path (1,1,1) carries weight;
    ht_j^1 = unit x in channel 0; W_o = I, W_g = 0 (gate 1/2), h_i = 0 except h^0
    for the query.  By hand: v^1 = w (x_hat cross Y_1(y_hat)) / sqrt 2 with
    Y_1(y_hat) = sqrt(3/4pi) y_hat, so m_i^1 = sqrt(3/4pi)/sqrt2 w z_hat (one
    neighbour: alpha = 1) and h_i^1 gains half of it."""
    C, H = 2, 1
    cfg = ModelConfig(n_species=1, channels=C, lmax=1, n_bessel=8, heads=H, layers=1, cutoff=4.0,
                      radial_hidden=4)
    rng = np.random.default_rng(3)
    w1 = rng.standard_normal((4, 8)).astype(np.float32)
    P = cfg.n_paths  # (0,0,0) (0,1,1) (1,0,1) (1,1,0) (1,1,1)
    w2 = np.zeros((P * C, 4), np.float32)
    w2[4 * C + 0] = rng.standard_normal(4)
    eye = np.eye(C, dtype=np.float32)
    named = {"w1": w1, "w2": w2, "wq": eye, "wv0": eye, "wv1": eye, "wo0": eye, "wo1": eye,
             "wg": np.zeros((C, C), np.float32)}
    blob = _blob(cfg, named)
    r = 2.3
    pos = np.array([[0.0, 0.0, 0.0], [0.0, r, 0.0]])
    h_in = np.zeros((2, 4, C))
    h_in[1, 3, 0] = 1.0  # sender: l = 1 along x (k = 3 is m = +1, the x component)
    rp, col = np.array([0, 1, 2], np.int32), np.array([1, 0], np.int32)
    got = model.layer_forward(cfg, blob, 0, h_in, pos, None, rp, col)
    rt = torch.tensor([r], dtype=torch.float64)
    B = basis.bessel(rt, 4.0, 8).numpy()[0]
    u = float(basis.envelope(rt, 4.0)[0])
    hid = B @ w1.astype(np.float64).T
    w = u * float(w2[4 * C].astype(np.float64) @ (hid / (1 + np.exp(-hid))))
    mz = math.sqrt(3 / (4 * math.pi)) / math.sqrt(2) * w
    want = np.zeros((4, C))
    want[2, 0] = 0.5 * mz  # k = 2 is m = 0, the z component
    assert abs(w) > 1e-3
    assert np.abs(got[0] - want).max() < 1e-14
    # atom 1 hears only atom 0, whose l = 1 input is zero: its features pass unchanged
    assert np.array_equal(got[1], h_in[1])


def _energy_open(cfg, W, P, sp):
    n = P.shape[0]
    rp = np.arange(0, n * (n - 1) + 1, n - 1, dtype=np.int32)
    col = np.array([j for i in range(n) for j in range(n) if j != i], np.int32)
    return model.energy(cfg, W, P, sp, None, rp, col, forces=False)["E"]


def test_energy_third_order_when_a_neighbour_crosses_cutoff():
    """Atoms 0, 1, 2 within r_cut of each other; atom 3 moves along +x past atom 0's
    cutoff sphere while staying beyond r_cut of 1 and 2.  E(r_c - eps) - E(r_c) must
    scale as eps^3 (envelope exponent 6: u ~ 56 (eps/r_c)^3)."""
    cfg = ModelConfig(n_species=2, channels=8, lmax=2, n_bessel=8, heads=2, layers=2, cutoff=4.0)
    W = make_weights(cfg, np.random.SeedSequence(77))
    base = np.array([[0.0, 0.0, 0.0], [-1.6, 1.1, 0.3], [-1.2, -1.4, 0.9]])
    sp = np.array([0, 1, 1, 0], np.int32)

    def E(x):
        P = np.vstack([base, [[x, 0.0, 0.0]]])
        return _energy_open(cfg, W, P, sp)

    P_at = np.vstack([base, [[4.0, 0.0, 0.0]]])
    assert np.linalg.norm(P_at[3] - P_at[1]) > 4.0 and np.linalg.norm(P_at[3] - P_at[2]) > 4.0
    e_out = E(4.0)
    assert E(4.3) == e_out  # beyond the cutoff nothing changes
    # leading term eps^3 (the softmax weight u); the message itself also carries
    # B_n(r_c) = 0, one order higher, so halving eps divides the change by 8 plus a
    # little; a C^1-only envelope would give 4, a jump 1
    d = [E(4.0 - eps) - e_out for eps in (0.02, 0.01, 0.005)]
    assert abs(d[0]) > 1e-10
    for a, b in zip(d, d[1:]):
        assert 7.0 < a / b < 12.0, d
