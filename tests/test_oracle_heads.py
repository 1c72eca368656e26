"""Pins of the oracle's several-readout-heads evaluation (oracle.model.energy_heads,
"Exascale Multi-Task Graph Foundation Models", Fig. 5) against the single-readout oracle
(oracle.model.energy, pinned by its own tests) and against central differences:

* one head with lam = 1 and the blob's own readout is the single-readout model;
* each head's energy equals a full single-readout evaluation with that head's readout
  placed in the blob (the encoder's output does not depend on the readout);
* E = sum_k lam_k E_k, and its forces equal sum_k lam_k F_k of those separate
  evaluations (differentiation is linear);
* the forces are minus the central-difference gradient of E.
"""
import numpy as np
import torch

from molecular_dynamics_amd.inputs import ModelConfig, make_weights
from oracle import model, neighbors

torch.set_num_threads(4)


def _setup(C=8, T=2, rc=3.5, n=120, seed=2):
    cfg = ModelConfig(n_species=3, channels=C, lmax=2, n_bessel=8, heads=2, layers=T, cutoff=rc)
    W = make_weights(cfg, np.random.SeedSequence(5))
    rng = np.random.default_rng(seed)
    L = np.float32(12.0)
    x = (rng.random((n, 3)) * L).astype(np.float32)
    sp = rng.integers(0, 3, n).astype(np.int32)
    nb = neighbors.build_neighbors(x, L, cfg.cutoff, 0.5)
    return cfg, W, L, nb["pos_sorted"], sp[nb["perm"]], nb["row_ptr"], nb["col"]


def _heads(C, R, seed=9):
    rng = np.random.default_rng(seed)
    wr = (rng.standard_normal((R, C, C)) / np.sqrt(C)).astype(np.float32)
    wout = (rng.standard_normal((R, C)) / np.sqrt(C)).astype(np.float32)
    return wr, wout


def _with_readout(W, C, wr, wout):
    w = np.array(W, np.float32).copy()
    w[-(C * C + C):-C] = wr.ravel()
    w[-C:] = wout.ravel()
    return w


def test_one_head_is_the_model_readout():
    cfg, W, L, x, sp, rp, col = _setup()
    C = cfg.channels
    ref = model.energy(cfg, W, x, sp, L, rp, col)
    wr = np.asarray(W[-(C * C + C):-C], np.float32).reshape(1, C, C)
    wout = np.asarray(W[-C:], np.float32).reshape(1, C)
    out = model.energy_heads(cfg, W, wr, wout, [1.0], x, sp, L, rp, col)
    assert abs(out["E"] - ref["E"]) <= 1e-12 * np.abs(ref["E_atoms"]).sum()
    assert abs(out["E_heads"][0] - ref["E"]) <= 1e-12 * np.abs(ref["E_atoms"]).sum()
    assert np.abs(out["E_atoms"][0] - ref["E_atoms"]).max() <= 1e-12
    assert np.abs(out["F"] - ref["F"]).max() <= 1e-11 * np.abs(ref["F"]).max()


def test_heads_equal_separate_evaluations_and_forces_are_linear():
    cfg, W, L, x, sp, rp, col = _setup()
    C, R = cfg.channels, 3
    wr, wout = _heads(C, R)
    lam = np.array([0.7, -1.3, 2.1], np.float32)
    out = model.energy_heads(cfg, W, wr, wout, lam, x, sp, L, rp, col)
    F_sum = np.zeros_like(out["F"])
    E_sum = 0.0
    for k in range(R):
        ref = model.energy(cfg, _with_readout(W, C, wr[k], wout[k]), x, sp, L, rp, col)
        scale = np.abs(ref["E_atoms"]).sum()
        assert abs(out["E_heads"][k] - ref["E"]) <= 1e-12 * scale
        assert np.abs(out["E_atoms"][k] - ref["E_atoms"]).max() <= 1e-12
        F_sum += float(lam[k]) * ref["F"]
        E_sum += float(lam[k]) * ref["E"]
    assert abs(out["E"] - E_sum) <= 1e-12 * max(1.0, abs(E_sum))
    assert abs(out["E"] - float(np.dot(lam.astype(np.float64), out["E_heads"]))) <= 1e-12 * max(1.0, abs(E_sum))
    assert np.abs(out["F"] - F_sum).max() <= 1e-11 * np.abs(F_sum).max()


def test_head_forces_equal_central_difference():
    cfg, W, L, x, sp, rp, col = _setup(n=40, seed=4)
    C = cfg.channels
    wr, wout = _heads(C, 2, seed=3)
    lam = np.array([1.5, -0.5], np.float32)
    x = x.astype(np.float64)
    out = model.energy_heads(cfg, W, wr, wout, lam, x, sp, L, rp, col)
    h = 1e-5
    fmax = np.abs(out["F"]).max()
    for i, a in [(0, 0), (3, 1), (7, 2), (11, 0), (20, 2), (33, 1)]:
        xp, xm = x.copy(), x.copy()
        xp[i, a] += h
        xm[i, a] -= h
        ep = model.energy_heads(cfg, W, wr, wout, lam, xp, sp, L, rp, col, forces=False)["E"]
        em = model.energy_heads(cfg, W, wr, wout, lam, xm, sp, L, rp, col, forces=False)["E"]
        assert abs(-(ep - em) / (2 * h) - out["F"][i, a]) <= 1e-7 * fmax
