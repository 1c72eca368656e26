"""Pins of the oracle's large-box force evaluation (oracle/model.py):

  * `layer_chunked` and `energy_forces_chunked` (whole receiver rows per chunk;
    a reverse sweep layer by layer) give the features, energy and forces of
    `layer` / `energy` to 1e-12, with chunks small enough that every row boundary
    case occurs (rows with no edges, a chunk of one row), also with subsets of
    receivers and of read atoms;
  * `forces_local` (the open cluster of radius 2 T r_cut + delta about a centre
    atom) equals the whole-box forces of `energy` for every atom within delta
    of the centre, on periodic boxes large enough for the cluster -- the
    locality of T stacked layers ("Ab Initio Accuracy Beyond the Cutoff",
    Abstract) made exact.
"""
import numpy as np
import pytest
import torch

from molecular_dynamics_amd.inputs import ModelConfig, box_uniform, make_weights
from oracle import model, neighbors

torch.set_num_threads(4)


def _open_csr(P, R):
    d = np.linalg.norm(P[:, None] - P[None], axis=-1)
    np.fill_diagonal(d, np.inf)
    src, dst = np.nonzero(d < R)
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(src, minlength=P.shape[0]))]).astype(np.int32)
    return row_ptr, dst.astype(np.int32)


def test_chunked_evaluation_equals_energy():
    """Features of `layer_chunked` and forces of `energy_forces_chunked` (forward by
    chunks of rows, reverse sweep layer by layer) against autograd through `energy`,
    with chunks of a few edges so every boundary case occurs (rows without edges,
    chunks of one row); also with a subset of receivers per layer and of read atoms."""
    cfg = ModelConfig(n_species=3, channels=8, lmax=2, n_bessel=8, heads=2, layers=2, cutoff=3.0)
    W = make_weights(cfg, np.random.SeedSequence(9))
    prm = model.Params(cfg, W)
    cgs = model.cg_table(cfg.lmax)
    rng = np.random.default_rng(4)
    X0 = rng.random((60, 3)) * 14.0  # sparse: some atoms have no neighbour at all
    n = X0.shape[0]
    rp, col = _open_csr(X0, cfg.cutoff)
    row = model.csr_rows(rp)
    assert (np.diff(rp) == 0).any()
    sp = rng.integers(0, 3, n)
    ref = model.energy(cfg, W, X0, sp, None, rp, col)
    X = torch.tensor(X0)
    h = model.embed(cfg, prm, sp)
    colt = torch.as_tensor(col.astype(np.int64))
    r, rhat = model.edge_geometry(X, None, row, colt)
    h1 = model.layer(cfg, prm.layers[0], h, r, rhat, row, colt, n, cgs)
    h2 = model.layer_chunked(cfg, prm.layers[0], h, X, None, row, colt, n, cgs, max_edges=7)
    for a, b in zip(h1, h2):
        assert torch.abs(a - b).max() <= 1e-12 * torch.abs(a).max()
    E, F = model.energy_forces_chunked(cfg, prm, cgs, X, sp, None, row, colt, max_edges=7)
    assert abs(E - ref["E"]) <= 1e-12 * np.abs(ref["E_atoms"]).sum()
    assert np.abs(ref["F"]).max() > 1e-3
    assert np.abs(F - ref["F"]).max() <= 1e-12 * np.abs(ref["F"]).max()
    # a subset of receivers in the first layer and of read atoms, against autograd
    keep0 = torch.as_tensor(rng.random(n) < 0.6)
    read = np.nonzero(rng.random(n) < 0.5)[0]
    Xg = torch.tensor(X0, requires_grad=True)
    r, rhat = model.edge_geometry(Xg, None, row, colt)
    e0 = keep0[row]
    hh = model.layer(cfg, prm.layers[0], h, r[e0], rhat[e0], row[e0], colt[e0], n, cgs)
    hh = model.layer(cfg, prm.layers[1], hh, r, rhat, row, colt, n, cgs)
    Es = model.readout(prm, hh[0])[torch.as_tensor(read)].sum()
    (g,) = torch.autograd.grad(Es, Xg)
    E2, F2 = model.energy_forces_chunked(cfg, prm, cgs, X, sp, None, row, colt,
                                         keep=[keep0, torch.ones(n, dtype=torch.bool)], read=read, max_edges=5)
    assert abs(E2 - float(Es.detach())) <= 1e-12 * abs(float(Es.detach())) + 1e-14
    assert np.abs(F2 + g.numpy()).max() <= 1e-12 * np.abs(g.numpy()).max()


@pytest.mark.parametrize("T, rc, delta, L, seed", [(2, 2.5, 1.0, 25.0, 1), (3, 2.0, 1.5, 30.0, 2)])
def test_forces_local_equals_whole_box(T, rc, delta, L, seed):
    cfg = ModelConfig(n_species=2, channels=8, lmax=2, n_bessel=8, heads=2, layers=T, cutoff=rc)
    W = make_weights(cfg, np.random.SeedSequence(30 + seed))
    n = int(round(0.1 * L ** 3))
    box = box_uniform(n, L, 2, 100 + seed)
    nb = neighbors.build_neighbors(box.pos, box.L, rc, 0.0)
    P = nb["pos_sorted"]
    sp = box.species[nb["perm"]]
    full = model.energy(cfg, W, P, sp, box.L, nb["row_ptr"], nb["col"])
    rng = np.random.default_rng(seed)
    checked = 0
    for center in rng.choice(n, 2, replace=False):
        idx, F = model.forces_local(cfg, W, P, sp, box.L, int(center), delta=delta, max_edges=500)
        assert int(center) in idx.tolist()
        ref = full["F"][idx]
        assert np.abs(F - ref).max() <= 1e-10 * np.abs(full["F"]).max(), (center, np.abs(F - ref).max())
        checked += idx.size
    assert checked >= 2


def test_forces_local_rejects_small_box():
    cfg = ModelConfig(n_species=1, channels=8, lmax=1, n_bessel=8, heads=2, layers=2, cutoff=3.0)
    W = make_weights(cfg, np.random.SeedSequence(1))
    box = box_uniform(200, 12.6, 1, 3)
    with pytest.raises(ValueError):
        model.forces_local(cfg, W, box.pos, box.species, box.L, 0)
