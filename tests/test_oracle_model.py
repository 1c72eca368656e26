"""Pins for the oracle's layers, energy and forces (oracle/model.py).

  * forces equal the negative central finite difference of the energy
    (float64, h = 1e-5 A) -- calculus, independent of autograd's wiring;
  * translation invariance (periodic shift, full rebuild) and sum F = 0;
  * permutation invariance (relabelled slots and CSR);
  * rotation: on an open cluster, E is invariant, F rotates with the atoms, and
    layer features of order l rotate by D^l taken from the harmonics;
  * isolated atoms: with no pair inside r_cut the energy is the readout of
    the embedding alone;
  * two atoms with lmax = 0: attention collapses (alpha = 1) and the layer is
    a scalar chain written out here by hand from the layer equations --
    wiring of W_1/W_2 rows, W_v/W_o/W_r orientation ([out][in]) and Y_00;
  * direction convention: for j directly above i the l = 1 message of i
    points along +z (r_ij = x_j - x_i);
  * the energy is continuous through r_cut, constant beyond it, and a list
    built with a skin gives the same energy and forces as one without.
"""
import math

import numpy as np
import torch

from molecular_dynamics_amd.inputs import ModelConfig, make_weights, split_weights
from oracle import cg, model, neighbors

torch.set_num_threads(4)


def _cfg(lmax=2, C=8, H=2, T=2, S=3, rc=4.0):
    return ModelConfig(n_species=S, channels=C, lmax=lmax, n_bessel=8, heads=H, layers=T, cutoff=rc)


def _cluster(n, seed, spread=5.0, S=3):
    rng = np.random.default_rng(seed)
    pts = []
    while len(pts) < n:
        p = rng.standard_normal(3) * spread / 2
        if all(np.linalg.norm(p - q) > 1.2 for q in pts):
            pts.append(p)
    return np.array(pts, np.float64), rng.integers(0, S, n).astype(np.int32)


def _open_csr(P, R):
    d = np.linalg.norm(P[:, None] - P[None], axis=-1)
    np.fill_diagonal(d, np.inf)
    src, dst = np.nonzero(d < R)
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(src, minlength=P.shape[0]))]).astype(np.int32)
    return row_ptr, dst.astype(np.int32)


def _w(cfg, seed=5):
    return make_weights(cfg, np.random.SeedSequence(seed))


def test_forces_equal_central_difference_open_cluster():
    cfg = _cfg()
    W = _w(cfg)
    P, sp = _cluster(14, 1)
    rp, col = _open_csr(P, cfg.cutoff + 1.0)
    out = model.energy(cfg, W, P, sp, None, rp, col)
    h = 1e-5
    fd = np.zeros_like(P)
    for i in range(P.shape[0]):
        for a in range(3):
            Pp, Pm = P.copy(), P.copy()
            Pp[i, a] += h
            Pm[i, a] -= h
            ep = model.energy(cfg, W, Pp, sp, None, rp, col, forces=False)["E"]
            em = model.energy(cfg, W, Pm, sp, None, rp, col, forces=False)["E"]
            fd[i, a] = -(ep - em) / (2 * h)
    fmax = np.abs(out["F"]).max()
    assert fmax > 1e-3
    assert np.abs(fd - out["F"]).max() < 1e-7 * max(1.0, fmax) + 1e-8


def test_forces_central_difference_periodic_tiny_box():
    from molecular_dynamics_amd.inputs import workload
    w = workload("tiny64")
    nb = neighbors.build_neighbors(w.box.pos, w.box.L, w.model.cutoff, w.skin)
    P = nb["pos_sorted"].astype(np.float64)
    sp = w.box.species[nb["perm"]]
    out = model.energy(w.model, w.weights, P, sp, w.box.L, nb["row_ptr"], nb["col"])
    h = 1e-5
    rng = np.random.default_rng(0)
    for i in rng.choice(P.shape[0], 6, replace=False):
        for a in range(3):
            Pp, Pm = P.copy(), P.copy()
            Pp[i, a] += h
            Pm[i, a] -= h
            ep = model.energy(w.model, w.weights, Pp, sp, w.box.L, nb["row_ptr"], nb["col"], forces=False)["E"]
            em = model.energy(w.model, w.weights, Pm, sp, w.box.L, nb["row_ptr"], nb["col"], forces=False)["E"]
            assert abs(-(ep - em) / (2 * h) - out["F"][i, a]) < 1e-7 * np.abs(out["F"]).max() + 1e-9
    assert np.abs(out["F"].sum(0)).max() < 1e-12


def test_translation_and_permutation_invariance():
    cfg = _cfg(T=2, rc=3.5)
    W = _w(cfg)
    rng = np.random.default_rng(2)
    L = np.float32(12.0)
    x = (rng.random((120, 3)) * L).astype(np.float32)
    sp = rng.integers(0, 3, 120).astype(np.int32)
    nb = neighbors.build_neighbors(x, L, cfg.cutoff, 0.5)
    e0 = model.energy(cfg, W, nb["pos_sorted"], sp[nb["perm"]], L, nb["row_ptr"], nb["col"])
    # exact test in float64: shifted (unwrapped) positions, same pair set, minimum image
    shift = np.array([3.3, -7.9, 25.1])
    e1 = model.energy(cfg, W, nb["pos_sorted"].astype(np.float64) + shift, sp[nb["perm"]], L,
                      nb["row_ptr"], nb["col"])
    assert abs(e0["E"] - e1["E"]) < 1e-11 * abs(e0["E"])
    assert np.abs(e0["F"] - e1["F"]).max() < 1e-10 * np.abs(e0["F"]).max()
    assert np.abs(e0["F"].sum(0)).max() < 1e-11
    # full rebuild from float32 shifted inputs: equal up to float32 rounding of the wrap
    x2 = x + shift.astype(np.float32)
    nb2 = neighbors.build_neighbors(x2, L, cfg.cutoff, 0.5)
    e2 = model.energy(cfg, W, nb2["pos_sorted"], sp[nb2["perm"]], L, nb2["row_ptr"], nb2["col"])
    assert abs(e0["E"] - e2["E"]) < 1e-6 * abs(e0["E"])
    f0 = np.empty_like(e0["F"]); f0[nb["perm"]] = e0["F"]
    f2 = np.empty_like(e2["F"]); f2[nb2["perm"]] = e2["F"]
    assert np.abs(f0 - f2).max() < 1e-4 * np.abs(f0).max()
    # relabel the slots: energy is a sum over atoms and edges, order must not matter
    q = rng.permutation(120)
    inv = np.argsort(q)
    P = nb["pos_sorted"][q]
    rp, col = nb["row_ptr"], nb["col"]
    rows = [inv[col[rp[s]:rp[s + 1]]] for s in q]
    rp3 = np.concatenate([[0], np.cumsum([r.size for r in rows])]).astype(np.int32)
    col3 = np.concatenate(rows).astype(np.int32)
    e3 = model.energy(cfg, W, P, sp[nb["perm"]][q], L, rp3, col3)
    assert abs(e0["E"] - e3["E"]) < 1e-12 * abs(e0["E"]) + 1e-12
    assert np.abs(e3["F"] - e0["F"][q]).max() < 1e-12


def test_rotation_invariance_and_feature_equivariance():
    cfg = _cfg(T=2)
    W = _w(cfg, 11)
    P, sp = _cluster(16, 4)
    rp, col = _open_csr(P, cfg.cutoff + 0.5)
    Q = cg._rotation(np.random.default_rng(8))
    a = model.energy(cfg, W, P, sp, None, rp, col, keep_features=True)
    b = model.energy(cfg, W, P @ Q.T, sp, None, rp, col, keep_features=True)
    assert abs(a["E"] - b["E"]) < 1e-10 * max(1.0, abs(a["E"]))
    assert np.abs(a["F"] @ Q.T - b["F"]).max() < 1e-10
    D = [cg.wigner_real(l, Q) for l in range(3)]
    for t in range(cfg.layers):
        ha, hb = a["h"][t], b["h"][t]
        k = 0
        for l in range(3):
            blk_a = ha[:, k:k + 2 * l + 1, :]
            blk_b = hb[:, k:k + 2 * l + 1, :]
            assert np.abs(np.einsum("mn,anc->amc", D[l], blk_a) - blk_b).max() < 1e-10
            if l > 0:
                assert np.abs(blk_a).max() > 1e-4, "l > 0 features must be populated"
            k += 2 * l + 1


def test_isolated_atoms_energy_is_embedding_readout():
    cfg = _cfg(T=3)
    W = _w(cfg, 2)
    P = np.array([[0, 0, 0], [10, 0, 0], [0, 10, 0]], np.float64)
    sp = np.array([0, 1, 2], np.int32)
    rp, col = _open_csr(P, cfg.cutoff + 1)
    out = model.energy(cfg, W, P, sp, None, rp, col)
    ws = split_weights(cfg, W)
    h0 = ws["emb"][sp].astype(np.float64)
    z = h0 @ ws["wr"].astype(np.float64).T
    expect = (z / (1 + np.exp(-z)) * ws["wout"][0]).sum()
    assert abs(out["E"] - expect) < 1e-12
    assert np.abs(out["F"]).max() == 0.0


def _silu(x):
    return x / (1 + np.exp(-x))


def test_two_atom_scalar_chain_lmax0():
    cfg = ModelConfig(n_species=2, channels=2, lmax=0, n_bessel=8, heads=1, layers=1, cutoff=5.0)
    W = _w(cfg, 21)
    ws = {k: v.astype(np.float64) for k, v in split_weights(cfg, W).items()}
    r = 2.7
    P = np.array([[0, 0, 0], [0.6, -1.1, 0.0]], np.float64)
    P[1] *= r / np.linalg.norm(P[1])
    sp = np.array([0, 1], np.int32)
    rp = np.array([0, 1, 2], np.int32)
    col = np.array([1, 0], np.int32)
    out = model.energy(cfg, W, P, sp, None, rp, col, forces=False)
    rc = cfg.cutoff
    n = np.arange(1, 9)
    B = math.sqrt(2 / rc) * np.sin(n * math.pi * r / rc) / r
    d = r / rc
    u = (1 - d) ** 3 * (1 + 3 * d + 6 * d ** 2 + 10 * d ** 3 + 15 * d ** 4 + 21 * d ** 5)
    w = u * (ws["l0.w2"] @ _silu(ws["l0.w1"] @ B))          # [C], single path (0,0,0)
    y00 = 0.5 / math.sqrt(math.pi)
    E = 0.0
    for i, j in [(0, 1), (1, 0)]:
        hi, hj = ws["emb"][sp[i]], ws["emb"][sp[j]]
        m = w * (ws["l0.wv0"] @ hj) * y00                  # alpha = 1 for a single neighbour
        hn = hi + _silu(ws["l0.wo0"] @ m)
        E += (ws["wout"][0] * _silu(ws["wr"] @ hn)).sum()
    assert abs(out["E"] - E) < 1e-12


def test_direction_convention_l1_message_points_to_sender():
    cfg = ModelConfig(n_species=1, channels=4, lmax=1, n_bessel=8, heads=1, layers=1, cutoff=5.0)
    W = _w(cfg, 3)
    ws = {k: v.astype(np.float64) for k, v in split_weights(cfg, W).items()}
    P = np.array([[0, 0, 0], [0, 0, 2.0]], np.float64)      # atom 1 directly above atom 0
    sp = np.zeros(2, np.int32)
    out = model.energy(cfg, W, P, sp, None, np.array([0, 1, 2], np.int32), np.array([1, 0], np.int32),
                       forces=False, keep_features=True)
    h1 = out["h"][0][0, 1:4, :]                              # atom 0, l = 1 block, m = -1, 0, 1
    assert np.abs(h1[[0, 2]]).max() < 1e-14                  # only the z (m = 0) component
    # m^1 of atom 0 from path (0,1,1): w * ht^0_j * Y_1(+z); gate gamma = sigmoid(W_g m^0)
    r = 2.0
    rc = cfg.cutoff
    n = np.arange(1, 9)
    B = math.sqrt(2 / rc) * np.sin(n * math.pi * r / rc) / r
    d = r / rc
    u = (1 - d) ** 3 * (1 + 3 * d + 6 * d ** 2 + 10 * d ** 3 + 15 * d ** 4 + 21 * d ** 5)
    w = (u * (ws["l0.w2"] @ _silu(ws["l0.w1"] @ B))).reshape(len(cg.paths(1)), 4)
    ht0 = ws["l0.wv0"] @ ws["emb"][0]
    m0 = w[0] * ht0 * 0.5 / math.sqrt(math.pi)
    m1z = w[1] * ht0 * math.sqrt(3 / (4 * math.pi))       # +z: r_ij = x_j - x_i
    gamma = 1 / (1 + np.exp(-(ws["l0.wg"] @ m0)))
    expect = gamma * (ws["l0.wo1"] @ m1z)
    assert np.abs(h1[1] - expect).max() < 1e-12


def test_cutoff_smoothness_and_skin_independence():
    cfg = _cfg(T=2, rc=4.0)
    W = _w(cfg, 7)
    sp = np.array([0, 1], np.int32)
    rp, col = np.array([0, 1, 2], np.int32), np.array([1, 0], np.int32)
    e = []
    for r in [3.999, 3.99999, 4.0, 4.5]:
        e.append(model.energy(cfg, W, np.array([[0, 0, 0], [r, 0, 0]]), sp, None, rp, col, forces=False)["E"])
    e_iso = model.energy(cfg, W, np.array([[0, 0, 0], [50, 0, 0]]), sp, None, rp, col, forces=False)["E"]
    assert e[2] == e_iso and e[3] == e_iso
    assert abs(e[1] - e_iso) < 1e-12 and abs(e[0] - e_iso) < 1e-6
    # skin 0 vs skin 1: same energy and forces
    rng = np.random.default_rng(4)
    L = np.float32(13.0)
    x = (rng.random((150, 3)) * L).astype(np.float32)
    s = rng.integers(0, 3, 150).astype(np.int32)
    n0 = neighbors.build_neighbors(x, L, cfg.cutoff, 0.0)
    n1 = neighbors.build_neighbors(x, L, cfg.cutoff, 1.0)
    assert n1["row_ptr"][-1] > n0["row_ptr"][-1]
    a = model.energy(cfg, W, n0["pos_sorted"], s[n0["perm"]], L, n0["row_ptr"], n0["col"])
    b = model.energy(cfg, W, n1["pos_sorted"], s[n1["perm"]], L, n1["row_ptr"], n1["col"])
    assert abs(a["E"] - b["E"]) < 1e-12 * abs(a["E"])
    assert np.abs(a["F"] - b["F"]).max() < 1e-12


def test_atom_energy_local_equals_full_box():
    """The receptive-field evaluation of one atom's energy equals that atom's
    entry of the whole-box evaluation (periodic box, two layers, so the field
    of 2 r_cut + margin fits in half the box)."""
    from molecular_dynamics_amd import inputs
    from oracle import model as OM
    from oracle import neighbors as NB
    box = inputs.box_uniform(900, 22.0, 3, 41)
    cfg = inputs.ModelConfig(n_species=3, channels=8, lmax=2, n_bessel=8, heads=2, layers=2, cutoff=4.5)
    w = inputs.make_weights(cfg, np.random.SeedSequence(41).spawn(3)[2])
    nb = NB.build_neighbors(box.pos, box.L, cfg.cutoff, 0.5)
    sp = box.species[nb["perm"]]
    full = OM.energy(cfg, w, nb["pos_sorted"], sp, box.L, nb["row_ptr"], nb["col"], forces=False)["E_atoms"]
    for k in (0, 13, 450, 899):
        e = OM.atom_energy_local(cfg, w, nb["pos_sorted"], sp, box.L, k)
        assert abs(e - full[k]) <= 1e-12 * max(1.0, abs(full[k]))
