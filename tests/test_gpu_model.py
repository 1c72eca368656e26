"""GPU energy, forces and single layers vs the oracle (float64 CPU).

Bars: float32 features -> energy within 1e-4 of sum_i |E_i| and forces
within 1e-4 of the largest atomic force (atom-wise Euclidean error);
bfloat16 features -> 2e-2 on the same scales.  Boxes span several 16-edge
tiles per row and ragged row ends; both channel-block layouts (C <= 64 and
C = 128) and both feature precisions are covered."""
import numpy as np
import pytest

from tests.helpers import energy_error, force_error, to_dev, workload

pytestmark = pytest.mark.gpu


def _small(n, L, S, C, lmax, H, T, rc, skin, bf16, seed):
    from molecular_dynamics_amd import inputs
    box = inputs.box_uniform(n, L, S, seed)
    cfg = inputs.ModelConfig(n_species=S, channels=C, lmax=lmax, n_bessel=8, heads=H, layers=T, cutoff=rc,
                             feat_bf16=bf16)
    w = inputs.make_weights(cfg, np.random.SeedSequence(seed).spawn(3)[2])
    return inputs.Workload(f"small{n}_{C}_{lmax}_{bf16}", box, cfg, skin, w)


def _lattice(m, spacing, C, lmax, H, T, rc, skin, bf16, seed):
    """m^3 atoms on a cubic lattice whose spacing exceeds r_c + skin: no edges at all"""
    from molecular_dynamics_amd import inputs
    g = (np.arange(m, dtype=np.float32) + 0.5) * np.float32(spacing)
    pos = np.stack(np.meshgrid(g, g, g, indexing="ij"), -1).reshape(-1, 3).astype(np.float32)
    L = float(np.float32(m * spacing))
    sp = (np.arange(pos.shape[0]) % 2).astype(np.int32)
    box = inputs.Box(pos, sp, L, 2)
    cfg = inputs.ModelConfig(n_species=2, channels=C, lmax=lmax, n_bessel=8, heads=H, layers=T, cutoff=rc,
                             feat_bf16=bf16)
    w = inputs.make_weights(cfg, np.random.SeedSequence(seed).spawn(3)[2])
    return inputs.Workload(f"lattice{m}", box, cfg, skin, w)


def _pair(d, L, C, lmax, H, T, rc, skin, bf16, seed):
    """two atoms d apart: one active edge each way"""
    from molecular_dynamics_amd import inputs
    pos = np.array([[2.0, 3.0, 4.0], [2.0 + d * 0.6, 3.0, 4.0 + d * 0.8]], np.float32)
    box = inputs.Box(pos, np.array([0, 1], np.int32), float(np.float32(L)), 2)
    cfg = inputs.ModelConfig(n_species=2, channels=C, lmax=lmax, n_bessel=8, heads=H, layers=T, cutoff=rc,
                             feat_bf16=bf16)
    w = inputs.make_weights(cfg, np.random.SeedSequence(seed).spawn(3)[2])
    return inputs.Workload("pair", box, cfg, skin, w)


CASES = {
    "tiny64": lambda: workload("tiny64"),
    "dense4k": lambda: workload("dense4k"),
    "c128_f32": lambda: _small(1200, 23.0, 3, 128, 2, 4, 2, 5.0, 1.0, False, 7),
    "c64_bf16": lambda: _small(2000, 27.1, 4, 64, 2, 4, 2, 5.0, 1.0, True, 8),
    "c128_bf16": lambda: _small(1500, 24.7, 4, 128, 2, 4, 3, 5.0, 1.0, True, 9),
    "c16_l2": lambda: _small(500, 17.1, 2, 16, 2, 2, 2, 4.5, 0.5, False, 10),
    # lmax 1 with 64 channels (the built lmax-1 instantiation at 32 or more channels):
    # the fragment-ordered weight copies of its three path sets
    "c64_l1_f32": lambda: _small(900, 20.8, 3, 64, 1, 4, 3, 5.0, 1.0, False, 16),
    # degenerate rows: at this density most rows hold 0-3 active edges, some padded
    # edges lie between r_c and r_c + skin, and many atoms have no neighbour at all
    "sparse_f32": lambda: _small(300, 40.0, 3, 128, 2, 4, 2, 5.0, 1.0, False, 11),
    "sparse_bf16": lambda: _small(300, 40.0, 3, 128, 2, 4, 2, 5.0, 1.0, True, 12),
    # no edges at all: E is the readout of the embedding, F = 0
    "isolated": lambda: _lattice(3, 7.0, 64, 2, 4, 2, 5.0, 1.0, False, 13),
    "pair": lambda: _pair(3.3, 13.0, 128, 2, 4, 2, 5.0, 1.0, False, 14),
}


def _gpu_run(w):
    import torch
    from molecular_dynamics_amd import mdmp
    pos, sp = to_dev(w.box)
    g = mdmp.build_neighbors(pos, sp, w.box.L, w.model.cutoff, w.skin)
    model = mdmp.Model(w.model, w.weights)
    e_at = torch.empty(w.box.n, dtype=torch.float32, device="cuda")
    E, F = mdmp.energy_forces(model, g, perm=g.perm, atom_energy=e_at)
    torch.cuda.synchronize()
    return E, F.cpu().numpy(), e_at.cpu().numpy(), g


@pytest.mark.parametrize("name", list(CASES))
def test_energy_forces_parity(name):
    from oracle import model as OM
    from oracle import neighbors as NB
    w = CASES[name]()
    print("case", name, w.box.n, flush=True)
    E, F, e_at, g = _gpu_run(w)
    nb = NB.build_neighbors(w.box.pos, w.box.L, w.model.cutoff, w.skin)
    ref = OM.energy(w.model, w.weights, nb["pos_sorted"], w.box.species[nb["perm"]], w.box.L, nb["row_ptr"],
                    nb["col"])
    Fref = np.empty_like(ref["F"])
    Fref[nb["perm"]] = ref["F"]
    tol = 2e-2 if w.model.feat_bf16 else 1e-4
    ee = energy_error(E, ref["E"], ref["E_atoms"])
    if np.abs(Fref).max() == 0:  # no active edge anywhere: the forces are exactly zero
        assert np.abs(F).max() == 0
        fe = 0.0
    else:
        fe = force_error(F, Fref)
    ae = np.abs(e_at - ref["E_atoms"]).max() / np.abs(ref["E_atoms"]).max()
    print(f"{name}: E {E:.8f} ref {ref['E']:.8f} energy err {ee:.2e} force err {fe:.2e} atom-E err {ae:.2e}",
          flush=True)
    assert ee <= tol
    assert ae <= tol
    assert fe <= tol


def test_determinism_bitwise():
    import torch
    from molecular_dynamics_amd import mdmp
    w = CASES["c128_bf16"]()
    pos, sp = to_dev(w.box)
    g = mdmp.build_neighbors(pos, sp, w.box.L, w.model.cutoff, w.skin)
    model = mdmp.Model(w.model, w.weights)
    ef = mdmp.EnergyForces(model, g.n, g.n_edges)
    E1, F1 = ef(g)
    E1, F1 = E1.clone(), F1.clone()
    E2, F2 = ef(g)
    torch.cuda.synchronize()
    assert torch.equal(E1, E2) and torch.equal(F1, F2)


@pytest.mark.parametrize("name,layer", [("dense4k", 0), ("dense4k", 1), ("c128_bf16", 1), ("tiny64", 0)])
def test_layer_forward_parity(name, layer):
    import torch
    from molecular_dynamics_amd import mdmp
    from oracle import model as OM
    w = CASES[name]()
    pos, sp = to_dev(w.box)
    g = mdmp.build_neighbors(pos, sp, w.box.L, w.model.cutoff, w.skin)
    model = mdmp.Model(w.model, w.weights)
    K, C = model.K, w.model.channels
    rng = np.random.default_rng(layer)
    h_in = rng.standard_normal((w.box.n, K, C)).astype(np.float32)
    if w.model.feat_bf16:
        hb = torch.tensor(h_in).view(torch.int32) >> 16
        h_dev = hb.to(torch.int16).cuda()
        h_in = mdmp.bf16_to_f32(h_dev).cpu().numpy()
    else:
        h_dev = torch.tensor(h_in, device="cuda")
    h_out = mdmp.layer_forward(model, layer, g, h_dev)
    torch.cuda.synchronize()
    got = mdmp.bf16_to_f32(h_out).cpu().numpy() if w.model.feat_bf16 else h_out.cpu().numpy()
    nb = {"row_ptr": g.row_ptr.cpu().numpy(), "col": g.col[:g.n_edges].cpu().numpy()}
    ref = OM.layer_forward(w.model, w.weights, layer, h_in, g.pos.cpu().numpy(), w.box.L, nb["row_ptr"], nb["col"])
    tol = 2e-2 if w.model.feat_bf16 else 1e-4
    if w.model.feat_bf16:
        # features are stored in bfloat16: compare the stored result itself
        err = np.abs(got - ref).max() / np.abs(ref).max()
    else:
        # float32: compare the update, the part the layer computes
        d_ref = ref - h_in
        err = np.abs((got - h_in) - d_ref).max() / np.abs(d_ref).max()
    print(f"layer {name}/{layer}: update err {err:.2e}", flush=True)
    assert err <= tol


def test_embed():
    import torch
    from molecular_dynamics_amd import inputs, mdmp
    w = workload("dense4k")
    pos, sp = to_dev(w.box)
    g = mdmp.build_neighbors(pos, sp, w.box.L, w.model.cutoff, w.skin)
    model = mdmp.Model(w.model, w.weights)
    h = mdmp.embed(model, g).cpu().numpy()
    emb = inputs.split_weights(w.model, w.weights)["emb"]
    assert np.array_equal(h[:, 0, :], emb[g.species.cpu().numpy()])
    assert np.all(h[:, 1:, :] == 0)


def test_single_atom_is_rejected():
    """n < 2 is outside the neighbour builder's contract (MP_ERR_ARG, no launch)."""
    from molecular_dynamics_amd import mdmp
    w = _lattice(1, 13.0, 16, 1, 2, 1, 5.0, 1.0, False, 15)
    pos, sp = to_dev(w.box)
    with pytest.raises(mdmp.MPError) as e:
        mdmp.build_neighbors(pos, sp, w.box.L, w.model.cutoff, w.skin)
    assert e.value.code == mdmp.MP_ERR_ARG


def test_atom_order_invariance():
    """Energy and (un-permuted) forces do not depend on the atom order of the neighbour
    build (Hilbert, Morton, input): they agree to float32 rounding of the reordered sums."""
    import torch
    from molecular_dynamics_amd import mdmp
    w = CASES["dense4k"]()
    pos, sp = to_dev(w.box)
    model = mdmp.Model(w.model, w.weights)
    out = {}
    for order in ("hilbert", "morton", "input"):
        g = mdmp.build_neighbors(pos, sp, w.box.L, w.model.cutoff, w.skin, order=order)
        E, F = mdmp.energy_forces(model, g, perm=g.perm)
        torch.cuda.synchronize()
        out[order] = (E, F.cpu().numpy())
    E0, F0 = out["hilbert"]
    for order in ("morton", "input"):
        E, F = out[order]
        de = abs(E - E0) / abs(E0)
        df = force_error(F, F0)
        print(f"order {order}: rel dE {de:.2e}, force diff {df:.2e}", flush=True)
        assert de < 1e-6 and df < 1e-5



def test_non_finite_output_is_reported():
    """A NaN readout weight with finite positions: mp_energy_forces only enqueues (MP_OK), and
    mp_energy_forces_status then returns MP_ERR_NUMERIC; the same workspace reports MP_OK
    again for finite weights.  An MD handle on the NaN model fails in mp_md_set_state."""
    import torch
    from molecular_dynamics_amd import inputs, mdmp
    w = CASES["c128_f32"]()
    pos, sp = to_dev(w.box)
    g = mdmp.build_neighbors(pos, sp, w.box.L, w.model.cutoff, w.skin)
    bad = w.weights.copy()
    bad[-3] = np.nan  # an entry of w_out, the readout's last vector
    ef_bad = mdmp.EnergyForces(mdmp.Model(w.model, bad), g.n, g.n_edges)
    E, F = ef_bad(g, check=False)
    with pytest.raises(mdmp.MPError) as e:
        ef_bad.status()
    assert e.value.code == mdmp.MP_ERR_NUMERIC
    assert not np.isfinite(float(E.item()))
    good = mdmp.EnergyForces(mdmp.Model(w.model, w.weights), g.n, g.n_edges)
    good.ws.copy_(ef_bad.ws)  # the flag of the failed call is cleared by the next evaluation
    E, F = good(g)
    torch.cuda.synchronize()
    assert np.isfinite(float(E.item())) and bool(torch.isfinite(F).all())
    md = mdmp.MD(mdmp.Model(w.model, bad), w.box.n, w.box.L, w.skin, 0.5, inputs.MASSES_SALT[:3])
    vel = torch.zeros_like(pos)
    with pytest.raises(mdmp.MPError) as e:
        md.set_state(pos, vel, sp)
    assert e.value.code == mdmp.MP_ERR_NUMERIC
    md.close()
