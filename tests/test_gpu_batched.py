"""Batches of small open structures (mp_build_neighbors_batched, mp_structure_energies)
vs the oracle, structure by structure: the list bit for bit; per-structure energies
and forces to the bars of the single-box parity tests (float32 1e-4, bf16 2e-2).
Structures of 1 to 40 atoms, including single atoms and structures without any
pair inside the cutoff."""
import numpy as np
import pytest

from tests.helpers import force_error

pytestmark = pytest.mark.gpu


def _batch(seed, n_struct=60, n_min=1, n_max=40):
    from molecular_dynamics_amd import inputs
    pos, sp, sptr = inputs.batch_molecules(n_struct, n_min, n_max, seed, n_species=3)
    # a few spread-out structures whose atoms have no partner at all
    for b in (3, 17):
        if b >= n_struct:
            continue
        a0, a1 = sptr[b], sptr[b + 1]
        pos[a0:a1] = pos[a0:a1] * np.float32(6.0)
    return pos, sp, sptr


def _gpu(pos, sp, sptr, cfg, w, rc, skin):
    import torch
    from molecular_dynamics_amd import mdmp
    d = lambda a: torch.tensor(a, device="cuda")  # noqa: E731
    g = mdmp.build_neighbors_batched(d(pos), d(sp), d(sptr), rc, skin)
    torch.cuda.synchronize()
    return g


def test_batched_list_bit_exact():
    from oracle import neighbors as NB
    pos, sp, sptr = _batch(31)
    g = _gpu(pos, sp, sptr, None, None, 4.0, 1.0)
    rp, col = NB.csr_open_batched(pos, sptr, 4.0, 1.0)
    rev = NB.reverse_index(rp, col)
    ne = g.n_edges
    print(f"batched list: {len(sptr) - 1} structures, {len(pos)} atoms, {ne} edges", flush=True)
    assert g.L == 0.0 and g.perm is None
    assert np.array_equal(g.row_ptr.cpu().numpy(), rp)
    assert np.array_equal(g.col[:ne].cpu().numpy(), col)
    assert np.array_equal(g.rev[:ne].cpu().numpy(), rev)


@pytest.mark.parametrize("C,bf16,T", [(64, False, 2), (128, True, 3)])
def test_batched_energies_forces(C, bf16, T):
    import torch
    from molecular_dynamics_amd import inputs, mdmp
    from oracle import model as OM
    from oracle import neighbors as NB
    pos, sp, sptr = _batch(32 + C)
    cfg = inputs.ModelConfig(n_species=3, channels=C, lmax=2, n_bessel=8, heads=4, layers=T, cutoff=4.5,
                             feat_bf16=bf16)
    w = inputs.make_weights(cfg, np.random.SeedSequence(C).spawn(3)[2])
    g = _gpu(pos, sp, sptr, cfg, w, cfg.cutoff, 0.5)
    model = mdmp.Model(cfg, w)
    e_at = torch.empty(len(pos), dtype=torch.float32, device="cuda")
    E, F = mdmp.energy_forces(model, g, atom_energy=e_at)
    Eb = mdmp.structure_energies(e_at, torch.tensor(sptr, device="cuda")).cpu().numpy()
    torch.cuda.synchronize()
    F = F.cpu().numpy()
    e_at = e_at.cpu().numpy()
    rp, col = NB.csr_open_batched(pos, sptr, cfg.cutoff, 0.5)
    ref_E, ref_F, ref_at = [], [], []
    for b in range(len(sptr) - 1):
        a0, a1 = int(sptr[b]), int(sptr[b + 1])
        r = OM.energy(cfg, w, pos[a0:a1], sp[a0:a1], None, rp[a0:a1 + 1] - rp[a0], col[rp[a0]:rp[a1]] - a0)
        ref_E.append(r["E"])
        ref_F.append(r["F"])
        ref_at.append(r["E_atoms"])
    ref_E, ref_F, ref_at = np.array(ref_E), np.concatenate(ref_F), np.concatenate(ref_at)
    tol = 2e-2 if bf16 else 1e-4
    scale = np.abs(ref_at).sum()
    # per structure, the energy bar of the single-box tests: |dE_b| <= tol * sum_{i in b} |E_i|
    s_abs = np.add.reduceat(np.abs(ref_at), sptr[:-1])
    ee = (np.abs(Eb - ref_E) / s_abs).max()
    ae = np.abs(e_at - ref_at).max() / np.abs(ref_at).max()
    fe = force_error(F, ref_F)
    print(f"batched C={C} bf16={bf16}: structure-E err {ee:.2e}, atom-E err {ae:.2e}, force err {fe:.2e}, "
          f"total E {E:.6f} ref {ref_E.sum():.6f}", flush=True)
    assert ee <= tol and ae <= tol and fe <= tol
    assert abs(E - ref_E.sum()) <= tol * scale
    # the per-structure sums are the float64 sums of the atom energies, and sum to E
    assert np.allclose(Eb, np.add.reduceat(e_at.astype(np.float64), sptr[:-1]), rtol=1e-12, atol=1e-9)
    assert abs(Eb.sum() - E) <= 1e-9 * max(1.0, abs(E))


def test_batched_errors():
    import torch
    from molecular_dynamics_amd import mdmp
    pos, sp, sptr = _batch(33, n_struct=5)
    d = lambda a: torch.tensor(a, device="cuda")  # noqa: E731
    with pytest.raises(mdmp.MPError) as e:
        mdmp.build_neighbors_batched(d(pos), d(sp), d(sptr), 4.0, 1.0, capacity=3)
    assert e.value.code == mdmp.MP_ERR_CAPACITY
    with pytest.raises(mdmp.MPError) as e:
        mdmp.build_neighbors_batched(d(pos), d(sp), d(sptr), -1.0, 1.0)
    assert e.value.code == mdmp.MP_ERR_ARG
    torch.cuda.synchronize()
