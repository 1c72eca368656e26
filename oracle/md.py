"""NVE (and Langevin NVT) molecular dynamics with skin-triggered neighbour rebuilds (oracle).

"Ab Initio Accuracy Beyond the Cutoff" (Abstract): molecular dynamics
integrates trajectories from atomic forces; a conservative skin keeps the
neighbour graph valid between rebuilds, and energy drift in NVE is the
fidelity measure ("Unlocking Tensor Core Performance", section "Choosing a
Precision Strategy").  The integrator is textbook velocity Verlet:

  1  v += (dt/2) a        2  x += dt v
  3  if max_i |x_i - x_i^ref| > skin/2: wrap, re-sort along the Hilbert curve,
     rebuild the list at r_cut + skin, x^ref = x
  4  a = F(x) / m          5  v += (dt/2) a

Units: A, fs, amu, eV.  a [A/fs^2] = F [eV/A] / m [amu] * 9.64853321e-3;
KE [eV] = 1/2 sum m v^2 * 103.642696.  State is float64 here (the neighbour
decision at a rebuild looks at its float32 image).
"""
import numpy as np

from . import model, neighbors

ACC = 9.64853321e-3         # (eV/A)/amu in A/fs^2
KE_UNIT = 103.642696        # amu (A/fs)^2 in eV


def _rebuild(st, cfg, L, skin):
    """Wrap (float64 state), re-sort along the Hilbert curve, rebuild the list.

    The sort key and the pair decision use the float32 image of the positions,
    exactly as a float32 state would; the float64 state itself is kept."""
    Ld = float(np.float32(L))
    x = st["x"] - Ld * np.floor(st["x"] / Ld)
    x = np.where(x < 0, x + Ld, np.where(x >= Ld, x - Ld, x))
    nb = neighbors.build_neighbors(x.astype(np.float32), L, cfg.cutoff, skin, method="auto")
    perm = nb["perm"]
    for k in ("v", "ids", "species", "mass"):
        st[k] = st[k][perm]
    st["x"] = x[perm]
    st["row_ptr"], st["col"] = nb["row_ptr"], nb["col"]
    st["x_ref"] = st["x"].copy()
    st["n_rebuilds"] += 1


def _forces(st, cfg, weights, L):
    if st.get("chunk_edges"):
        # the same energy and forces, evaluated over chunks of rows (model.energy_forces_chunked)
        import torch
        prm = st.setdefault("prm", model.Params(cfg, weights))
        cgs = st.setdefault("cgs", model.cg_table(cfg.lmax))
        Ld = float(np.float32(L))
        X = torch.tensor(st["x"])
        row, col = model._active_edges(X, Ld, st["row_ptr"], st["col"], cfg.cutoff)
        return model.energy_forces_chunked(cfg, prm, cgs, X, st["species"], Ld, row, col,
                                           max_edges=st["chunk_edges"])
    out = model.energy(cfg, weights, st["x"], st["species"], L, st["row_ptr"], st["col"], forces=True)
    return out["E"], out["F"]


def run_nve(cfg, weights, pos, vel, species, masses_per_species, L, skin, dt, n_steps, rebuild=True,
            chunk_edges=None):
    """Returns dict(x, v, ids (input index per slot), E_kin [n+1], E_pot [n+1], n_rebuilds).
    chunk_edges: evaluate the forces over chunks of about that many edges (for boxes whose
    whole-box autograd graph would not fit in memory)."""
    n = pos.shape[0]
    st = {"x": np.asarray(pos, np.float64).copy(), "v": np.asarray(vel, np.float64).copy(),
          "ids": np.arange(n, dtype=np.int32), "species": np.asarray(species, np.int32).copy(),
          "n_rebuilds": -1, "chunk_edges": chunk_edges}
    st["mass"] = np.asarray(masses_per_species, np.float64)[st["species"]]
    _rebuild(st, cfg, L, skin)
    epot, f = _forces(st, cfg, weights, L)
    acc = f / st["mass"][:, None] * ACC
    ek = [0.5 * (st["mass"][:, None] * st["v"] ** 2).sum() * KE_UNIT]
    ep = [epot]
    for _ in range(n_steps):
        st["v"] += 0.5 * dt * acc
        st["x"] += dt * st["v"]
        if rebuild and np.sqrt(((st["x"] - st["x_ref"]) ** 2).sum(1)).max() > 0.5 * skin:
            _rebuild(st, cfg, L, skin)
        epot, f = _forces(st, cfg, weights, L)
        acc = f / st["mass"][:, None] * ACC
        st["v"] += 0.5 * dt * acc
        ek.append(0.5 * (st["mass"][:, None] * st["v"] ** 2).sum() * KE_UNIT)
        ep.append(epot)
    return {"x": st["x"], "v": st["v"], "ids": st["ids"], "species": st["species"],
            "E_kin": np.array(ek), "E_pot": np.array(ep), "n_rebuilds": st["n_rebuilds"]}


KB = 8.617333262e-5          # Boltzmann constant, eV/K


def run_nvt_baoab(cfg, weights, pos, vel, species, masses_per_species, L, skin, dt, n_steps, temperature, gamma_ps,
                  noise, rebuild=True):
    """Langevin dynamics by the BAOAB splitting (Leimkuhler & Matthews, "Rational construction of
    stochastic numerical methods for molecular sampling", Appl. Math. Res. Express 2013).  The
    Tessera abstract runs its capsid in NVT without naming the thermostat; this is the plain reading.
    One step:

      B  v += (dt/2) a          A  x += (dt/2) v
      O  v = c1 v + sqrt((1 - c1^2) k_B T / m) xi,   c1 = exp(-gamma dt)   (exact Ornstein-Uhlenbeck step)
      A  x += (dt/2) v          rebuild check as in run_nve
      a = F(x) / m              B  v += (dt/2) a

    noise [n_steps][n][3]: the standard normal deviates xi, indexed by input atom.  gamma in 1/ps,
    dt in fs, T in K.  Returns what run_nve returns."""
    n = pos.shape[0]
    st = {"x": np.asarray(pos, np.float64).copy(), "v": np.asarray(vel, np.float64).copy(),
          "ids": np.arange(n, dtype=np.int32), "species": np.asarray(species, np.int32).copy(),
          "n_rebuilds": -1}
    st["mass"] = np.asarray(masses_per_species, np.float64)[st["species"]]
    _rebuild(st, cfg, L, skin)
    epot, f = _forces(st, cfg, weights, L)
    acc = f / st["mass"][:, None] * ACC
    c1 = np.exp(-gamma_ps * 1e-3 * dt)
    ek = [0.5 * (st["mass"][:, None] * st["v"] ** 2).sum() * KE_UNIT]
    ep = [epot]
    for s in range(n_steps):
        sig = np.sqrt((1.0 - c1 * c1) * KB * temperature * ACC / st["mass"])
        st["v"] += 0.5 * dt * acc
        st["x"] += 0.5 * dt * st["v"]
        st["v"] = c1 * st["v"] + sig[:, None] * np.asarray(noise[s], np.float64)[st["ids"]]
        st["x"] += 0.5 * dt * st["v"]
        if rebuild and np.sqrt(((st["x"] - st["x_ref"]) ** 2).sum(1)).max() > 0.5 * skin:
            _rebuild(st, cfg, L, skin)
        epot, f = _forces(st, cfg, weights, L)
        acc = f / st["mass"][:, None] * ACC
        st["v"] += 0.5 * dt * acc
        ek.append(0.5 * (st["mass"][:, None] * st["v"] ** 2).sum() * KE_UNIT)
        ep.append(epot)
    return {"x": st["x"], "v": st["v"], "ids": st["ids"], "species": st["species"],
            "E_kin": np.array(ek), "E_pot": np.array(ep), "n_rebuilds": st["n_rebuilds"]}


def drift_per_atom_per_ps(e_tot, n_atoms, dt_fs):
    """Least-squares slope of E_tot/N against time, in micro-eV per atom per ps."""
    t_ps = np.arange(e_tot.size) * dt_fs * 1e-3
    slope = np.polyfit(t_ps, np.asarray(e_tot) / n_atoms, 1)[0]
    return slope * 1e6
