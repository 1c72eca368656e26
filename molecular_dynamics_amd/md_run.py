"""NVE (or Langevin NVT) molecular dynamics on a named synthetic workload with the GPU library.

    python -m molecular_dynamics_amd.md_run --workload salt131k_md --steps 400 [--warmup 4] [--log FILE]
        [--nvt TEMPERATURE_K GAMMA_PER_PS] [--seed S]

Prints one JSON line: ns/day (mean wall time of the steps after the warm-up,
rebuilds included), energy drift as the least-squares slope of (KE + PE) / N
against time in micro-eV per atom per picosecond, max |E(t) - E(0)| / N, the
rebuild and graph-capture counts and the minimum pair distance seen at rebuilds.
Velocity Verlet with the skin/2 rebuild rule, hipGraph replay between rebuilds
("Ab Initio Accuracy Beyond the Cutoff", Abstract: NVE with a conservative skin;
energy drift as the fidelity measure of "Unlocking Tensor Core Performance",
section "Choosing a Precision Strategy").  With --nvt the BAOAB Langevin thermostat runs
(the abstract's capsid runs NVT with an unnamed thermostat); its standard normals are drawn
on the GPU by torch from the seed, and the mean kinetic temperature of the timed steps is
reported.  For water boxes the stability monitor of the abstract (no broken bonds, no
anomalously close pairs) is reported as the largest O-H distance and the number of O-H
pairs beyond 1.5 A at the end, next to the minimum pair distance.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def drift_uev_per_atom_per_ps(e_tot, n_atoms, dt_fs):
    """Least-squares slope of e_tot / n_atoms (eV) over time, in micro-eV per atom per ps."""
    t_ps = np.arange(len(e_tot)) * dt_fs * 1e-3
    if len(e_tot) < 2:
        return 0.0
    slope = np.polyfit(t_ps, np.asarray(e_tot, np.float64) / n_atoms, 1)[0]
    return float(slope * 1e6)


KB = 8.617333262e-5  # eV/K


def bond_monitor(box, pos):
    """largest O-H distance (minimum image) of the water molecules and the count beyond 1.5 A"""
    nw = box.meta.get("n_water", 0)
    if not nw:
        return {}
    w0 = 2 * box.meta.get("n_pair", 0)
    x = np.asarray(pos, np.float64)[w0:w0 + 3 * nw].reshape(nw, 3, 3)
    L = float(box.L)
    d = x[:, 1:, :] - x[:, :1, :]
    d -= L * np.round(d / L)
    r = np.linalg.norm(d, axis=2)
    return {"max_OH_A": float(r.max()), "OH_beyond_1p5A": int((r > 1.5).sum()), "OH_bonds": int(r.size)}


def run(workload, steps, warmup, chunk, log_path=None, nvt=None, seed=0):
    import torch

    from molecular_dynamics_amd import inputs, mdmp
    w = inputs.workload(workload)
    if "dt_fs" not in w.extra:
        raise SystemExit(f"{workload} has no MD settings")
    box, cfg = w.box, w.model
    dt = w.extra["dt_fs"]
    model = mdmp.Model(cfg, w.weights)
    md = mdmp.MD(model, box.n, box.L, w.skin, dt, w.extra["masses"])
    if nvt:
        md.set_langevin(nvt[0], nvt[1])
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)

        def advance(k):
            return md.step_nvt(torch.randn(k, box.n, 3, generator=gen, device="cuda"), e_log=True)
    else:
        def advance(k):
            return md.step(k, e_log=True)
    md.set_state(torch.tensor(box.pos, device="cuda"), torch.tensor(w.extra["vel"], device="cuda"),
                 torch.tensor(box.species, device="cuda"))
    t0 = time.perf_counter()
    logs = [advance(warmup)] if warmup else []
    torch.cuda.synchronize()
    t_warm = time.perf_counter() - t0
    s0 = md.state()
    t0 = time.perf_counter()
    done = 0
    while done < steps:
        k = min(chunk, steps - done)
        logs.append(advance(k))
        done += k
        print(f"[md] {done}/{steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s1 = md.state()
    md.close()
    log = np.concatenate(logs)
    e = log.sum(1)
    e_run = e[warmup:]
    if log_path:
        np.savetxt(log_path, log, header="kinetic_eV potential_eV (one row per step)")
    ms = wall * 1e3 / steps
    out = {"ensemble": f"NVT Langevin BAOAB {nvt[0]} K, gamma {nvt[1]}/ps" if nvt else "NVE"}
    if nvt:
        out["mean_kinetic_temperature_K"] = float(log[warmup:, 0].mean() / (1.5 * box.n * KB))
    out.update(bond_monitor(box, s1["pos"]))
    return {**out, "workload": w.name, "atoms": box.n, "dt_fs": dt, "steps": steps, "warmup_steps": warmup,
            "warmup_s": t_warm, "ms_per_step": ms, "ns_per_day": dt * 1e-6 * 86400.0 / (ms * 1e-3),
            "drift_uev_per_atom_per_ps": drift_uev_per_atom_per_ps(e_run, box.n, dt),
            "max_abs_dE_per_atom_eV": float(np.abs(e_run - e_run[0]).max() / box.n),
            "rebuilds": s1["n_rebuilds"], "rebuilds_timed": s1["n_rebuilds"] - s0["n_rebuilds"],
            "captures": s1["n_captures"], "min_pair_A": s1["min_pair"],
            "e0_eV": float(e[0]), "kinetic0_eV": float(log[0, 0])}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="salt131k_md")
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--chunk", type=int, default=50, help="steps per mp_md_step call (progress granularity)")
    ap.add_argument("--log", default=None, help="write the per-step (KE, PE) log to this file")
    ap.add_argument("--nvt", type=float, nargs=2, metavar=("TEMPERATURE_K", "GAMMA_PER_PS"), default=None)
    ap.add_argument("--seed", type=int, default=0, help="seed of the thermostat's normal deviates")
    a = ap.parse_args()
    print(json.dumps(run(a.workload, a.steps, a.warmup, a.chunk, a.log, a.nvt, a.seed)))


if __name__ == "__main__":
    main()
