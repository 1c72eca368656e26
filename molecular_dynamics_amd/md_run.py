"""NVE (or Langevin NVT) molecular dynamics on a named synthetic workload with the GPU library.

    python -m molecular_dynamics_amd.md_run --workload salt131k_md --steps 400 [--warmup 4] [--log FILE]
        [--nvt TEMPERATURE_K GAMMA_PER_PS] [--seed S] [--save STATE.npz] [--resume STATE.npz]

--save writes the state after the run (positions and velocities in input order, the
per-step energy log, the timed steps and wall time, counters); --resume continues such a
run from its state (the list is rebuilt and the graph captured when it starts), and the
statistics then cover the whole trajectory, every part of it together.

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
pairs beyond 1.5 A at the end, next to the minimum pair distance; --monitor-every records
them (and the kinetic temperature) along the run.  A non-finite energy or force stops the
run (MP_ERR_NUMERIC), and the record says where.
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


def run(workload, steps, warmup, chunk, log_path=None, nvt=None, seed=0, save=None, resume=None, monitor_every=0):
    import torch

    from molecular_dynamics_amd import inputs, mdmp
    w = inputs.workload(workload)
    if "dt_fs" not in w.extra:
        raise SystemExit(f"{workload} has no MD settings")
    box, cfg = w.box, w.model
    dt = w.extra["dt_fs"]
    prev = dict(np.load(resume)) if resume else None
    if prev is not None and (str(prev["workload"]) != w.name or int(prev["nvt"]) != bool(nvt)):
        raise SystemExit(f"{resume} is a state of another run")
    model = mdmp.Model(cfg, w.weights)
    md = mdmp.MD(model, box.n, box.L, w.skin, dt, w.extra["masses"])
    if nvt:
        md.set_langevin(nvt[0], nvt[1])
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed + (int(prev["steps_done"]) if prev is not None else 0))

        def advance(k):
            return md.step_nvt(torch.randn(k, box.n, 3, generator=gen, device="cuda"), e_log=True)
    else:
        def advance(k):
            return md.step(k, e_log=True)
    pos0 = prev["pos"] if prev is not None else box.pos
    vel0 = prev["vel"] if prev is not None else w.extra["vel"]
    md.set_state(torch.tensor(pos0, device="cuda"), torch.tensor(vel0, device="cuda"),
                 torch.tensor(box.species, device="cuda"))
    t0 = time.perf_counter()
    logs = [advance(warmup)] if warmup else []
    torch.cuda.synchronize()
    t_warm = time.perf_counter() - t0
    s0 = md.state()
    t0 = time.perf_counter()
    done = 0
    monitors, stopped = [], None
    while done < steps:
        k = min(chunk, steps - done)
        try:
            logs.append(advance(k))
        except mdmp.MPError as err:
            if err.code != mdmp.MP_ERR_NUMERIC:
                raise
            stopped = {"at_step": warmup + done, "error": str(err)}  # within the last chunk
            print(f"[md] stopped: {err}", file=sys.stderr, flush=True)
            break
        done += k
        print(f"[md] {done}/{steps} steps, {time.perf_counter() - t0:.0f} s", file=sys.stderr, flush=True)
        if monitor_every and done % monitor_every == 0:
            st = md.state()
            mon = {"step": warmup + done, "min_pair_A": st["min_pair"],
                   "temperature_K": float(logs[-1][-1, 0] / (1.5 * box.n * KB))}
            mon.update(bond_monitor(box, st["pos"]))
            monitors.append(mon)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steps = done
    s1 = md.state()
    md.close()
    log = np.concatenate(logs) if logs else np.zeros((0, 2))
    # the whole trajectory: the resumed run's log first, then this part's steps (one row per step,
    # the energies after that step)
    full = np.concatenate([prev["log"], log]) if prev is not None else log
    timed_steps = steps + (int(prev["timed_steps"]) if prev is not None else 0)
    timed_wall = wall + (float(prev["timed_wall_s"]) if prev is not None else 0.0)
    rebuilds = s1["n_rebuilds"] + (int(prev["rebuilds"]) if prev is not None else 0)
    captures = s1["n_captures"] + (int(prev["captures"]) if prev is not None else 0)
    min_pair = min(s1["min_pair"], float(prev["min_pair"])) if prev is not None else s1["min_pair"]
    parts = (int(prev["parts"]) if prev is not None else 0) + 1
    if save:
        np.savez(save, workload=w.name, nvt=bool(nvt), pos=s1["pos"], vel=s1["vel"], log=full,
                 steps_done=len(full), timed_steps=timed_steps, timed_wall_s=timed_wall, rebuilds=rebuilds,
                 captures=captures, min_pair=min_pair, parts=parts)
    if log_path:
        np.savetxt(log_path, full, header="kinetic_eV potential_eV (one row per step)")
    e = full.sum(1)
    ms = timed_wall * 1e3 / timed_steps
    out = {"ensemble": f"NVT Langevin BAOAB {nvt[0]} K, gamma {nvt[1]}/ps" if nvt else "NVE"}
    if nvt:
        out["mean_kinetic_temperature_K"] = float(full[:, 0].mean() / (1.5 * box.n * KB))
    out.update(bond_monitor(box, s1["pos"]))
    return {**out, "workload": w.name, "atoms": box.n, "dt_fs": dt, "steps_total": len(full),
            "parts": parts,
            "steps": steps, "warmup_steps": warmup, "warmup_s": t_warm, "timed_steps": timed_steps,
            "ms_per_step": ms, "ns_per_day": dt * 1e-6 * 86400.0 / (ms * 1e-3),
            "drift_uev_per_atom_per_ps": drift_uev_per_atom_per_ps(e, box.n, dt),
            "max_abs_dE_per_atom_eV": float(np.abs(e - e[0]).max() / box.n),
            "rebuilds": rebuilds, "rebuilds_this_part_timed": s1["n_rebuilds"] - s0["n_rebuilds"],
            "captures": captures, "min_pair_A": min_pair, "e0_eV": float(e[0]), "kinetic0_eV": float(full[0, 0]),
            **({"monitors": monitors} if monitor_every else {}), **({"stopped": stopped} if stopped else {})}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="salt131k_md")
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--chunk", type=int, default=50, help="steps per mp_md_step call (progress granularity)")
    ap.add_argument("--log", default=None, help="write the per-step (KE, PE) log to this file")
    ap.add_argument("--nvt", type=float, nargs=2, metavar=("TEMPERATURE_K", "GAMMA_PER_PS"), default=None)
    ap.add_argument("--seed", type=int, default=0, help="seed of the thermostat's normal deviates")
    ap.add_argument("--save", default=None, help="write the final state (.npz) for --resume")
    ap.add_argument("--resume", default=None, help="continue the run saved in this state file")
    ap.add_argument("--monitor-every", type=int, default=0,
                    help="every this many steps (a multiple of --chunk): minimum pair distance, O-H monitor, "
                         "kinetic temperature")
    a = ap.parse_args()
    print(json.dumps(run(a.workload, a.steps, a.warmup, a.chunk, a.log, a.nvt, a.seed, a.save, a.resume,
                         a.monitor_every)))


if __name__ == "__main__":
    main()
