"""Benchmark: neighbour build + energy + forces of the equivariant attention
potential on the 1,048,576-atom heterogeneous box (dense 5-species shell in
dilute solvent, cutoff 5 A, skin 1 A, 4 layers, 128 channels per irrep
l <= 2, bfloat16 features with float32 arithmetic), one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-md]
                    [--no-extra] [--md-steps M] [--md-cpu-steps S] [--calib-copy]

Prints one JSON line.  A step is one pass of the whole evaluation path over
the box: Hilbert sort + cell list + skin-padded radius graph, edge geometry,
4 layers forward, readout, the full backward pass and the force gather.
value = edge-messages/s = layers * active edges / mean step time (inputs
resident in HBM before the timed region).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edge-messages/s fwd+force, 4-layer l<=2 at 1M atoms; ns/day; % HBM/MFMA roof"
PEAK_VALU_FP32 = 157.3e12     # published fp32 vector peak (packed); non-packed issue is half of it
PEAK_HBM = 8.0e12


MODES = {0: "", 1: "_first", 2: "_last", 3: "_single"}


def layer_mode(t, T):
    """first layer: only paths with l1 = 0 carry nonzero inputs; last layer: only
    paths with l3 = 0 reach the energy (both restrictions are exact)."""
    return (1 if t == 0 else 0) | (2 if t == T - 1 else 0)


def tp_macs_mode(lmax, mode):
    s1 = s2 = 0
    for a in range(lmax + 1):
        for b in range(lmax + 1):
            for c in range(lmax + 1):
                if abs(a - b) <= c <= a + b and not (mode & 1 and a) and not (mode & 2 and c):
                    s1 += (2 * a + 1) * (2 * c + 1)
                    s2 += 2 * c + 1
    return s1, s2


def recv_bwd_flops_per_edge(cfg, mode):
    """Algorithmic VALU flops per active edge of the receiver-side backward:
    recompute the product (s1 + s2), dE/dw (s2), dE/dY via dE/dM_p (s1) and the
    value/logit gradients (3K) multiply-adds per channel, 2 flops each."""
    s1, s2 = tp_macs_mode(cfg.lmax, mode)
    K = (cfg.lmax + 1) ** 2
    return 2.0 * cfg.channels * (2 * s1 + 2 * s2 + 3 * K)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="shell1m")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-md", action="store_true")
    ap.add_argument("--md-steps", type=int, default=20)
    ap.add_argument("--cpu-radius", type=float, default=16.0)
    ap.add_argument("--md-cpu-steps", type=int, default=0,
                    help="also time the float64 oracle MD on the 4,096-atom salt replica for this many steps "
                         "(about a minute per step on 16 host cores; off by default)")
    ap.add_argument("--no-extra", action="store_true", help="skip the 262,144-atom salt box line")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; the measured value is "
              "one GPU's throughput on its share of the work", file=sys.stderr)
        sys.exit(2)

    import torch

    from molecular_dynamics_amd import inputs, mdmp, prof_summary

    if args.calib_copy:
        # a plain 1 GiB device-to-device copy, the scale for the HBM byte counters, and a
        # read-only sum over the same 1 GiB as a second calibration of the read counter
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        total = src.sum()
        torch.cuda.synchronize()
        del src, dst, total
        torch.cuda.empty_cache()

    t_gen = time.time()
    w = inputs.workload(args.workload)
    cfg, box = w.model, w.box
    print(f"[bench] workload {w.name}: {box.n} atoms, L={box.L:.3f}, generated in {time.time() - t_gen:.1f}s",
          file=sys.stderr, flush=True)
    pos = torch.tensor(box.pos, device="cuda")
    sp = torch.tensor(box.species, device="cuda")
    model = mdmp.Model(cfg, w.weights)
    g = mdmp.build_neighbors(pos, sp, box.L, cfg.cutoff, w.skin)
    cap = int(g.n_edges * 1.05) + 4096
    # fixed-capacity buffers reused by every step
    g = mdmp.build_neighbors(pos, sp, box.L, cfg.cutoff, w.skin, capacity=cap)
    ef = mdmp.EnergyForces(model, box.n, cap)
    forces = torch.empty(box.n, 3, dtype=torch.float32, device="cuda")
    e_at = torch.empty(box.n, dtype=torch.float32, device="cuda")

    def step():
        gg = mdmp.build_neighbors(pos, sp, box.L, cfg.cutoff, w.skin, capacity=cap)
        E, F = ef(gg, perm=gg.perm, forces=forces, atom_energy=e_at)
        return gg, E

    for _ in range(args.warmup):
        g, E = step()
    torch.cuda.synchronize()
    # active edges (r < r_cut) of this box
    r_act = int(ef_active_edges(g, cfg.cutoff))
    print(f"[bench] padded edges {g.n_edges}, active {r_act}", file=sys.stderr, flush=True)

    mdmp.profile_reset()
    mdmp.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        g, E = step()
        print(f"[bench] step {k + 1}/{args.steps}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mdmp.profile_enable(False)
    ms_step = wall * 1e3 / args.steps
    names = ["build_neighbors", "geometry", "forces"] + [k + m for k in ("edge_fwd", "edge_bwd_recv", "edge_bwd_send")
                                                        for m in MODES.values()]
    prof = {name: mdmp.profile_read(name) for name in names}
    prof = {k: v for k, v in prof.items() if v[1] > 0}
    energy = float(E.item())
    msgs = cfg.layers * r_act
    value = msgs / (ms_step * 1e-3)
    build_ms = prof["build_neighbors"][0] / max(1, prof["build_neighbors"][1])
    ef_ms = ms_step - build_ms

    # dominant kernel: receiver-side edge backward (VALU-bound tensor-product work),
    # all its launches of the timed steps: sum of algorithmic flops / sum of durations
    t_recv = sum(v[0] for k, v in prof.items() if k.startswith("edge_bwd_recv"))
    n_recv = sum(v[1] for k, v in prof.items() if k.startswith("edge_bwd_recv"))
    flops_recv = sum(recv_bwd_flops_per_edge(cfg, layer_mode(t, cfg.layers)) for t in range(cfg.layers)) * r_act
    flops_recv *= n_recv / cfg.layers
    roof = {"kernel": "k_edge_bwd_recv", "bound": "alu", "achieved": flops_recv / (t_recv * 1e-3) / 1e12,
            "peak": PEAK_VALU_FP32 / 1e12, "unit": "TFLOP/s", "launches": n_recv,
            "avg_ms": t_recv / max(1, n_recv)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary, if it
    # was taken on the current kernel sources
    tr = prof_summary.read_traffic(os.path.join(ROOT, "profiles", f"k_edge_bwd_recv_{w.name}_traffic.txt"))
    roof["traffic"] = tr[0] if tr and tr[1] == prof_summary.kernel_source_hash() else None
    kernels_ms = {k: round(v[0] / max(1, v[1]), 3) for k, v in prof.items()}
    # gather (edge geometry) and aggregation (force gather) passes over their mean measured
    # duration against the HBM peak: the method's byte count (80 B / 32 B per padded edge)
    # and, beside it, the bytes this design moves
    hbm = {"peak_GBps": prof_summary.HBM_PEAK_GBS}
    for name in ("geometry", "forces"):
        if name in prof:
            t = prof[name][0] / prof[name][1]
            alg = prof_summary.pass_bytes_algorithmic(name, box.n, g.n_edges)
            by = prof_summary.pass_bytes(name, box.n, g.n_edges, r_act, cfg.channels, cfg.lmax, cfg.feat_bf16)
            hbm[name] = {"kernels": list(prof_summary.PASS_KERNELS[name]), "ms": t, "bytes": alg,
                         "GBps": alg / t / 1e6, "frac": alg / t / 1e6 / prof_summary.HBM_PEAK_GBS,
                         "design_bytes": by, "design_GBps": by / t / 1e6,
                         "design_frac": by / t / 1e6 / prof_summary.HBM_PEAK_GBS}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "edge-messages/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.feat_bf16 else "fp32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {box.n} atoms, L={box.L:.3f} A, cutoff {cfg.cutoff} A, skin {w.skin} A, "
                               f"{cfg.layers} layers, C={cfg.channels}, lmax={cfg.lmax}, heads={cfg.heads}, "
                               f"{'bf16' if cfg.feat_bf16 else 'fp32'} features",
                   "atoms": box.n, "edges_padded": g.n_edges, "edges_active": r_act},
        "roofline": roof,
        "edge_messages_per_s_without_build": msgs / (ef_ms * 1e-3),
        "padded_edge_messages_per_s": cfg.layers * g.n_edges / (ms_step * 1e-3),
        "build_ms": build_ms,
        "energy_forces_ms": ef_ms,
        "kernel_avg_ms": kernels_ms,
        "hbm_passes": hbm,
        "energy_eV": energy,
    }
    if not args.no_md or not args.no_extra:
        del ef
        torch.cuda.empty_cache()
    if not args.no_extra:
        out["salt262k"] = other_box("salt262k", args.steps, args.warmup)
        out["mol16k"] = batched_rate(args.steps, args.warmup)
    if not args.no_md:
        out["md"] = md_rate(args.md_steps)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, g, args.cpu_radius)
    if args.md_cpu_steps > 0:
        out["md_cpu_baseline"] = md_cpu_baseline(args.md_cpu_steps)
    print(json.dumps(out))


def other_box(name, steps, warmup):
    """The same timed step (neighbour build + energy + forces) on another box."""
    import torch

    from molecular_dynamics_amd import inputs, mdmp
    w = inputs.workload(name)
    cfg, box = w.model, w.box
    pos = torch.tensor(box.pos, device="cuda")
    sp = torch.tensor(box.species, device="cuda")
    model = mdmp.Model(cfg, w.weights)
    g = mdmp.build_neighbors(pos, sp, box.L, cfg.cutoff, w.skin)
    cap = int(g.n_edges * 1.05) + 4096
    ef = mdmp.EnergyForces(model, box.n, cap)
    forces = torch.empty(box.n, 3, dtype=torch.float32, device="cuda")

    def step():
        gg = mdmp.build_neighbors(pos, sp, box.L, cfg.cutoff, w.skin, capacity=cap)
        ef(gg, perm=gg.perm, forces=forces)
        return gg

    for _ in range(max(1, warmup)):
        g = step()
    torch.cuda.synchronize()
    r_act = ef_active_edges(g, cfg.cutoff)
    t0 = time.perf_counter()
    for _ in range(steps):
        g = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del ef
    torch.cuda.empty_cache()
    return {"workload": f"{name}: {box.n} atoms, L={box.L:.3f} A, cutoff {cfg.cutoff} A, skin {w.skin} A, "
                        f"{cfg.layers} layers, C={cfg.channels}, lmax={cfg.lmax}, "
                        f"{'bf16' if cfg.feat_bf16 else 'fp32'} features",
            "edge_messages_per_s": cfg.layers * r_act / (ms * 1e-3), "ms_per_step": ms,
            "edges_active": r_act, "edges_padded": g.n_edges}


def batched_rate(steps, warmup):
    """structures/s on a batch of 16,384 open structures of 8-32 atoms (build + energy + forces +
    per-structure energies per step; the 1M-atom box's model, bf16 features)."""
    import torch

    from molecular_dynamics_amd import inputs, mdmp
    pos, sp, sptr, cfg, wts = inputs.molecule_batch("mol16k")
    d = lambda a: torch.tensor(a, device="cuda")  # noqa: E731
    pos_d, sp_d, sptr_d = d(pos), d(sp), d(sptr)
    model = mdmp.Model(cfg, wts)
    g = mdmp.build_neighbors_batched(pos_d, sp_d, sptr_d, cfg.cutoff, 0.0)
    cap = int(g.n_edges * 1.05) + 4096
    ef = mdmp.EnergyForces(model, len(pos), cap)
    e_at = torch.empty(len(pos), dtype=torch.float32, device="cuda")
    forces = torch.empty(len(pos), 3, dtype=torch.float32, device="cuda")
    eb = torch.empty(len(sptr) - 1, dtype=torch.float64, device="cuda")

    def step():
        gg = mdmp.build_neighbors_batched(pos_d, sp_d, sptr_d, cfg.cutoff, 0.0, capacity=cap)
        ef(gg, forces=forces, atom_energy=e_at)
        mdmp.structure_energies(e_at, sptr_d, out=eb)
        return gg

    for _ in range(max(warmup, 1)):
        g = step()
    torch.cuda.synchronize()
    n_act = ef_active_edges(g, cfg.cutoff)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps

    # 16 readout heads on the same encoder: every head's per-structure energies, and the
    # forces of the heads' weighted energy from one reverse pass
    R, C = 16, cfg.channels
    rng = np.random.default_rng(16)
    heads = mdmp.Heads(model, (rng.standard_normal((R, C, C)) / np.sqrt(C)).astype(np.float32),
                       (rng.standard_normal((R, C)) / np.sqrt(C)).astype(np.float32), np.full(R, 1.0 / R, np.float32))
    ebh = torch.empty(R, len(sptr) - 1, dtype=torch.float64, device="cuda")

    def step_heads():
        gg = mdmp.build_neighbors_batched(pos_d, sp_d, sptr_d, cfg.cutoff, 0.0, capacity=cap)
        _, _, _, e_h = mdmp.energy_forces_heads(model, heads, gg, ws=ef.ws)
        for k in range(R):
            mdmp.structure_energies(e_h[k], sptr_d, out=ebh[k])

    for _ in range(max(warmup, 1)):
        step_heads()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step_heads()
    torch.cuda.synchronize()
    dth = (time.perf_counter() - t0) / steps
    heads.close()
    return {"workload": f"mol16k: {len(sptr) - 1} open structures of 8-32 atoms ({len(pos)} atoms), cutoff "
                        f"{cfg.cutoff} A, {cfg.layers} layers, C={cfg.channels}, lmax={cfg.lmax}, bf16 features",
            "structures_per_s": (len(sptr) - 1) / dt, "ms_per_step": dt * 1e3,
            "edge_messages_per_s": cfg.layers * n_act / dt, "edges_active": n_act,
            "heads16_structures_per_s": (len(sptr) - 1) / dth, "heads16_ms_per_step": dth * 1e3}


def md_rate(steps, warm=4):
    """ns/day of velocity-Verlet NVE on the 131,072-atom salt solution (float32
    features, r_c 6 A, skin 1 A, dt 0.5 fs, Maxwell-Boltzmann 300 K start): mean
    wall time of `steps` steps after `warm` steps (the first build and graph capture
    are in the warm-up); rebuilds inside the timed steps are included."""
    import torch

    from molecular_dynamics_amd import inputs, mdmp
    w = inputs.workload("salt131k_md")
    box, cfg = w.box, w.model
    model = mdmp.Model(cfg, w.weights)
    md = mdmp.MD(model, box.n, box.L, w.skin, w.extra["dt_fs"], w.extra["masses"])
    md.set_state(torch.tensor(box.pos, device="cuda"), torch.tensor(w.extra["vel"], device="cuda"),
                 torch.tensor(box.species, device="cuda"))
    md.step(warm, e_log=False)
    s0 = md.state()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    log = md.step(steps, e_log=True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    s1 = md.state()
    md.close()
    e = log.sum(1)
    from molecular_dynamics_amd.md_run import drift_uev_per_atom_per_ps
    return {"workload": f"{w.name}: {box.n} atoms, L={box.L:.3f} A, cutoff {cfg.cutoff} A, skin {w.skin} A, "
                        f"{cfg.layers} layers, C={cfg.channels}, lmax={cfg.lmax}, float32 features, "
                        f"dt {w.extra['dt_fs']} fs",
            "ns_per_day": w.extra["dt_fs"] * 1e-6 * 86400.0 / dt, "ms_per_step": dt * 1e3, "steps": steps,
            "warmup": warm, "rebuilds_in_timed": s1["n_rebuilds"] - s0["n_rebuilds"],
            "captures_total": s1["n_captures"], "max_abs_dE_per_atom_eV": float(np.abs(e - e[0]).max() / box.n),
            "drift_uev_per_atom_per_ps": drift_uev_per_atom_per_ps(e, box.n, w.extra["dt_fs"]),
            "drift_stderr_uev_per_atom_per_ps": drift_stderr(e, box.n, w.extra["dt_fs"]),
            "drift_window_fs": steps * w.extra["dt_fs"],
            "drift_note": "least-squares slope over this short window: it follows the integrator's energy "
                          "oscillation (dt^2 error) rather than a long-run drift; --md-steps 2000 runs the "
                          "configured trajectory",
            "min_pair_A": s1["min_pair"]}


def drift_stderr(e, n, dt_fs):
    """standard error of the least-squares slope of E/N against t (micro-eV per atom per ps):
    over a short window the slope is mostly the scatter of the per-step energies"""
    t = np.arange(len(e)) * dt_fs * 1e-3
    y = np.asarray(e, np.float64) / n
    if len(e) < 3:
        return None
    A = np.vstack([t, np.ones_like(t)]).T
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    resid = y - A @ coef
    s2 = float(resid @ resid) / (len(e) - 2)
    return float(np.sqrt(s2 / ((t - t.mean()) ** 2).sum()) * 1e6)


def md_cpu_baseline(steps):
    """ns/day of the oracle's float64 velocity-Verlet MD (forces by autograd, evaluated over
    chunks of rows) on the 4,096-atom salt replica of the MD box, on the host cores: the
    wall time of `steps` steps after the first force evaluation."""
    import torch

    from molecular_dynamics_amd import inputs
    from oracle import md as OMD
    n_thr = len(os.sched_getaffinity(0))
    torch.set_num_threads(n_thr)
    w = inputs.workload("salt4k_md")
    t0 = time.perf_counter()
    OMD.run_nve(w.model, w.weights, w.box.pos, w.extra["vel"], w.box.species, w.extra["masses"], w.box.L, w.skin,
                w.extra["dt_fs"], 0, chunk_edges=1024)
    t_first = time.perf_counter() - t0
    t0 = time.perf_counter()
    r = OMD.run_nve(w.model, w.weights, w.box.pos, w.extra["vel"], w.box.species, w.extra["masses"], w.box.L,
                    w.skin, w.extra["dt_fs"], steps, chunk_edges=1024)
    per_step = (time.perf_counter() - t0 - t_first) / steps
    return {"value": w.extra["dt_fs"] * 1e-6 * 86400.0 / per_step, "unit": "ns/day", "cores": n_thr, "cpu": cpu_model(),
            "kind": "oracle", "s_per_step": per_step,
            "sample": f"{w.name}: {w.box.n} atoms, the model of the MD box, {steps} float64 velocity-Verlet steps "
                      f"after the first force evaluation ({t_first:.0f} s)", "E_pot_eV": [float(x) for x in r["E_pot"]]}


def ef_active_edges(g, rc):
    import torch
    n = g.n
    rp = g.row_ptr.long()
    col = g.col[:g.n_edges].long()
    row = torch.repeat_interleave(torch.arange(n, device="cuda"), rp[1:] - rp[:-1])
    d = g.pos[col] - g.pos[row]
    if g.L > 0:  # periodic box; L = 0 marks an open boundary
        d = d - g.L * torch.round(d / g.L)
    r = torch.linalg.norm(d, dim=1)
    return int((r < rc).sum().item())


def cpu_model():
    """the host CPU's model name (/proc/cpuinfo)"""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, g, radius):
    """The oracle (float64, PyTorch CPU) on an open cluster cut from the same box:
    atoms within `radius` of the box centre, same model and weights."""
    import torch

    from oracle import model as OM
    n_thr = len(os.sched_getaffinity(0))
    torch.set_num_threads(n_thr)
    P = w.box.pos.astype(np.float64)
    ctr = np.full(3, w.box.L / 2)
    sel = np.nonzero(np.linalg.norm(P - ctr, axis=1) < radius)[0]
    Pc = P[sel]
    sp = w.box.species[sel]
    R = w.model.cutoff + w.skin
    d = np.linalg.norm(Pc[:, None] - Pc[None], axis=-1)
    np.fill_diagonal(d, np.inf)
    src, dst = np.nonzero(d < R)
    rp = np.concatenate([[0], np.cumsum(np.bincount(src, minlength=sel.size))]).astype(np.int32)
    t0 = time.perf_counter()
    out = OM.energy(w.model, w.weights, Pc, sp, None, rp, dst.astype(np.int32))
    dt = time.perf_counter() - t0
    msgs = w.model.layers * out["n_active"]
    return {"value": msgs / dt, "unit": "edge-messages/s", "cores": n_thr, "cpu": cpu_model(), "kind": "oracle",
            "sample": f"open cluster of the {sel.size} atoms within {radius} A of the box centre "
                      f"({out['n_active']} active edges, {w.model.layers} layers), float64 energy + forces, "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
