"""Single-GPU ablations of two claims of the Tessera abstract ("Ab Initio Accuracy
Beyond the Cutoff", Abstract):

* atom order: the space-filling curve against Morton order and against no order
  at all (the caller's order), measured as the neighbour-build time and the time of
  each kernel group of one energy + forces evaluation (the abstract compares the
  growth of the neighbour-search cost of its curve with Morton order);
* graph reuse: MD steps replaying the captured hipGraphs against the same kernels
  enqueued one by one (the abstract reports the full-step time cut by graph reuse).

Prints one JSON line.

    python -m molecular_dynamics_amd.ablation [--workload shell1m] [--orders hilbert,morton,input]
        [--steps 2] [--md-steps 10] [--no-md]

Energy and forces do not depend on the order (checked here against the first order,
and bit for bit for eager vs graph MD in the GPU tests); only the time does.
"""
import argparse
import json
import sys
import time

import numpy as np

KERNEL_GROUPS = ["build_neighbors", "geometry", "forces"] + [
    k + m for k in ("edge_fwd", "edge_bwd_recv", "edge_bwd_send") for m in ("", "_first", "_last", "_single")]


def active_edges(g, rc):
    import torch
    rp = g.row_ptr.long()
    col = g.col[:g.n_edges].long()
    row = torch.repeat_interleave(torch.arange(g.n, device="cuda"), rp[1:] - rp[:-1])
    d = g.pos[col] - g.pos[row]
    if g.L > 0:  # periodic box; L = 0 marks an open boundary
        d = d - g.L * torch.round(d / g.L)
    return int((torch.linalg.norm(d, dim=1) < rc).sum().item())


def order_run(w, order, steps):
    """build + energy/forces in the given atom order: mean times over `steps` after one warm-up"""
    import torch

    from molecular_dynamics_amd import mdmp
    box, cfg = w.box, w.model
    pos = torch.tensor(box.pos, device="cuda")
    sp = torch.tensor(box.species, device="cuda")
    model = mdmp.Model(cfg, w.weights)
    g = mdmp.build_neighbors(pos, sp, box.L, cfg.cutoff, w.skin, order=order)
    cap = int(g.n_edges * 1.05) + 4096
    ef = mdmp.EnergyForces(model, box.n, cap)
    forces = torch.empty(box.n, 3, dtype=torch.float32, device="cuda")

    def step():
        gg = mdmp.build_neighbors(pos, sp, box.L, cfg.cutoff, w.skin, capacity=cap, order=order)
        E, _ = ef(gg, perm=gg.perm, forces=forces)
        return gg, E

    g, E = step()
    torch.cuda.synchronize()
    n_act = active_edges(g, cfg.cutoff)
    mdmp.profile_reset()
    mdmp.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        g, E = step()
        print(f"[ablation] {order} step {k + 1}/{steps}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    mdmp.profile_enable(False)
    prof = {k: mdmp.profile_read(k) for k in KERNEL_GROUPS}
    kernels = {k: round(v[0] / v[1], 3) for k, v in prof.items() if v[1] > 0}
    out = {"ms_per_step": ms, "build_ms": kernels.get("build_neighbors"),
           "edge_messages_per_s": cfg.layers * n_act / (ms * 1e-3), "kernel_avg_ms": kernels,
           "energy_eV": float(E.item()), "forces_input_order": forces.cpu().numpy()}
    del ef
    torch.cuda.empty_cache()
    return out


def md_run(name, steps, graphs, warm=2):
    import torch

    from molecular_dynamics_amd import inputs, mdmp
    w = inputs.workload(name)
    box, cfg = w.box, w.model
    model = mdmp.Model(cfg, w.weights)
    md = mdmp.MD(model, box.n, box.L, w.skin, w.extra["dt_fs"], w.extra["masses"])
    md.use_graphs(graphs)
    md.set_state(torch.tensor(box.pos, device="cuda"), torch.tensor(w.extra["vel"], device="cuda"),
                 torch.tensor(box.species, device="cuda"))
    md.step(warm, e_log=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    md.step(steps, e_log=False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    st = md.state()
    md.close()
    return {"ms_per_step": ms, "ns_per_day": w.extra["dt_fs"] * 1e-6 * 86400.0 / (ms * 1e-3),
            "rebuilds": st["n_rebuilds"], "captures": st["n_captures"]}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="shell1m")
    ap.add_argument("--orders", default="hilbert,morton,input")
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--md-workload", default="salt131k_md")
    ap.add_argument("--md-steps", type=int, default=10)
    ap.add_argument("--no-md", action="store_true")
    a = ap.parse_args(argv)

    import torch

    from molecular_dynamics_amd import inputs
    if not torch.cuda.is_available():
        raise SystemExit("ablation: needs a GPU")
    w = inputs.workload(a.workload)
    res = {"workload": f"{w.name}: {w.box.n} atoms, L={w.box.L:.3f} A, cutoff {w.model.cutoff} A, skin {w.skin} A, "
                       f"{w.model.layers} layers, C={w.model.channels}, "
                       f"{'bf16' if w.model.feat_bf16 else 'float32'} features", "orders": {}}
    ref = None
    for order in a.orders.split(","):
        r = order_run(w, order, a.steps)
        F = r.pop("forces_input_order")
        if ref is None:
            ref = (r["energy_eV"], F)
        else:
            r["rel_energy_diff_vs_first"] = abs(r["energy_eV"] - ref[0]) / abs(ref[0])
            r["force_diff_vs_first"] = float(np.linalg.norm(F - ref[1], axis=1).max()
                                             / np.linalg.norm(ref[1], axis=1).max())
        res["orders"][order] = r
    if not a.no_md:
        res["md"] = {"workload": a.md_workload, "steps": a.md_steps,
                     "graphs": md_run(a.md_workload, a.md_steps, True),
                     "eager": md_run(a.md_workload, a.md_steps, False)}
        res["md"]["eager_over_graph"] = res["md"]["eager"]["ms_per_step"] / res["md"]["graphs"]["ms_per_step"]
    print(json.dumps(res))


if __name__ == "__main__":
    sys.exit(main())
