"""Short text summaries of rocprofv3 output (kernel statistics and HBM byte counters).

    python -m molecular_dynamics_amd.prof_summary stats  KERNEL_STATS_CSV --cmd "..." [--top 24]
    python -m molecular_dynamics_amd.prof_summary traffic FETCH_CSV WRITE_CSV --kernel k_edge_bwd_recv --cmd "..."
    python -m molecular_dynamics_amd.prof_summary hbm FETCH_CSV WRITE_CSV KERNEL_STATS_CSV --cmd "..." \
        --atoms N --edges-padded EP --edges-active EA --channels C --lmax L [--bf16]
    python -m molecular_dynamics_amd.prof_summary mfma PMC_CSV KERNEL_STATS_CSV --cmd "..."
    python -m molecular_dynamics_amd.prof_summary l2 LABEL=PMC_CSV [LABEL=PMC_CSV ...] --cmd "..."

`stats` lists the kernels of a `rocprofv3 --kernel-trace --stats --output-format csv`
run by total time and aggregates every instantiation of the named edge kernels.
`traffic` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a program that
first copies 1 GiB device-to-device: the counters of that copy (2^30 bytes read and
written) give the scale from counter units to bytes, which is then applied to every
dispatch of the named kernel.  The result records a hash of the kernel sources so
that a reader can tell whether the counters still describe the current kernels.
`hbm` tabulates, for the memory-bound kernels, the counter bytes per launch and the
bytes each kernel has to move in this design (formulas in DESIGN_BYTES), both as GB/s
over the kernel's mean duration and as a fraction of the 8 TB/s HBM peak.  `mfma` reads
a `--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32
SQ_BUSY_CYCLES GRBM_GUI_ACTIVE` run: matrix-core busy fraction = busy cycles summed over
the 1,024 SIMDs / (GUI-active cycles of one XCD x 1,024), and the MFMA flops (512 per
MOPS unit) over the kernel's mean duration against the bf16 (2.5 PFLOP/s) and f32
(157.3 TFLOP/s) dense peaks.  `l2` compares `--pmc TCC_HIT_sum TCC_MISS_sum` runs of the
same program under different labels (e.g. atom orders): L2 hit rate and misses per kernel.
"""
import argparse
import csv
import hashlib
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
# the kernels' sources and the build script (whose flags also shape the kernels' code)
KERNEL_SOURCES = ["csrc/model.hip", "csrc/model.hpp", "csrc/kernels.hpp", "csrc/cg_real.hpp", "csrc/common.hpp",
                  "build.py"]
COPY_BYTES = 1 << 30
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFS = {"bf16": 2500.0, "f32": 157.3}
N_SIMD, N_XCD = 1024, 8

# Bytes per launch each memory-bound kernel must move in this design (every array
# element it reads or writes counted once; positions and row pointers of neighbouring
# rows are cache-served and counted once).  N atoms, EP padded edges, EA active edges,
# K = (lmax+1)^2, C channels, FB feature bytes, NCB = C / 32 channel-block partials of
# the per-edge geometry gradient.
DESIGN_BYTES = {
    "nb::k_count": lambda z: 4 * z["N"] + 12 * z["N"],                  # degree out, sorted positions in
    "nb::k_fill": lambda z: 4 * z["EP"] + 16 * z["N"],                  # col out
    "nb::k_rev": lambda z: 8 * z["EP"] + 4 * z["N"],                    # col in, rev out
    "k_active_count": lambda z: 4 * z["EP"] + 20 * z["N"],              # col in; counts out
    "k_active_fill": lambda z: 8 * z["EP"] + 104 * z["EA"] + 20 * z["N"],  # col in, amap out; 96 B record + 2 indices
    "k_arev": lambda z: 16 * z["EA"] + 4 * z["N"],                      # a_e, rev, amap in; arev out
    "k_grad_sum": lambda z: 12 * (z["NCB"] + 1) * z["EA"],             # NCB partials in, their sum out
    "k_forces": lambda z: 28 * z["EA"] + 20 * z["N"],                   # arev, own and reverse record in; F out
    "k_embed": lambda z: z["N"] * z["K"] * z["C"] * z["FB"] + 4 * z["N"],
    "k_pre_linear": lambda z: 2 * z["N"] * z["K"] * z["C"] * z["FB"] + 4 * z["N"] * z["C"],
    "k_node_update": lambda z: 3 * z["N"] * z["K"] * z["C"] * z["FB"],
    "k_node_bwd": lambda z: z["N"] * z["K"] * z["C"] * (z["FB"] + 8),
    "k_pre_linear_bwd": lambda z: z["N"] * z["K"] * z["C"] * 12 + 4 * z["N"] * z["C"],
    "k_readout": lambda z: z["N"] * z["C"] * z["FB"] + 4 * z["N"],
    "k_readout_bwd": lambda z: z["N"] * z["C"] * z["FB"] + 4 * z["N"] * z["K"] * z["C"],
}


# kernels of the timed passes that bench.py reports next to the HBM peak
PASS_KERNELS = {"geometry": ("k_active_count", "k_active_fill", "k_arev"), "forces": ("k_grad_sum", "k_forces")}


def pass_bytes(name, n, edges_padded, edges_active, channels, lmax=2, bf16=True):
    """bytes the named pass has to move in this design (sum over its kernels)"""
    z = {"N": n, "EP": edges_padded, "EA": edges_active, "C": channels, "K": (lmax + 1) ** 2, "FB": 2 if bf16 else 4,
         "NCB": max(1, channels // 32)}
    ks = [k for k in PASS_KERNELS[name] if not (k == "k_grad_sum" and z["NCB"] == 1)]
    return sum(DESIGN_BYTES[k](z) for k in ks)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name):
    n = name.replace("void ", "").split("(")[0]
    return n.replace("mdmp::", "")


def stats(path, cmd, top):
    rows = list(csv.DictReader(open(path)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# rocprofv3 kernel statistics", f"# command: {cmd}", "",
           f"{'kernel':64s} {'calls':>6s} {'avg ms':>10s} {'total ms':>10s} {'%':>6s}"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows[:top]:
        out.append(f"{short_name(r['Name'])[:64]:64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e6:10.3f} "
                   f"{float(r['TotalDurationNs']) / 1e6:10.3f} {100 * float(r['TotalDurationNs']) / tot:6.2f}")
    out.append("")
    out.append("aggregates over all instantiations (average = total / calls):")
    for k in ("k_edge_fwd", "k_edge_bwd_recv", "k_edge_bwd_send", "k_node_bwd", "k_node_update", "k_pre_linear<",
              "k_pre_linear_bwd"):
        sel = [r for r in rows if ("mdmp::" + k) in r["Name"]]
        if not sel:
            continue
        t = sum(float(r["TotalDurationNs"]) for r in sel)
        c = sum(int(r["Calls"]) for r in sel)
        out.append(f"  {k.rstrip('<'):20s} calls {c:4d}  total {t / 1e6:10.3f} ms  average {t / c / 1e6:10.3f} ms")
    out.append(f"all kernels: {tot / 1e6:.3f} ms")
    return "\n".join(out)


def _per_dispatch(path, counter):
    vals = defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        vals[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return vals, names


def _copy_scale(vals, names):
    cand = [d for d in vals if "copy" in names[d]]
    if not cand:
        raise SystemExit("no copy dispatch found (run the program with its 1 GiB calibration copy)")
    d = max(cand, key=lambda x: vals[x])
    return COPY_BYTES / (vals[d] * 1024.0), d


def traffic(fetch_csv, write_csv, kernel, cmd):
    fv, fn = _per_dispatch(fetch_csv, "FETCH_SIZE")
    wv, wn = _per_dispatch(write_csv, "WRITE_SIZE")
    fs, fd = _copy_scale(fv, fn)
    ws, wd = _copy_scale(wv, wn)
    fk = sorted(d for d in fv if ("mdmp::" + kernel + "<") in fn[d] or ("mdmp::" + kernel + "(") in fn[d])
    wk = sorted(d for d in wv if ("mdmp::" + kernel + "<") in wn[d] or ("mdmp::" + kernel + "(") in wn[d])
    if not fk or len(fk) != len(wk):
        raise SystemExit(f"dispatches of {kernel}: fetch {len(fk)} write {len(wk)}")
    out = [f"# HBM traffic of {kernel} from rocprofv3 counters", f"# command (FETCH_SIZE, then WRITE_SIZE): {cmd}", "",
           f"calibration copy (1 GiB read + 1 GiB written): FETCH_SIZE {fv[fd]:.0f} KiB -> scale {fs:.4f}; "
           f"WRITE_SIZE {wv[wd]:.0f} KiB -> scale {ws:.4f}", "",
           f"{'dispatch':>8s}  {'kernel':48s} {'FETCH KiB':>14s} {'WRITE KiB':>14s} {'bytes (scaled)':>16s}"]
    tot = 0.0
    for a, b in zip(fk, wk):
        by = fv[a] * 1024.0 * fs + wv[b] * 1024.0 * ws
        tot += by
        out.append(f"{a:8d}  {short_name(fn[a])[:48]:48s} {fv[a]:14.0f} {wv[b]:14.0f} {by:16.4e}")
    out += ["", f"launches: {len(fk)}", f"bytes_per_launch: {tot / len(fk):.6e}",
            f"source_sha256: {kernel_source_hash()}"]
    return "\n".join(out)


def _base(name):
    n = short_name(name)
    return n.split("<")[0]


def _stats_ms(stats_csv):
    """kernel base name -> (calls, total ms) summed over instantiations"""
    out = defaultdict(lambda: [0, 0.0])
    for r in csv.DictReader(open(stats_csv)):
        b = _base(r["Name"])
        out[b][0] += int(r["Calls"])
        out[b][1] += float(r["TotalDurationNs"]) / 1e6
    return out


def hbm(fetch_csv, write_csv, stats_csv, cmd, sizes):
    fv, fn = _per_dispatch(fetch_csv, "FETCH_SIZE")
    wv, wn = _per_dispatch(write_csv, "WRITE_SIZE")
    fs, fd = _copy_scale(fv, fn)
    ws, wd = _copy_scale(wv, wn)
    ms = _stats_ms(stats_csv)
    z = dict(sizes)
    out = [f"# HBM traffic and bandwidth of the memory-bound kernels (rocprofv3 counters)",
           f"# command (FETCH_SIZE run, WRITE_SIZE run, kernel-trace run): {cmd}",
           f"# workload: N {z['N']}, padded edges {z['EP']}, active edges {z['EA']}, C {z['C']}, K {z['K']}, "
           f"feature bytes {z['FB']}, channel-block partials {z['NCB']}",
           f"# calibration copy: FETCH_SIZE scale {fs:.4f}, WRITE_SIZE scale {ws:.4f}; HBM peak {HBM_PEAK_GBS:.0f} GB/s",
           "", f"{'kernel':18s} {'launches':>8s} {'mean ms':>8s} {'counter GB':>10s} {'GB/s':>8s} {'frac':>6s} "
               f"{'design GB':>10s} {'GB/s':>8s} {'frac':>6s}"]
    for k, f in DESIGN_BYTES.items():
        fk = [d for d in fv if _base(fn[d]) == k]
        wk = [d for d in wv if _base(wn[d]) == k]
        if not fk or not wk or k not in ms:
            continue
        cb = (sum(fv[d] for d in fk) * 1024.0 * fs / len(fk) + sum(wv[d] for d in wk) * 1024.0 * ws / len(wk))
        t = ms[k][1] / ms[k][0]
        db = f(z)
        out.append(f"{k:18s} {ms[k][0]:8d} {t:8.3f} {cb / 1e9:10.3f} {cb / t / 1e6:8.0f} {cb / t / 1e6 / HBM_PEAK_GBS:6.3f} "
                   f"{db / 1e9:10.3f} {db / t / 1e6:8.0f} {db / t / 1e6 / HBM_PEAK_GBS:6.3f}")
    out += ["", "counter GB = (FETCH_SIZE + WRITE_SIZE) per launch, scaled; design GB = bytes the kernel has to move "
                "(every element of its inputs and outputs once); GB/s over the mean kernel duration of the "
                "kernel-trace run.", f"source_sha256: {kernel_source_hash()}"]
    return "\n".join(out)


def mfma(pmc_csv, stats_csv, cmd):
    vals = defaultdict(lambda: defaultdict(float))
    names = {}
    for r in csv.DictReader(open(pmc_csv)):
        d = int(r["Dispatch_Id"])
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = short_name(r["Kernel_Name"])
    st = {}
    for r in csv.DictReader(open(stats_csv)):
        st[short_name(r["Name"])] = float(r["AverageNs"]) / 1e6
    agg = {}
    for d in sorted(vals):
        a = agg.setdefault(names[d], defaultdict(float))
        a["n"] += 1
        for c, v in vals[d].items():
            a[c] += v
    out = [f"# MFMA activity per kernel (rocprofv3 counters)", f"# command (counter run, kernel-trace run): {cmd}",
           f"# busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} x {N_SIMD} SIMDs); flops = MOPS x 512; "
           f"peaks bf16 {MFMA_PEAK_TFS['bf16']:.0f}, f32 {MFMA_PEAK_TFS['f32']} TFLOP/s", "",
           f"{'kernel':48s} {'n':>3s} {'mean ms':>8s} {'busy':>6s} {'bf16 TF':>8s} {'TF/s':>7s} {'frac':>6s} "
           f"{'f32 TF':>7s} {'TF/s':>6s} {'frac':>6s}"]
    for k, a in agg.items():
        if a["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + a["SQ_INSTS_VALU_MFMA_MOPS_F32"] == 0 or k not in st:
            continue
        n, t = a["n"], st[k]
        busy = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (a["GRBM_GUI_ACTIVE"] / N_XCD * N_SIMD)
        bf = a["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / n
        f3 = a["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512 / n
        out.append(f"{k[:48]:48s} {int(n):3d} {t:8.3f} {busy:6.3f} {bf / 1e12:8.3f} {bf / t / 1e9:7.1f} "
                   f"{bf / t / 1e9 / MFMA_PEAK_TFS['bf16']:6.3f} {f3 / 1e12:7.3f} {f3 / t / 1e9:6.1f} "
                   f"{f3 / t / 1e9 / MFMA_PEAK_TFS['f32']:6.3f}")
    out += ["", f"source_sha256: {kernel_source_hash()}"]
    return "\n".join(out)


def l2(runs, cmd):
    tabs = {}
    for label, path in runs:
        agg = defaultdict(lambda: defaultdict(float))
        vals = defaultdict(lambda: defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            d = int(r["Dispatch_Id"])
            vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
            names[d] = short_name(r["Kernel_Name"])
        for d, v in vals.items():
            a = agg[names[d]]
            a["n"] += 1
            for c, x in v.items():
                a[c] += x
        tabs[label] = agg
    labels = [lb for lb, _ in runs]
    kern = sorted({k for t in tabs.values() for k in t if k.startswith(("k_", "nb::"))},
                  key=lambda k: -sum(t.get(k, {}).get("TCC_MISS_sum", 0) for t in tabs.values()))
    out = ["# L2 (TCC) hit rate and misses per launch, by run (rocprofv3 TCC_HIT_sum, TCC_MISS_sum)",
           f"# command: {cmd}", "",
           f"{'kernel':48s} " + " ".join(f"{lb + ' hit':>12s} {lb + ' Mmiss':>13s}" for lb in labels)]
    for k in kern[:24]:
        row = f"{k[:48]:48s} "
        for lb in labels:
            a = tabs[lb].get(k)
            if not a:
                row += f"{'-':>12s} {'-':>13s} "
                continue
            h, m = a["TCC_HIT_sum"], a["TCC_MISS_sum"]
            row += f"{h / max(h + m, 1):12.3f} {m / a['n'] / 1e6:13.1f} "
        out.append(row.rstrip())
    out += ["", f"source_sha256: {kernel_source_hash()}"]
    return "\n".join(out)


def read_traffic(path):
    """(bytes per launch, source hash) from a `traffic` summary, or None."""
    if not os.path.exists(path):
        return None
    by = sh = None
    for line in open(path):
        if line.startswith("bytes_per_launch:"):
            by = float(line.split(":", 1)[1])
        elif line.startswith("source_sha256:"):
            sh = line.split(":", 1)[1].strip()
    return None if by is None or sh is None else (by, sh)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--top", type=int, default=24)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--kernel", required=True)
    t.add_argument("--cmd", required=True)
    h = sub.add_parser("hbm")
    h.add_argument("fetch_csv")
    h.add_argument("write_csv")
    h.add_argument("stats_csv")
    h.add_argument("--cmd", required=True)
    h.add_argument("--atoms", type=int, required=True)
    h.add_argument("--edges-padded", type=int, required=True)
    h.add_argument("--edges-active", type=int, required=True)
    h.add_argument("--channels", type=int, default=128)
    h.add_argument("--lmax", type=int, default=2)
    h.add_argument("--bf16", action="store_true")
    l2p = sub.add_parser("l2")
    l2p.add_argument("runs", nargs="+", help="LABEL=PMC_CSV")
    l2p.add_argument("--cmd", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("pmc_csv")
    m.add_argument("stats_csv")
    m.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.what == "stats":
        print(stats(a.csv, a.cmd, a.top))
    elif a.what == "traffic":
        print(traffic(a.fetch_csv, a.write_csv, a.kernel, a.cmd))
    elif a.what == "hbm":
        sizes = {"N": a.atoms, "EP": a.edges_padded, "EA": a.edges_active, "C": a.channels,
                 "K": (a.lmax + 1) ** 2, "FB": 2 if a.bf16 else 4, "NCB": max(1, a.channels // 32)}
        print(hbm(a.fetch_csv, a.write_csv, a.stats_csv, a.cmd, sizes))
    elif a.what == "l2":
        print(l2([tuple(x.split("=", 1)) for x in a.runs], a.cmd))
    else:
        print(mfma(a.pmc_csv, a.stats_csv, a.cmd))


if __name__ == "__main__":
    sys.exit(main())
