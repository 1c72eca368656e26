"""Short text summaries of rocprofv3 output (kernel statistics and HBM byte counters).

    python -m molecular_dynamics_amd.prof_summary stats  KERNEL_STATS_CSV --cmd "..." [--top 24]
    python -m molecular_dynamics_amd.prof_summary traffic FETCH_CSV WRITE_CSV --kernel k_edge_bwd_recv --cmd "..."
    python -m molecular_dynamics_amd.prof_summary hbm FETCH_CSV WRITE_CSV KERNEL_STATS_CSV --cmd "..." \
        --atoms N --edges-padded EP --edges-active EA --channels C --lmax L [--bf16]
    python -m molecular_dynamics_amd.prof_summary mfma PMC_CSV KERNEL_STATS_CSV --cmd "..."
    python -m molecular_dynamics_amd.prof_summary l2 LABEL=PMC_CSV [LABEL=PMC_CSV ...] --cmd "..."
    python -m molecular_dynamics_amd.prof_summary sq KERNEL_STATS_CSV PMC_CSV [PMC_CSV ...] --cmd "..."
    python -m molecular_dynamics_amd.prof_summary tcp PMC_CSV --cmd "..." --edges-active EA

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
`sq` reads the three counter runs of SQ_PASSES: instruction mix per wave, VALU issue
utilisation and wait fractions per kernel.  `tcp` reads a `--pmc TCP_TCC_READ_REQ_sum
TCP_TOTAL_CACHE_ACCESSES_sum TCC_HIT_sum TCC_MISS_sum` run of a program that first copies
1 GiB (whose 2^30 bytes read give the bytes per L1-to-L2 read request): per kernel the
vector L1 accesses, the read bytes the L1s request from L2 per launch and per active
edge, and the L2 hit rate.
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
# K = (lmax+1)^2, C channels, FB feature bytes, NCB channel-block partials of the
# per-edge geometry gradient (C / 32, at least 1), GS of them the force pass reads per
# edge: the partials sit in even and odd halves of (NCB + 1) / 2 slots each, and the
# first layer's bf16 receiver (channel blocks of 64, C >= 64) folds the odd half into
# the even one, so then only the even half is read.
DESIGN_BYTES = {
    "nb::k_count": lambda z: 4 * z["N"] + 12 * z["N"],                  # degree out, sorted positions in
    "nb::k_fill": lambda z: 4 * z["EP"] + 16 * z["N"],                  # col out
    "nb::k_rev": lambda z: 8 * z["EP"] + 4 * z["N"],                    # col in, rev out
    # col, rev in, amap out; 64 B record + sender + reverse padded index per active edge;
    # positions, row pointers in, row end out
    "k_active_fill": lambda z: 12 * z["EP"] + 72 * z["EA"] + 24 * z["N"],
    "k_arev": lambda z: 12 * z["EA"] + 8 * z["N"],                      # a_r, amap in; arev out
    # arev and the edge's GS partials in (the reverse edge's are the same array, read
    # as another row's own); row bounds, perm in, F out
    "k_forces": lambda z: (4 + 12 * z["GS"]) * z["EA"] + 24 * z["N"],
    "k_embed": lambda z: z["N"] * z["K"] * z["C"] * z["FB"] + 4 * z["N"],
    "k_pre_linear": lambda z: 2 * z["N"] * z["K"] * z["C"] * z["FB"] + 4 * z["N"] * z["C"],
    "k_node_update": lambda z: 3 * z["N"] * z["K"] * z["C"] * z["FB"],
    "k_node_bwd": lambda z: z["N"] * z["K"] * z["C"] * (z["FB"] + 8),
    "k_pre_linear_bwd": lambda z: z["N"] * z["K"] * z["C"] * 12 + 4 * z["N"] * z["C"],
    "k_readout": lambda z: z["N"] * z["C"] * z["FB"] + 4 * z["N"],
    "k_readout_bwd": lambda z: z["N"] * z["C"] * (z["FB"] + 4),  # h^0 in, row 0 of g_h out
}

# variant labels of the summaries (the trailing bool template arguments)
VARIANT_LABEL = {("k_embed", (False,)): "h0 only", ("k_pre_linear", (True,)): "first",
                 ("k_node_update", (True, False)): "last", ("k_node_update", (False, True)): "first",
                 ("k_node_bwd", (True,)): "last", ("k_pre_linear_bwd", (True,)): "last"}

# The per-atom kernels' pruned instantiations (their trailing bool template arguments):
# the first layer's (BOT) and the last layer's (TOP) move only the rows that reach the energy.
DESIGN_BYTES_VARIANT = {
    # embedding without the zero rows: h^0 only
    ("k_embed", (False,)): lambda z: z["N"] * z["C"] * z["FB"] + 4 * z["N"],
    # first layer: h^0 in; ht^0 and q out
    ("k_pre_linear", (True,)): lambda z: 2 * z["N"] * z["C"] * z["FB"] + 4 * z["N"] * z["C"],
    # last layer (TOP): m^0, h^0 in, h^0 out; first layer (BOT): m in, h^0 in, h out
    ("k_node_update", (True, False)): lambda z: 3 * z["N"] * z["C"] * z["FB"],
    ("k_node_update", (False, True)): lambda z: (2 * z["K"] + 1) * z["N"] * z["C"] * z["FB"],
    # last layer: m^0 and row 0 of g_h in, g_m^0 out
    ("k_node_bwd", (True,)): lambda z: z["N"] * z["C"] * (z["FB"] + 8),
    # last layer: g_ht, g_q and row 0 of g_h in; g_h out
    ("k_pre_linear_bwd", (True,)): lambda z: z["N"] * z["C"] * (8 * z["K"] + 8),
}


def _flags(name):
    """the trailing bool template arguments of a kernel name, e.g. (True, False)"""
    n = short_name(name)
    if "<" not in n or ">" not in n:
        return ()
    args = [a.strip() for a in n[n.index("<") + 1:n.rindex(">")].split(",")]
    out = []
    for a in reversed(args):
        if a not in ("true", "false"):
            break
        out.append(a == "true")
    return tuple(reversed(out))


def design_bytes(name, z):
    """bytes the kernel instantiation `name` has to move (None if it has no formula)"""
    b, f = _base(name), _flags(name)
    if (b, f) in DESIGN_BYTES_VARIANT:
        return DESIGN_BYTES_VARIANT[(b, f)](z)
    f = DESIGN_BYTES.get(b)
    return f(z) if f else None


def force_slots(channels, bf16):
    """geometry-gradient partials the force pass reads per edge"""
    ncb = max(1, channels // 32)
    half = (ncb + 1) // 2
    folded = ncb == 1 or (bf16 and channels >= 64)
    return half if folded else 2 * half


# kernels of the timed passes that bench.py reports next to the HBM peak
PASS_KERNELS = {"geometry": ("k_active_fill", "k_arev"), "forces": ("k_forces",)}

# The method's own byte count per pass, independent of this design: the edge-geometry
# gather writes a 4-byte index and a 76-byte geometry record per padded edge (80 B);
# the force aggregation reads a 12-byte geometry gradient twice (own and reverse edge)
# plus 8 bytes of indices per padded edge (32 B) and writes 12 bytes per atom.
ALGORITHMIC_BYTES = {"geometry": lambda n, ep: 80 * ep, "forces": lambda n, ep: 32 * ep + 12 * n}


def pass_bytes(name, n, edges_padded, edges_active, channels, lmax=2, bf16=True):
    """bytes the named pass has to move in this design (sum over its kernels)"""
    z = {"N": n, "EP": edges_padded, "EA": edges_active, "C": channels, "K": (lmax + 1) ** 2, "FB": 2 if bf16 else 4,
         "NCB": max(1, channels // 32), "GS": force_slots(channels, bf16)}
    return sum(DESIGN_BYTES[k](z) for k in PASS_KERNELS[name])


def pass_bytes_algorithmic(name, n, edges_padded):
    """the method's byte count of the named pass (per padded edge and atom)"""
    return ALGORITHMIC_BYTES[name](n, edges_padded)


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


def _sum_check(fetch_vals, fetch_names):
    """the read counter's scale from the 1 GiB read-only sum (the largest reduction
    dispatch), as a check of the copy's; None if the run has no such dispatch"""
    cand = [d for d in fetch_vals if "reduce" in fetch_names[d].lower()]
    if not cand:
        return None
    d = max(cand, key=lambda x: fetch_vals[x])
    return f"cross-check: read-only sum of the same 1 GiB: FETCH_SIZE {fetch_vals[d]:.0f} KiB -> scale " \
           f"{COPY_BYTES / (fetch_vals[d] * 1024.0):.4f}"


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
           f"WRITE_SIZE {wv[wd]:.0f} KiB -> scale {ws:.4f}", _sum_check(fv, fn) or "", "",
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
    # mean duration per instantiation (base name, trailing bool template arguments)
    ms = defaultdict(lambda: [0, 0.0])
    for r in csv.DictReader(open(stats_csv)):
        key = (_base(r["Name"]), _flags(r["Name"]))
        ms[key][0] += int(r["Calls"])
        ms[key][1] += float(r["TotalDurationNs"]) / 1e6
    z = dict(sizes)
    out = [f"# HBM traffic and bandwidth of the memory-bound kernels (rocprofv3 counters)",
           f"# command (FETCH_SIZE run, WRITE_SIZE run, kernel-trace run): {cmd}",
           f"# workload: N {z['N']}, padded edges {z['EP']}, active edges {z['EA']}, C {z['C']}, K {z['K']}, "
           f"feature bytes {z['FB']}",
           f"# calibration copy: FETCH_SIZE scale {fs:.4f}, WRITE_SIZE scale {ws:.4f}; HBM peak {HBM_PEAK_GBS:.0f} GB/s",
           "# " + (_sum_check(fv, fn) or "no read-only sum in this run"),
           "", f"{'kernel':26s} {'launches':>8s} {'mean ms':>8s} {'counter GB':>10s} {'GB/s':>8s} {'frac':>6s} "
               f"{'design GB':>10s} {'GB/s':>8s} {'frac':>6s}"]
    keys = sorted({(_base(fn[d]), _flags(fn[d])) for d in fv if _base(fn[d]) in DESIGN_BYTES},
                  key=lambda k: (list(DESIGN_BYTES).index(k[0]), k[1]))
    for key in keys:
        fk = [d for d in fv if (_base(fn[d]), _flags(fn[d])) == key]
        wk = [d for d in wv if (_base(wn[d]), _flags(wn[d])) == key]
        if not fk or not wk or key not in ms:
            continue
        cb = (sum(fv[d] for d in fk) * 1024.0 * fs / len(fk) + sum(wv[d] for d in wk) * 1024.0 * ws / len(wk))
        t = ms[key][1] / ms[key][0]
        db = design_bytes(fn[fk[0]], z)
        label = key[0] + (f" ({VARIANT_LABEL[key]})" if key in VARIANT_LABEL else "")
        out.append(f"{label:26s} {ms[key][0]:8d} {t:8.3f} {cb / 1e9:10.3f} {cb / t / 1e6:8.0f} "
                   f"{cb / t / 1e6 / HBM_PEAK_GBS:6.3f} {db / 1e9:10.3f} {db / t / 1e6:8.0f} "
                   f"{db / t / 1e6 / HBM_PEAK_GBS:6.3f}")
    out += ["", "counter GB = (FETCH_SIZE + WRITE_SIZE) per launch, scaled; design GB = bytes the kernel has to move "
                "(every element of its inputs and outputs once); GB/s over the mean kernel duration of the "
                "kernel-trace run.  first / last: the instantiations of the first and last layer, which move "
                "only the feature rows that reach the energy; h0 only: the embedding without its zero rows.",
            f"source_sha256: {kernel_source_hash()}"]
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


def tcp(pmc_csv, cmd, edges_active):
    vals = defaultdict(lambda: defaultdict(float))
    names = {}
    for r in csv.DictReader(open(pmc_csv)):
        d = int(r["Dispatch_Id"])
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    copies = [d for d in vals if "copy" in names[d]]
    if not copies:
        raise SystemExit("no copy dispatch found (run the program with its 1 GiB calibration copy)")
    d0 = max(copies, key=lambda d: vals[d]["TCP_TCC_READ_REQ_sum"])
    bpr = COPY_BYTES / vals[d0]["TCP_TCC_READ_REQ_sum"]
    agg = defaultdict(lambda: defaultdict(float))
    for d, v in vals.items():
        a = agg[short_name(names[d])]
        a["n"] += 1
        for c, x in v.items():
            a[c] += x
    kern = sorted((k for k in agg if k.startswith(("k_", "nb::"))), key=lambda k: -agg[k]["TCP_TCC_READ_REQ_sum"])
    out = ["# vector L1 (TCP) accesses, L1-to-L2 read requests and L2 (TCC) hit rate per kernel (rocprofv3 counters)",
           f"# command: {cmd}",
           f"# bytes per L1-to-L2 read request from the 1 GiB calibration copy: {bpr:.1f}; "
           f"per edge: over the {edges_active} active edges", "",
           f"{'kernel':52s} {'n':>3s} {'L1 acc M':>10s} {'L1->L2 GB':>10s} {'B/edge':>8s} {'L2 hit':>7s}"]
    for k in kern[:24]:
        a = agg[k]
        n = a["n"]
        gb = a["TCP_TCC_READ_REQ_sum"] * bpr / n / 1e9
        h, m = a["TCC_HIT_sum"], a["TCC_MISS_sum"]
        out.append(f"{k[:52]:52s} {int(n):3d} {a['TCP_TOTAL_CACHE_ACCESSES_sum'] / n / 1e6:10.1f} {gb:10.1f} "
                   f"{gb * 1e9 / max(edges_active, 1):8.0f} {h / max(h + m, 1):7.3f}")
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


SQ_PASSES = {
    "mix": "SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_INSTS_SALU SQ_INSTS_MFMA SQ_WAVES "
           "SQ_INSTS_VALU_CVT",
    "cycles": "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_ANY SQ_WAIT_ANY "
              "SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE",
    "valu": "SQ_THREAD_CYCLES_VALU SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_MUL_F32 SQ_INSTS_VALU_ADD_F32 "
            "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_VALU_INT32 SQ_ACTIVE_INST_ANY SQ_INSTS_SMEM",
}
CLOCK_GHZ = 2.4


def _sq_counters(paths):
    """{kernel: {counter: mean per dispatch}} over several --pmc counter_collection files"""
    vals = defaultdict(lambda: defaultdict(list))
    for path in paths:
        per = defaultdict(dict)
        for r in csv.DictReader(open(path)):
            per[(r["Dispatch_Id"], r["Kernel_Name"])][r["Counter_Name"]] = float(r["Counter_Value"])
        for (_, k), cs in per.items():
            for c, v in cs.items():
                vals[short_name(k)][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}


def sq(pmc_csvs, stats_csv, cmd, match):
    """Instruction mix and issue/wait fractions per kernel from the SQ_PASSES counter runs.

    VALU issue utilisation = SQ_INSTS_VALU x 4 cycles (a wave64 VALU instruction on a
    16-lane SIMD) / (mean duration x 2.4 GHz x 1,024 SIMDs); the instruction classes are
    fractions of SQ_INSTS_VALU; the wait and active fractions are over SQ_WAVE_CYCLES."""
    cnt = _sq_counters(pmc_csvs)
    ms = {short_name(r["Name"]): float(r["AverageNs"]) / 1e6 for r in csv.DictReader(open(stats_csv))}
    out = ["# SQ counters of the edge kernels (rocprofv3 --pmc, one run per pass, counters per dispatch averaged)",
           f"# command (one per pass, COUNTERS = each line of prof_summary.SQ_PASSES): {cmd}",
           "# per wave: instructions issued by one 64-lane wave; VALU% columns: share of its VALU instructions",
           "", f"{'kernel':50s} {'ms':>7s} {'waves':>9s} {'VALU':>6s} {'LDS':>5s} {'VMrd':>5s} {'SALU':>5s} "
               f"{'MFMA':>5s} {'CVT':>5s} | {'issue':>5s} {'FMA%':>5s} {'MUL%':>5s} {'ADD%':>5s} {'INT%':>5s} "
               f"{'TRN%':>5s} {'other%':>6s} | {'VALUact':>7s} {'waitdep':>7s} {'waitany':>7s} {'LDSconf':>7s}"]
    for k in sorted((k for k in cnt if any(m in k for m in match)), key=lambda k: -ms.get(k, 0)):
        c = cnt[k]
        W, V = c.get("SQ_WAVES", 0), c.get("SQ_INSTS_VALU", 0)
        if not W or not V or k not in ms:
            continue
        frac = {x: c.get(f"SQ_INSTS_VALU_{x}", 0) / V for x in ("FMA_F32", "MUL_F32", "ADD_F32", "INT32", "TRANS_F32")}
        other = 1 - sum(frac.values()) - c.get("SQ_INSTS_VALU_CVT", 0) / V
        wc = c.get("SQ_WAVE_CYCLES", 1)
        out.append(f"{k[:50]:50s} {ms[k]:7.2f} {W:9.0f} {V / W:6.0f} {c.get('SQ_INSTS_LDS', 0) / W:5.0f} "
                   f"{c.get('SQ_INSTS_VMEM_RD', 0) / W:5.0f} {c.get('SQ_INSTS_SALU', 0) / W:5.0f} "
                   f"{c.get('SQ_INSTS_MFMA', 0) / W:5.0f} {c.get('SQ_INSTS_VALU_CVT', 0) / W:5.0f} | "
                   f"{V * 4 / (ms[k] * 1e6 * CLOCK_GHZ * N_SIMD):5.3f} {100 * frac['FMA_F32']:5.1f} "
                   f"{100 * frac['MUL_F32']:5.1f} {100 * frac['ADD_F32']:5.1f} {100 * frac['INT32']:5.1f} "
                   f"{100 * frac['TRANS_F32']:5.1f} {100 * other:6.1f} | {c.get('SQ_ACTIVE_INST_VALU', 0) / wc:7.3f} "
                   f"{c.get('SQ_WAIT_INST_ANY', 0) / wc:7.3f} {c.get('SQ_WAIT_ANY', 0) / wc:7.3f} "
                   f"{c.get('SQ_LDS_BANK_CONFLICT', 0) / max(1.0, c.get('SQ_ACTIVE_INST_LDS', 0)):7.3f}")
    out += ["", "issue: VALU issue utilisation; other%: VALU instructions outside the FMA/MUL/ADD/INT/TRANS/CVT classes "
            "(moves, cross-lane DPP/permlane, selects, bit operations); VALUact, waitdep, waitany: "
            "SQ_ACTIVE_INST_VALU, SQ_WAIT_INST_ANY, SQ_WAIT_ANY over SQ_WAVE_CYCLES; LDSconf: "
            "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS.", f"source_sha256: {kernel_source_hash()}"]
    return "\n".join(out)


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
    q = sub.add_parser("sq")
    q.add_argument("stats_csv")
    q.add_argument("pmc_csvs", nargs="+")
    q.add_argument("--cmd", required=True)
    q.add_argument("--match", nargs="+", default=["k_edge", "k_active", "k_arev", "k_forces"])
    tp = sub.add_parser("tcp")
    tp.add_argument("pmc_csv")
    tp.add_argument("--cmd", required=True)
    tp.add_argument("--edges-active", type=int, required=True)
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
                 "K": (a.lmax + 1) ** 2, "FB": 2 if a.bf16 else 4, "NCB": max(1, a.channels // 32),
                 "GS": force_slots(a.channels, a.bf16)}
        print(hbm(a.fetch_csv, a.write_csv, a.stats_csv, a.cmd, sizes))
    elif a.what == "sq":
        print(sq(a.pmc_csvs, a.stats_csv, a.cmd, a.match))
    elif a.what == "l2":
        print(l2([tuple(x.split("=", 1)) for x in a.runs], a.cmd))
    elif a.what == "tcp":
        print(tcp(a.pmc_csv, a.cmd, a.edges_active))
    else:
        print(mfma(a.pmc_csv, a.stats_csv, a.cmd))


if __name__ == "__main__":
    sys.exit(main())
