"""Short text summaries of rocprofv3 output (kernel statistics and HBM byte counters).

    python -m molecular_dynamics_amd.prof_summary stats  KERNEL_STATS_CSV --cmd "..." [--top 24]
    python -m molecular_dynamics_amd.prof_summary traffic FETCH_CSV WRITE_CSV --kernel k_edge_bwd_recv --cmd "..."

`stats` lists the kernels of a `rocprofv3 --kernel-trace --stats --output-format csv`
run by total time and aggregates every instantiation of the named edge kernels.
`traffic` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a program that
first copies 1 GiB device-to-device: the counters of that copy (2^30 bytes read and
written) give the scale from counter units to bytes, which is then applied to every
dispatch of the named kernel.  The result records a hash of the kernel sources so
that a reader can tell whether the counters still describe the current kernels.
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
    a = ap.parse_args(argv)
    if a.what == "stats":
        print(stats(a.csv, a.cmd, a.top))
    else:
        print(traffic(a.fetch_csv, a.write_csv, a.kernel, a.cmd))


if __name__ == "__main__":
    sys.exit(main())
