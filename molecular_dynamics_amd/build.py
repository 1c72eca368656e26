"""Build libmdmp.so (HIP for gfx950) in-tree with hipcc, and the input helper.

    python -m molecular_dynamics_amd.build
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmdmp.so")
OBJ = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fconstexpr-steps=200000000",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# the neighbour list is decided in float64 with a fixed operation order; the edge
# kernels recompute tile addresses from the edge index instead of carrying one
# strength-reduced pointer per array across the tile loop (fewer live registers)
PER_FILE = {"neighbors.hip": ["-ffp-contract=off"], "model.hip": ["-mllvm", "-disable-lsr"]}
SOURCES = ["neighbors.hip", "model.hip", "md.hip", "noalloc.hip", "api.cpp", "prof.cpp"]


def _compile(src):
    obj = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-4000:])
    os.replace(tmp, OUT)
    from . import inputs
    inputs.build_rsa(force=True)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
