"""Host-side check of the edge-frame identities used by the unpruned edge kernels.

The kernels' own helpers (csrc/kernels.hpp, compiled for the host with hipcc) are
checked against the lab-frame products of the same header: Y(R v) = D Y(v) for the
Wigner blocks built from the edge frame, R rhat = z-hat, and for the forward product,
the receiver's dot products, the tangential r-hat gradient and the sender's input
gradient (edge seen from the other end), over 20,000 random directions including
both poles.  The equivariance of the coupling tensors ("Unlocking Tensor Core
Performance", section "Why MLIPs Need Dedicated Performance Optimization") makes
these exact up to float32 rounding.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not installed")
def test_edge_frame_identities(tmp_path):
    exe = str(tmp_path / "frame_identities")
    src = os.path.join(ROOT, "tests", "native", "frame_identities.hip")
    cmd = [HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-std=c++17", "-O1", "-fconstexpr-steps=200000000", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "molecular_dynamics_amd", "csrc"), src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
