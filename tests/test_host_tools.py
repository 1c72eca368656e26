"""Host-side logic of the measurement tools, on the CPU: the benchmark's one-GPU guard, its
per-edge flop count, and the rocprofv3 summaries' byte arithmetic on small synthetic counter
files (the calibration copy sets each counter's scale)."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_receiver_flop_count():
    """Paths (l1, l2, l3) with l <= 2 and the triangle rule: s1 = sum (2 l1 + 1)(2 l3 + 1) and
    s2 = sum (2 l3 + 1) are 179 and 51 over all 15 paths, 9 and 9 over the first layer's
    (l1 = 0) and 9 and 3 over the last layer's (l3 = 0)."""
    sys.path.insert(0, ROOT)
    import bench
    from molecular_dynamics_amd import inputs
    assert bench.tp_macs_mode(2, 0) == (179, 51)
    assert bench.tp_macs_mode(2, 1) == (9, 9)
    assert bench.tp_macs_mode(2, 2) == (9, 3)
    cfg = inputs.ModelConfig(n_species=4, channels=128, lmax=2, n_bessel=8, heads=4, layers=4, cutoff=5.0)
    assert bench.recv_bwd_flops_per_edge(cfg, 0) == 2.0 * 128 * (2 * 179 + 2 * 51 + 3 * 9)
    assert [bench.layer_mode(t, 4) for t in range(4)] == [1, 0, 0, 2]
    assert bench.layer_mode(0, 1) == 3


def test_force_pass_slots():
    from molecular_dynamics_amd import prof_summary as P
    # 32-channel partials in even/odd halves; the first bf16 receiver (64-channel blocks)
    # folds the odd half into the even one
    assert P.force_slots(128, True) == 2 and P.force_slots(128, False) == 4
    assert P.force_slots(64, True) == 1 and P.force_slots(64, False) == 2
    assert P.force_slots(32, True) == 1 and P.force_slots(16, False) == 1


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_arithmetic(tmp_path):
    from molecular_dynamics_amd import prof_summary as P
    recv = "void mdmp::k_edge_bwd_recv<2, 0, 128, unsigned short, 32>(mdmp::EdgeArgs, mdmp::LayerW, mdmp::BwdArgs)"
    copy = "void at::native::elementwise_copy_kernel(int)"
    red = "void at::native::reduce_kernel<512, 1>(float)"
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the 1 GiB copy reads 524,288 KiB by FETCH_SIZE (scale 2) and writes 1,048,576 KiB (scale 1)
    _counters(f, "FETCH_SIZE", [(1, copy, 524288), (2, red, 573106), (5, recv, 1000), (9, recv, 3000)])
    _counters(w, "WRITE_SIZE", [(1, copy, 1048576), (5, recv, 500), (9, recv, 700)])
    text = P.traffic(str(f), str(w), "k_edge_bwd_recv", "synthetic")
    per_launch = ((1000 + 3000) * 1024.0 * 2.0 + (500 + 700) * 1024.0) / 2
    path = tmp_path / "summary.txt"
    path.write_text(text)
    got, sha = P.read_traffic(str(path))
    assert got == pytest.approx(per_launch, rel=1e-6)
    assert sha == P.kernel_source_hash()
    assert "scale 2.0000" in text and "scale 1.0000" in text
    assert "read-only sum" in text and "scale 1.8296" in text


def test_traffic_summary_needs_the_calibration_copy(tmp_path):
    from molecular_dynamics_amd import prof_summary as P
    recv = "void mdmp::k_edge_bwd_recv<2, 0, 128, unsigned short, 32>(mdmp::EdgeArgs)"
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counters(f, "FETCH_SIZE", [(5, recv, 1000)])
    _counters(w, "WRITE_SIZE", [(5, recv, 500)])
    with pytest.raises(SystemExit):
        P.traffic(str(f), str(w), "k_edge_bwd_recv", "synthetic")


def test_l1_l2_request_summary_arithmetic(tmp_path):
    """bytes per L1-to-L2 read request come from the 1 GiB copy; per-launch means and the
    L2 hit rate per kernel"""
    import csv
    from molecular_dynamics_amd import prof_summary as P
    recv = "void mdmp::k_edge_bwd_recv<2, 0, 128, unsigned short, 32>(mdmp::EdgeArgs, mdmp::LayerW, mdmp::BwdArgs)"
    copy = "void at::native::elementwise_copy_kernel(int)"
    path = tmp_path / "tcp.csv"
    rows = [(1, copy, {"TCP_TCC_READ_REQ_sum": 8388608, "TCP_TOTAL_CACHE_ACCESSES_sum": 1, "TCC_HIT_sum": 0,
                       "TCC_MISS_sum": 1}),
            (5, recv, {"TCP_TCC_READ_REQ_sum": 1000, "TCP_TOTAL_CACHE_ACCESSES_sum": 3e6, "TCC_HIT_sum": 900,
                       "TCC_MISS_sum": 100}),
            (9, recv, {"TCP_TCC_READ_REQ_sum": 3000, "TCP_TOTAL_CACHE_ACCESSES_sum": 5e6, "TCC_HIT_sum": 2700,
                       "TCC_MISS_sum": 300})]
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, k, cs in rows:
            for c, v in cs.items():
                wr.writerow([d, k, c, v])
    text = P.tcp(str(path), "synthetic", edges_active=1000)
    assert "128.0" in text.splitlines()[2]  # 2^30 bytes over 8,388,608 requests
    line = next(x for x in text.splitlines() if x.startswith("k_edge_bwd_recv"))
    f = line.split()
    # 2 launches; L1 accesses 4 M per launch; (1000 + 3000) / 2 requests x 128 B = 256,000 B = 0.0 GB,
    # 256 B per edge; hit rate 0.9
    assert f[-5] == "2" and f[-4] == "4.0" and f[-2] == "256" and f[-1] == "0.900"
