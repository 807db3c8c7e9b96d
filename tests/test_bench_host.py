"""CPU checks of bench.py's host logic: the rocprofv3 counter summation behind the live HBM
byte count, its fallback when the profiler is absent, the timing mode of each workload, and the
one-GPU guard (no GPU needed)."""
import argparse
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "FETCH_SIZE",
                        "Counter_Value": value})


def test_counter_sum_picks_the_named_kernels(tmp_path):
    p = tmp_path / "run_counter_collection.csv"
    write_counters(p, [("void sbl::(anonymous namespace)::k_gemm_nt_bf16<512, 1>(...)", "100.5"),
                       ("sbl::(anonymous namespace)::k_codes_t(unsigned short const*)", "2.5"),
                       ("void sbl::k_act_quant<4, 1>(...)", "1000"),
                       ("__amd_rocclr_copyBuffer", "524300")])
    bwd = ("k_codes_t", "k_gemm_nt_bf16", "k_splitk_reduce", "k_splitk_add_tail")
    total, n = bench._counter_kib(str(p), lambda k: any(b in k for b in bwd))
    assert (total, n) == (103.0, 2)
    total, n = bench._counter_kib(str(p), lambda k: "copyBuffer" in k)
    assert (total, n) == (524300.0, 1)
    assert bench._counter_kib(str(p), lambda k: False) == (0.0, 0)


def test_live_traffic_without_the_profiler(monkeypatch):
    import shutil
    monkeypatch.setattr(shutil, "which", lambda name: None)
    assert bench.live_traffic(14) is None


def test_live_traffic_failed_pass_gives_none(monkeypatch, tmp_path):
    # a profiler that runs but leaves no result file: the fallback, not an exception
    import shutil

    fake = tmp_path / "rocprofv3"
    fake.write_text("#!/bin/sh\nexit 139\n")
    fake.chmod(0o755)
    monkeypatch.setattr(shutil, "which", lambda name: str(fake))
    assert bench.live_traffic(14, timeout_s=30) is None


@pytest.mark.parametrize("workload,timing,graph", [(0, "auto", True), (1, "auto", True), (2, "auto", False),
                                                    (3, "auto", False), (3, "graph", True), (0, "eager", False)])
def test_timing_mode(workload, timing, graph):
    assert bench.use_graph(argparse.Namespace(workload=workload, timing=timing)) is graph


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
