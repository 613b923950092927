"""bench.py on the CPU: its command-line contract and the accounting behind
the numbers it reports (no GPU call is made here)."""

import json
import os
import subprocess
import sys

import numpy as np

import bench
from oracle import solattn_ref as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_studies():
    r = run_bench("--help")
    assert r.returncode == 0
    for study in ("accuracy", "seq", "routing", "first-order"):
        assert study in r.stdout


def test_executed_flops_match_the_oracle_accounting():
    # the FLOPs behind the reported TFLOP/s: exact + token-to-block tile +
    # approximate product, summed over heads, as the oracle defines them
    rng = np.random.default_rng(3)
    for L, d, block in ((1000, 64, 64), (4096, 128, 128), (300, 128, 128)):
        N = ref.num_blocks(L, block)
        sel = rng.random((3, N, N)) < 0.3
        ex, tile, ap = bench.executed_flops(sel, L, d, block)
        want = sum(ref.executed_flops(L, d, block, sel[h]) for h in range(3))
        assert abs((ex + tile + ap) - want) <= 1e-9 * want


def test_traffic_is_used_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    src = tmp_path / "attn.hip"
    src.write_text("kernel source\n")
    prof = tmp_path / "traffic.json"
    hdr = tmp_path / "common.hpp"
    hdr.write_text("helpers\n")
    prof.write_text(json.dumps({"kernel_sources_sha256_16": bench.source_hash([str(src), str(hdr)]),
                                "hbm_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src), str(hdr)])
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(prof))
    assert bench.measured_traffic() == 123
    hdr.write_text("helpers, changed\n")
    assert bench.measured_traffic() is None
    hdr.write_text("helpers\n")
    assert bench.measured_traffic() == 123
    src.write_text("kernel source, changed\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_committed_traffic_matches_the_committed_kernel():
    # the counters under profiles/ were taken on the fused kernel as it is
    assert bench.measured_traffic() is not None
