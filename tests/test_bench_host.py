"""Host-side checks of bench.py (CPU only): the one-GPU contract, the lookup of
committed traffic counters, and the oracle legs of the CPU baseline."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_paged_kv_nvfp4_amd import workload as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_committed_traffic_lookup():
    # the committed counter summary matches the split kernel's current sources
    t = bench.committed_traffic("llama70b_layer_32k_b44", 47)
    assert t is None or t > 1_660_944_384  # at least the KV bytes when present
    # no summary for another split count or workload
    assert bench.committed_traffic("llama70b_layer_32k_b44", 46) is None
    assert bench.committed_traffic("no_such_workload", 47) is None


def test_cpu_extend_baseline_runs():
    w = W.config(5)
    r = bench.cpu_extend_baseline(w, W, torch, prefix_sample=1024)
    assert r["kind"] == "oracle" and r["cores"] >= 1
    assert r["quantize_chunk"]["value"] > 0 and r["dequant_prefix"]["value"] > 0
    assert "1024 of 163840" in r["dequant_prefix"]["sample"]
