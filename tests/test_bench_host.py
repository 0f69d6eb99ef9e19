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


def test_headline_is_the_largest_decode_workload():
    a = bench.parse([])
    assert a.config == 4 and a.gpus == 1
    kv = {c: W.config(c).kv_bytes_per_step() for c in range(1, 6)}
    assert max(kv, key=kv.get) == a.config
    assert sorted(int(x) for x in a.workloads.split(",")) == [1, 2, 3, 5]


def test_trace_summary_of_a_kernel_trace(tmp_path, capsys):
    import json

    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp,Grid_Size_X"]
    t = 0
    for i, d in enumerate([900, 500, 400, 410, 420]):
        rows.append(f'"void nvfp4kv::(anonymous namespace)::k_decode_split(nvfp4kv::DecodeArgs)",{t},{t + d},1024')
        t += d + 10
    rows.append(f"__amd_rocclr_copyBuffer,{t},{t + 5},64")
    (tmp_path / "run").mkdir()
    (tmp_path / "run" / "x_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.trace_summary(str(tmp_path), 2)
    out = json.loads(capsys.readouterr().out)
    assert list(out) == ["k_decode_split"]
    k = out["k_decode_split"]
    assert k["launches"] == 5 and k["steady_launches"] == 3 and k["steady_mean_ns"] == 410 and k["max_ns"] == 900


def test_cpu_baseline_sample_is_bounded():
    # the sample is whole sequences within the token budget, at least one
    w = W.config(4)
    n, tok = 0, 0
    while n < w.batch and (n == 0 or tok + int(w.seq_lens[n]) <= 786432):
        tok += int(w.seq_lens[n])
        n += 1
    assert n == 4 and tok == 4 * 163840
