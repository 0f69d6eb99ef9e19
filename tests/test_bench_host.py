"""Host-side checks of bench.py (CPU only): the one-GPU contract, the lookup of
committed traffic counters, and the oracle legs of the CPU baseline."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_paged_kv_nvfp4_amd import binding as B  # noqa: E402
from bit_paged_kv_nvfp4_amd import workload as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_committed_traffic_lookup():
    # every decode workload bench.py times has a counter summary taken on the
    # split kernel's current sources (re-take them after changing the kernel);
    # its bytes are at least the KV bytes and within 2% of them
    for c in (2, 3, 4, 5):
        w = W.config(c)
        splits = w.num_splits or B.nvfp4_paged_decode_attn_default_splits(w.batch, w.num_kv_heads, w.max_seq_len)
        t = bench.committed_traffic(w.name, splits)
        assert t is not None, f"no current traffic summary for {w.name} ({splits} splits)"
        kv = w.kv_bytes_per_step()
        assert kv < t < 1.02 * kv, (w.name, t, kv)
    # no summary for another split count or workload
    assert bench.committed_traffic("llama70b_layer_32k_b44", 46) is None
    assert bench.committed_traffic("no_such_workload", 47) is None


def test_committed_traffic_skips_stale_summaries(tmp_path, monkeypatch):
    # a summary whose source hash no longer matches is passed over, also when
    # a current one for the same workload follows it
    import hashlib
    import shutil

    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel")
    cur = hashlib.sha256(b"kernel").hexdigest()
    for name, sha, val in (("a", "0" * 64, 1), ("b", cur, 2)):
        (tmp_path / "profiles" / f"k_decode_split_{name}_traffic.md").write_text(
            f"x\n\n    kernel: k_decode_split\n    kernel_source: k.hip\n    kernel_source_sha256: {sha}\n"
            f"    workload: wl\n    num_splits: 8\n    traffic_bytes_per_launch: {val}\n")
    shutil.copy(bench.__file__, tmp_path / "bench.py")
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_copy", tmp_path / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.committed_traffic("wl", 8) == 2
    (tmp_path / "profiles" / "k_decode_split_b_traffic.md").unlink()
    assert mod.committed_traffic("wl", 8) is None


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


def test_trace_decode_phases(tmp_path, capsys):
    # a synthetic trace in decode_step()'s launch order: 1 warm-up pair, then
    # 3 passes of 2 fused + 2 three-launch steps, then 2 kernel-timing steps
    import json

    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp,Grid_Size_X"]
    t = [0]

    def launch(name, d):
        rows.append(f'"void nvfp4kv::(anonymous namespace)::{name}(nvfp4kv::DecodeArgs)",{t[0]},{t[0] + d},64')
        t[0] += d + 5

    launch("k_quantize", 50)  # the pool fill before the step
    split = iter(range(1000, 2000, 10))

    def fused():
        launch("k_decode_split", next(split))
        launch("k_decode_combine", 20)

    def three():
        launch("k_quantize", 30)
        launch("k_decode_split", next(split))
        launch("k_decode_combine", 20)

    fused()
    three()
    for _ in range(3):
        fused()
        fused()
        three()
        three()
    fused()
    fused()
    launch("k_decode_split_fp8", 700)  # another kernel after the step
    (tmp_path / "run").mkdir()
    (tmp_path / "run" / "x_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.trace_summary(str(tmp_path), 0, steps=2, warmup=1)
    ph = json.loads(capsys.readouterr().out)["decode_phases"]
    assert [p["phase"] for p in ph][0].startswith("warm-up") and len(ph) == 8
    assert [p["steps"] for p in ph] == [2, 2, 2, 2, 2, 2, 2, 2]
    # split durations 1000, 1010, ... in launch order
    assert ph[0]["split_mean_us"] == 1.0  # 1000 and 1010 ns
    assert ph[1]["phase"] == "pass 0, fused" and ph[1]["split_min_us"] == 1.0 and ph[1]["split_max_us"] == 1.0
    assert ph[2]["quantize_mean_us"] == 0.0 and ph[1]["quantize_mean_us"] is None
    assert ph[-1]["phase"].startswith("kernel-timing") and ph[-1]["combine_mean_us"] == 0.0
    # a fused step spans split + gap + combine
    assert ph[1]["step_span_mean_us"] == round((1020 + 5 + 20 + 1030 + 5 + 20) / 2 / 1000, 1)
    # too few steps in the trace: no phases
    bench.trace_summary(str(tmp_path), 0, steps=5, warmup=1)
    assert json.loads(capsys.readouterr().out)["decode_phases"] == []


def test_cpu_baseline_sample_is_bounded():
    # the sample is whole sequences within the token budget, at least one
    w = W.config(4)
    n, tok = 0, 0
    while n < w.batch and (n == 0 or tok + int(w.seq_lens[n]) <= 786432):
        tok += int(w.seq_lens[n])
        n += 1
    assert n == 4 and tok == 4 * 163840
