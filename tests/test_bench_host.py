"""bench.py's host logic on the CPU: the work each stage is charged with, the roofline
arithmetic, the lookup of recorded HBM traffic, the one-GPU guard and the host record."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_stage_work_of_the_large_layer():
    w = W.BY_NAME["large_bf16_S32768_M4096_E128_k8_H1536"]
    C, kept = 4096, 240711
    st = bench.algorithmic(w, C, kept)
    # every expert GEMM of forward and backward is one M x H product over the kept rows
    for name in ("fc1", "fc2", "fc2_bwd_data", "fc2_wgrad", "fc1_bwd_data", "fc1_wgrad"):
        assert st[name] == ("flops", 2 * 4096 * 1536 * kept), name
    # encode writes every row of the [E*C, M] buffer (padding included) and reads x once
    kind, enc = st["encode"]
    assert kind == "bytes" and enc == 32768 * 4096 * 2 + 128 * C * 4096 * 2 + 8 * 8 * 32768
    # decode reads the kept rows and writes the output; the encode backward the same shapes
    assert st["decode"][1] == kept * 4096 * 2 + 32768 * 4096 * 2 + 12 * 8 * 32768
    assert st["encode_bwd"][1] == kept * 4096 * 2 + 32768 * 4096 * 2 + 8 * 8 * 32768
    # the decode backward reads dout once and the kept y rows, writes the kept dy rows
    assert st["decode_bwd"][1] == 32768 * 4096 * 2 + 2 * kept * 4096 * 2 + 16 * 8 * 32768
    assert "gate" not in st  # the large layer takes its logits as input


def test_gate_stages_only_with_a_projected_gate():
    g = bench.algorithmic(W.BY_NAME["gated_train_bf16_S4096_M1024_E8_k2_H4096"], 1280, 8192)
    assert g["gate"] == ("bytes", 4096 * 1024 * 2 + 4 * 1024 * 8 + 4 * 4096 * 8)
    assert "gate_wgrad" in g and "fc1_wgrad" in g
    f = bench.algorithmic(W.BY_NAME["gated_bf16_S4096_M1024_E8_k2_H4096"], 1280, 8192)
    assert "fc1_wgrad" not in f and "decode_bwd" not in f


def test_roofline_arithmetic():
    r = bench.roofline_of("bytes", 8e9, 2.0)  # 8 GB in 2 ms = 4 TB/s
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0) and r["frac"] == pytest.approx(0.5)
    r = bench.roofline_of("flops", 2.5e12, 2.0)  # 2.5 TFLOP in 2 ms = 1.25 PFLOP/s
    assert r["bound"] == "mfma" and r["peak"] == bench.MFMA_BF16_PEAK_TFS
    assert r["frac"] == pytest.approx(0.5)
    assert bench.roofline_of("flops", 5e12, 2.0, mx=True)["frac"] == pytest.approx(0.5)  # fp8 peak
    r = bench.roofline_of("flops", 1.573e11, 2.0, dtype_bf16=False)  # fp32 data: vector ALU peak
    assert r["bound"] == "alu" and r["frac"] == pytest.approx(0.5)


def _traffic_file(root, stage, sha, traffic=123456789):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"traffic_{stage}_wl.md"), "w") as f:
        f.write(f"# x\n\n- stage: `{stage}`\n- sources_sha256: `{sha}`\n- traffic_bytes_per_launch: `{traffic}`\n")


def test_recorded_traffic_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    root = str(tmp_path)
    for rel in set(bench.GEMM_SOURCES) | set(bench.ROW_SOURCES):
        os.makedirs(os.path.dirname(os.path.join(root, rel)), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), os.path.join(root, rel))
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.recorded_traffic("fc1", "wl") is None  # no file
    _traffic_file(root, "fc1", bench.sources_sha256("fc1"))
    assert bench.recorded_traffic("fc1", "wl") == 123456789
    _traffic_file(root, "fc1", "0" * 64)  # taken on other sources
    assert bench.recorded_traffic("fc1", "wl") is None
    # a GEMM stage's record does not depend on the row-copy kernels' file, and vice versa
    _traffic_file(root, "fc2_wgrad", bench.sources_sha256("fc2_wgrad"))
    _traffic_file(root, "decode", bench.sources_sha256("decode"))
    with open(os.path.join(root, "combine_softmax_top_amd/csrc/dispatch.hip"), "a") as f:
        f.write("\n// edited\n")
    assert bench.recorded_traffic("fc2_wgrad", "wl") == 123456789
    assert bench.recorded_traffic("decode", "wl") is None


def test_committed_traffic_records_are_well_formed():
    d = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(d) if f.startswith("traffic_")]
    assert files
    for f in files:
        text = open(os.path.join(d, f)).read()
        stage = f[len("traffic_"):].split("_large_")[0].split("_gated_")[0]
        assert f"- stage: `{stage}`" in text, f
        assert "- sources_sha256: `" in text and "- traffic_bytes_per_launch: `" in text, f
        assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text, f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_host_record():
    h = bench.host_info()
    assert h["nproc"] >= 1 and 1 <= h["affinity_cores"] <= h["nproc"]
    assert isinstance(h["cpu_model"], str)
