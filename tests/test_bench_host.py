"""Host logic of bench.py (no GPU): the kernel-code hash that keys the
committed counter record, the record's use, the algorithmic byte and flop
counts, the kernel name per workload, and the one-GPU refusal."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_sha_ignores_comments_and_blank_lines(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int x = 1;  // one\n\n// note\nint y = 2;\n")
    b = tmp_path / "b.hip"
    b.write_text("int x = 1;  // a different comment\nint y = 2;   \n\n")
    c = tmp_path / "c.hip"
    c.write_text("int x = 1;\nint y = 3;\n")
    assert bench.code_sha(a) == bench.code_sha(b)
    assert bench.code_sha(a) != bench.code_sha(c)


def test_traffic_record_used_only_on_the_same_code_and_workload(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int k = 0;\n")
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"workload": "w", "kernel_code_sha": bench.code_sha(src),
                               "hbm_bytes_per_launch": 1234}))
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.load_traffic("w") == 1234
    assert bench.load_traffic("other") is None
    src.write_text("int k = 1;\n")          # the kernel changed: no record
    assert bench.load_traffic("w") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic("w") is None


def test_committed_traffic_record():
    """The committed record is well formed and scaled from its counters;
    taken on other kernel code it is skipped here (and the bench line
    carries traffic = null until the counters are taken again)."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["workload"] == workloads.get("c3").name
    cal = t["copy_calibration"]
    kib = t["fetch_size_kib_per_dispatch"] * cal["fetch_scale"] + \
        t["write_size_kib_per_dispatch"] * cal["write_scale"]
    assert abs(kib * 1024 - t["hbm_bytes_per_launch"]) < 1e-4 * t["hbm_bytes_per_launch"]
    assert 0.99 < t["hbm_bytes_per_launch"] / t["algorithmic_bytes_per_launch"] < 1.05
    if t["kernel_code_sha"] != bench.code_sha(bench.ATTN_SRC):
        pytest.skip("the counter record was taken on other kernel code")


@pytest.mark.parametrize("dtype,e", [("bf16", 2), ("f32", 4)])
def test_attention_bytes_and_flops_tensor_by_tensor(dtype, e):
    cfg = workloads.scaled(workloads.get("c2"), batch=3, block=5, hq=6, hkv=2, head_dim=64,
                           dtype=dtype)
    plen = np.array([7, 0, 40])
    n, blk, hq, hkv, d = 3, 5, 6, 2, 64
    tensors = {
        "q": n * blk * hq * d * e, "out": n * blk * hq * d * e,
        "k_blk": n * blk * hkv * d * e, "v_blk": n * blk * hkv * d * e,
        "k_cache": int(plen.sum()) * hkv * d * e, "v_cache": int(plen.sum()) * hkv * d * e,
        "imp": n * hq * blk * 4,
    }
    assert bench.attn_bytes(cfg, plen) == sum(tensors.values())
    assert bench.attn_bytes(cfg, plen, with_lse=True) == sum(tensors.values()) + n * hq * blk * 4
    no_v = sum(v for k, v in tensors.items() if k not in ("out", "v_blk", "v_cache"))
    assert bench.attn_bytes(cfg, plen, with_out=False) == no_v
    # Q K^T and P V: one multiply-add per (query row, key, d) each, per head
    macs = sum(hq * blk * (int(p) + blk) * d for p in plen) * 2
    assert bench.attn_flops(cfg, plen) == 2 * macs


def test_kernel_names_per_workload():
    assert bench.attn_kernel_name(workloads.get("c3")) == "attn_bf16_kernel<false, 1, true, false, 2>"
    assert bench.attn_kernel_name(workloads.get("c6")) == "attn_bf16_kernel<false, 2, true, false, 2>"
    assert bench.attn_kernel_name(workloads.get("c4")) == "attn_bf16_kernel<false, 4, true, false, 0>"
    assert bench.attn_kernel_name(workloads.get("c1")) == "attn_kernel (generic)"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
