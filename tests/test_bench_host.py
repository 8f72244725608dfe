"""Host logic of bench.py that needs no GPU: the one-GPU guard, the
ideal-traffic model, input rotation, the kernel-source hash that keeps stored
counters honest, and the traffic lookup."""
import json
import os
import subprocess
import sys

import pytest

import bench
from dense_gemm_tn_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_read_once_write_once():
    W = inputs.WORKLOADS
    assert bench.algorithmic_bytes(W["f16_4096"]) == 3 * 4096 * 4096 * 2
    assert bench.algorithmic_bytes(W["f8_8192"]) == 2 * 8192 * 8192 + 8192 * 8192 * 2
    assert bench.algorithmic_bytes(W["qkt_64x4096x4096x128"]) == \
        64 * (2 * 4096 * 128 * 2 + 4096 * 4096 * 2)
    assert bench.algorithmic_bytes(W["attn_64x4096x4096x128"]) == 64 * 4 * 4096 * 128 * 2
    assert bench.algorithmic_bytes(W["f16_512x512x32768_splitk"]) == \
        2 * 512 * 32768 * 2 + 512 * 512 * 2


def test_rotation_exceeds_the_last_level_cache():
    for w in inputs.WORKLOADS.values():
        R = bench.rotation_sets(w)
        assert 1 <= R <= 8
        assert R == 8 or R * bench.algorithmic_bytes(w) >= 512 * 2 ** 20


def test_flops_count_two_per_multiply_add():
    W = inputs.WORKLOADS
    assert W["f16_4096"].flops == 2 * 4096 ** 3
    assert W["attn_64x4096x4096x128"].flops == 64 * 4 * 4096 * 4096 * 128


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "source_file", lambda kind: str(src))
    src.write_text("int f() { return 1; }  // one\n/* block */\n\n")
    h0 = bench.source_hash()
    src.write_text("// header\nint f() { return 1; }   // changed comment\n")
    assert bench.source_hash() == h0
    src.write_text("int f() { return 2; }\n")
    assert bench.source_hash() != h0


def test_traffic_lookup_needs_matching_source(tmp_path, monkeypatch):
    w = inputs.WORKLOADS["f16_4096"]
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_for("f16_4096", w, 1e-4) is None          # no file
    entry = {"hbm_bytes_per_launch": 123.0, "source_sha256_16": bench.source_hash("f16")}
    path.write_text(json.dumps({"workloads": {"f16_4096": entry}}))
    assert bench.traffic_for("f16_4096", w, 1e-4) == 123.0
    entry["source_sha256_16"] = "0" * 16                              # taken on other code
    path.write_text(json.dumps({"workloads": {"f16_4096": entry}}))
    assert bench.traffic_for("f16_4096", w, 1e-4) is None
    path.write_text("not json")
    assert bench.traffic_for("f16_4096", w, 1e-4) is None


@pytest.mark.parametrize("name", sorted(inputs.WORKLOADS))
def test_every_workload_names_its_kernel(name):
    assert bench.kernel_name(inputs.WORKLOADS[name])
