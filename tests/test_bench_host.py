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


# The instantiation each workload's launch dispatches on a 256-CU part (the
# library's selector, ring depth and whole-K-step choice), as the kernel traces
# under profiles/ recorded it; every one is a kernel the build compiles.
DISPATCHED = {
    "f16_4096": "gemm_tn_ring_kernel<0, 8, true>",
    "f8_8192": "gemm_tn_ring_kernel<1, 8, true>",
    "f16_1920x13900x4096": "gemm_tn_ring_kernel<0, 7, true>",
    "qkt_64x4096x4096x128": "gemm_tn_skinny_kernel<0>",
    "f16_256_pm1": "gemm_tn_mid_kernel<0, false, false, false, 2, true>",
    "f16_2048": "gemm_tn_mid_kernel<0, false, false, false, 4, true>",
    "f16_512x512x32768": "gemm_tn_mid_kernel<0, false, false, false, 4, true>",
    "f16_512x512x32768_splitk": "gemm_tn_mid_kernel<0, false, false, true, 4, true>",
    "f16_nn_4096": "gemm_tn_kernel<0, 8, true, false, false>",
    "f8_nt_8192": "gemm_tn_kernel<1, 8, true, true, false>",
}


@pytest.mark.parametrize("name", sorted(DISPATCHED))
def test_kernel_names_match_dispatch(name):
    import os

    assert bench.kernel_name(inputs.WORKLOADS[name]) == DISPATCHED[name]
    report = open(os.path.join(os.path.dirname(bench.__file__), "profiles",
                               "kernel_resources.md")).read()
    assert "dg::%s(dg::Params)" % DISPATCHED[name] in report


def test_default_list_starts_with_the_five_configurations():
    five = ("f16_4096", "f8_8192", "f16_256_pm1", "f16_1920x13900x4096", "qkt_64x4096x4096x128")
    assert bench.DEFAULT_WORKLOADS[:5] == five
    assert all(n in inputs.WORKLOADS for n in bench.DEFAULT_WORKLOADS)
    assert len(set(bench.DEFAULT_WORKLOADS)) == len(bench.DEFAULT_WORKLOADS)


def test_clock_summary_from_records():
    import numpy as np
    # Block 0 on XCD 0: 2000 shader ticks in 100 real ticks (2 GHz), with the
    # loop from real tick 10 to 90; block 1 on XCD 1 at 1.5 GHz without loop
    # points; an empty record is skipped.
    rec = np.array([[10, 0, 30, 10, 1830, 90, 2010, 100, 0, 0],
                    [100, 50, 0, 0, 0, 0, 1600, 150, 1, 1],
                    [0] * 10], dtype=np.uint64)
    c = bench.clock_summary(rec)
    assert c["blocks"] == 2
    assert c["sclk_mhz_per_xcd"] == {0: 2000.0, 1: 1500.0}
    assert c["sclk_mhz"] == 1750.0 and c["block_us_median"] == 1.0
    assert "loop_us_median" not in c           # block 1 has no loop points
    c = bench.clock_summary(rec[:1])
    assert c["prologue_us_median"] == 0.1 and c["loop_us_median"] == 0.8
    assert c["epilogue_us_median"] == 0.1 and c["loop_sclk_mhz"] == 2250.0
    assert bench.clock_summary(np.zeros((3, 10), np.uint64)) is None


def test_launch_spans_from_records():
    import numpy as np
    rec = np.zeros((4, 10), np.uint64)
    # launch 0: blocks from 100..300 and 120..350 ticks -> 2.5 us; launch 1: 1000..1400 -> 4 us
    rec[0, [1, 7]] = [100, 300]
    rec[1, [1, 7]] = [120, 350]
    rec[2, [1, 7]] = [1000, 1300]
    rec[3, [1, 7]] = [1100, 1400]
    s = bench.launch_spans_us(rec, 2)
    assert s == {"median": 3.25, "min": 2.5, "max": 4.0, "launches": 2}
    rec[3, 7] = 0                                  # an unfinished record drops its launch
    assert bench.launch_spans_us(rec, 2)["launches"] == 1


def test_processes_option_is_stripped_for_children():
    assert bench.strip_processes(["--steps", "5", "--processes", "3", "--no-cpu"]) == \
        ["--steps", "5", "--no-cpu"]
    assert bench.strip_processes(["--processes=2", "--workload", "f16_4096"]) == \
        ["--workload", "f16_4096"]


def test_merge_processes_reports_the_median_process():
    def line(ms, med, cpu):
        w = {"tflops": 1.0 / ms, "ms_per_step": ms, "frac_of_peak": 0.5,
             "per_launch_us": {"median": med, "min": med, "max": med},
             "roofline": {"bound": "mfma", "achieved": 1.0 / ms, "peak": 2.0, "unit": "x",
                          "frac": 0.5 / ms, "traffic": None, "kernel": "k"},
             "clock": {"sclk_mhz": 2000.0 + ms}}
        return {"metric": "m", "value": 1.0 / ms, "ms_per_step": ms, "parity_ok": True,
                "config": {"workload": "f16_4096"}, "cpu_baseline": cpu,
                "workloads": {"f16_4096": w}}
    merged = bench.merge_processes([line(0.30, 300.0, {"v": 1}), line(0.10, 100.0, None),
                                    line(0.20, 210.0, None)])
    w = merged["workloads"]["f16_4096"]
    assert merged["ms_per_step"] == 0.20 and merged["value"] == 5.0   # the median process
    assert w["processes"]["reported_process"] == 2
    assert w["processes"]["ms_per_step"] == [0.30, 0.10, 0.20]
    assert w["processes"]["median_of_medians_us"] == 210.0
    assert w["processes"]["range_of_medians_us"] == [100.0, 300.0]
    assert merged["cpu_baseline"] == {"v": 1} and merged["processes"] == 3
    assert merged["clock"]["sclk_mhz"] == 2000.2
