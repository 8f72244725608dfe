#!/usr/bin/env python3
"""Throughput of the gfx950 TN GEMM (and fused attention) on synthetic inputs in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME ...] [--no-cpu]

A step is one launch of the GEMM over one set of inputs (A, B -> C).  Inputs
are generated on the host with fixed seeds, copied to HBM before timing, and
rotated over R buffer sets so the working set exceeds the 256 MB last-level
cache (the method of the MI355X FP8 GEMM page: warm-up runs, timed runs,
normally distributed data, rotating buffers).  Per workload:
  1. every set is launched once and set 0's output is checked against the CPU
     oracle on sampled entries (parity before timing; exact on +-1 data);
  2. W untimed steps, then exactly K timed steps bracketed by
     torch.cuda.synchronize(); HIP events recorded on the launch stream give
     the average kernel duration (`ms_per_step`), from which
     throughput = 2*M*N*K per step / time (section 11.1 of the hello-gpu
     chapter counts a multiply-add as two flops);
  3. a second pass of the same K launches, back to back, writes per-block
     clock records (gemm_clock_record): each launch's span from its first
     block's start to its last block's end gives the per-launch median / min /
     max (the hello-gpu chapter, section 11.5, reports medians with their
     range); a third pass brackets each launch with its own event pair
     (isolated launches, reported beside it);
  4. set 0 is launched again and its output must equal, bit for bit, the one
     checked in step 1 (parity after timing);
  5. the clock records of step 3 (the kernels' shader-clock and 100 MHz
     counters at each block's start, K-loop start and end, and end, and the XCD
     it ran on) give the clock the kernel actually ran at, overall and per XCD,
     and the split of a block's time into prologue, K loop and epilogue, which
     explains run-to-run and box-to-box spread of a power-limited part.
Before the warm-up steps, each workload runs back to back for --settle-ms
(0.25 s) so timing starts at the clock the load sustains rather than on the
ramp up from idle.  All of this runs in --processes (3) independent processes,
one after another; each workload is reported as measured by the process with
the median time, with every process's mean and per-launch median, the median
of those medians and their range (the hello-gpu chapter, section 11.5: three
processes, median of medians with the range).

Prints ONE JSON line.  The headline `value` is the FP16 TN 4096^3 workload;
every other workload of the default list (the five configurations of the
hot path -- FP16 256^3 +-1, FP16 4096^3, FP16 1920 x 13900 x 4096, FP8 8192^3,
batched QK^T 64 x 4096 x 4096 x 128 -- then the fused attention forward, FP16
2048^3 on the 128 x 128 kernel, the NN/TT/NT op codes, 512 x 512 x 32768
without and with split-K, and the 8-wave ping-pong kernel) is reported under
"workloads".  `roofline` is for the FP16 kernel (the QK^T workload carries an
HBM roofline of its own); `traffic` comes from a stored rocprofv3 counter
summary and is null when the kernel source changed after the counters were
taken.  `cpu_baseline` times the CPU oracle on a bounded column sample of the
headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % of dense MFMA peak: FP16 TN 4096^3, FP8 e4m3 8192^3"
# Published MI355X dense peaks: 256 CUs x 2.4 GHz x 4096 (fp16) / 8192 (fp8) flop/clk/CU.
PEAK_TFLOPS = {"f16": 2516.6, "qkt": 2516.6, "attn": 2516.6, "f8": 5033.2}
HBM_PEAK_GBS = 8000.0


def kernel_name(w):
    """The kernel the library launches for workload w (its configuration
    selector, queried through the C ABI)."""
    import dense_gemm_tn_amd as dg

    if w.kind == "attn":
        return "attention_fwd_kernel"
    kind = 1 if w.kind == "f8" else 0
    layout = w.extra.get("layout", "TN")
    kstep = 128 if w.kind == "f8" else 64

    def tiles128(M, N):
        return ((M + 127) // 128) * ((N + 127) // 128)

    def mid(M, N, batch, K, split=False, splits=1):
        """The 128 x 128 kernel on that grid (its ring depth from the library)."""
        nk = (K + kstep - 1) // kstep
        per = (nk + splits - 1) // splits if nk else 0
        ranges = (nk + per - 1) // per if per else 0
        blocks = tiles128(M, N) * (ranges if split else batch)
        # Whole K-steps (K a multiple of the K-step) take the fixed-offset form.
        return "gemm_tn_mid_kernel<%d, false, false, %s, %d, %s>" % (
            kind, "true" if split else "false", dg.mid_stages(blocks, per if split else nk),
            "true" if K % kstep == 0 else "false")

    if layout != "TN":
        amn = "true" if layout[0] == "N" else "false"
        bmn = "true" if layout[1] == "T" else "false"
        cfg_of = dg.f8_config if w.kind == "f8" else dg.f16_config
        if cfg_of(layout[0], layout[1], w.M, w.N, w.K) == 2:
            nk = (w.K + kstep - 1) // kstep
            return "gemm_tn_mid_kernel<%d, %s, %s, false, %d, false>" % (
                kind, amn, bmn, dg.mid_stages(tiles128(w.M, w.N), nk))
        return "gemm_tn_kernel<%d, 8, %s, %s, false>" % (kind, amn, bmn)
    fp8 = w.kind == "f8"
    if w.extra.get("splitk"):
        s = dg.splitk_choose(w.M, w.N, w.K, fp8=fp8)
        if s > 1:
            return mid(w.M, w.N, 1, w.K, split=True, splits=s)

    # The 256-row TN kernel with whole K-steps (K a multiple of the K-step) is
    # the instantiation with fixed copy offsets (last template flag).
    kf = "true" if w.K % (64 if kind == 0 else 128) == 0 else "false"

    def names(cfg, M, N):
        return {0: "gemm_tn_ring_kernel<%d, 8, %s>" % (kind, kf),
                1: "gemm_tn_ring_kernel<%d, 7, %s>" % (kind, kf),
                3: "gemm_tn_skinny_kernel<%d>" % kind,
                4: "gemm_tn_pp_kernel<%d>" % kind}.get(cfg) or mid(M, N, w.batch, w.K)

    ws = dg.tn_workspace_bytes(w.M, w.N, w.K, fp8=fp8) if w.extra.get("ws") else 0
    plan = dg.tn_plan(w.M, w.N, w.K, w.batch, ws, fp8=fp8)
    if plan["dp_cols"] > 0 or plan["splits"] > 1:
        # Two launches per call (whole rounds of columns, then the rest, or
        # split-K and its reduction): the label names both.
        nt = w.N - plan["dp_cols"]
        split = mid(w.M, nt, 1, w.K, split=True, splits=plan["splits"])
        if plan["dp_cols"] == 0:
            return split
        tail = split if plan["splits"] > 1 else \
            names(dg.tn_config(w.M, nt, w.K, w.batch, fp8=fp8), w.M, nt)
        return "%s + %s" % (names(plan["dp_config"], w.M, plan["dp_cols"]), tail)
    return names(dg.tn_config(w.M, w.N, w.K, w.batch, fp8=fp8), w.M, w.N)


# The five configurations of the hot path first (the headline FP16 4096^3, FP8
# 8192^3, FP16 256^3 +-1, the wide ragged FP16 shape, batched QK^T), then the
# adjacent parts.
DEFAULT_WORKLOADS = (
    "f16_4096", "f8_8192", "f16_256_pm1", "f16_1920x13900x4096", "qkt_64x4096x4096x128",
    "attn_64x4096x4096x128", "f16_2048",
    "f16_nn_4096", "f16_tt_4096", "f16_nt_4096", "f8_nn_8192", "f8_tt_8192", "f8_nt_8192",
    "f16_512x512x32768", "f16_512x512x32768_splitk", "f16_4096_pingpong", "f8_8192_pingpong",
)

CSRC = os.path.join(ROOT, "dense_gemm_tn_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def source_file(kind: str) -> str:
    """The source that holds the kernel of a workload kind."""
    return os.path.join(CSRC, "attention.hip" if kind == "attn" else "gemm_tn.hip")


def source_hash(kind: str = "f16") -> str:
    """Hash of the kernel source's code: comments, blank lines and trailing blanks
    are dropped first, so a documentation-only edit keeps stored counters valid."""
    import re

    text = open(source_file(kind)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Read A and B once, write C once (the ideal-traffic model of section 11.6 of
    the hello-gpu chapter, with 2-byte fp16 / 1-byte fp8 inputs and 2-byte outputs).
    Attention: read Q, K and V once and write O once (M*D + 2*N*D + M*D fp16 per head)."""
    if w.kind == "attn":
        return w.batch * (2 * w.M * w.K + 2 * w.N * w.K) * 2
    es = 1 if w.kind == "f8" else 2
    return w.batch * ((w.M * w.K + w.N * w.K) * es + w.M * w.N * 2)


def rotation_sets(w) -> int:
    per_set = algorithmic_bytes(w)
    return max(1, min(8, -(-512 * 2 ** 20 // per_set)))


def make_launcher(w, dev):
    """Inputs for R rotating sets and a function launching step i on the current stream."""
    import numpy as np
    import torch

    import dense_gemm_tn_amd as dg
    from dense_gemm_tn_amd import inputs

    x = inputs.make(w)
    R = rotation_sets(w)
    layout = w.extra.get("layout", "TN")
    sets = []
    for r in range(R):
        if w.kind == "attn":
            q = torch.from_numpy(x["Q"]).to(dev)
            k = torch.from_numpy(x["K"]).to(dev)
            vt = torch.from_numpy(x["Vt"]).to(dev)
            o = torch.empty((w.batch, w.M, w.K), dtype=torch.float16, device=dev)
            sets.append((q, k, vt, o))
        elif w.kind == "qkt":
            q = torch.from_numpy(x["Q"]).to(dev)
            k = torch.from_numpy(x["K"]).to(dev)
            s = torch.empty((w.batch, w.N, w.M), dtype=torch.float16, device=dev)
            sets.append((q, k, s))
        else:
            # Operands as they lie for the workload's op codes: A 'N' is stored
            # [K, M] (M contiguous), B 'T' [K, N] (N contiguous).
            a = torch.from_numpy(np.ascontiguousarray(x["A"] if layout[0] == "T" else x["A"].T))
            b = torch.from_numpy(np.ascontiguousarray(x["B"] if layout[1] == "N" else x["B"].T))
            a, b = a.to(dev), b.to(dev)
            cdt = torch.float16 if w.kind == "f16" else torch.bfloat16
            c = torch.empty((w.N, w.M), dtype=cdt, device=dev)
            sets.append((a, b, c))

    scale = 1.0 / w.K ** 0.5
    splits, ws, ws_bytes = 1, None, 0
    if w.extra.get("ws"):
        # The planned call with the workspace its plan asks for.
        ws_bytes = dg.tn_workspace_bytes(w.M, w.N, w.K, fp8=(w.kind == "f8"))
        ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device=dev)
    if w.extra.get("splitk"):
        # One workspace serves every set: the launches are ordered on one stream.
        splits = dg.splitk_choose(w.M, w.N, w.K, fp8=(w.kind == "f8"))
        ws_bytes = dg.splitk_workspace_bytes(w.M, w.N, splits)
        ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device=dev)

    def launch(i):
        if w.kind == "attn":
            q, k, vt, o = sets[i % R]
            dg.attention_fwd_f16(q, k, vt, o, w.batch, w.M, w.N, w.K, w.K, w.K, w.N, w.K,
                                 w.M * w.K, w.N * w.K, w.K * w.N, w.M * w.K, scale)
            return
        a, b, c = sets[i % R]
        if w.kind == "f16" and layout != "TN":
            dg.gemm_f16(layout[0], layout[1], a, b, c, w.M, w.N, w.K, a.stride(0), b.stride(0),
                        w.M)
        elif w.kind == "f16" and w.extra.get("ws"):
            dg.gemm_f16_tn_ws(a, b, c, w.M, w.N, w.K, w.K, w.K, w.M, ws, ws_bytes)
        elif w.kind == "f16" and splits > 1:
            dg.gemm_f16_tn_splitk(a, b, c, w.M, w.N, w.K, w.K, w.K, w.M, splits, ws, ws_bytes)
        elif w.kind == "f16":
            dg.gemm_f16_tn(a, b, c, w.M, w.N, w.K, w.K, w.K, w.M)
        elif w.kind == "f8" and layout != "TN":
            dg.gemm_f8(layout[0], layout[1], a, b, c, w.M, w.N, w.K, a.stride(0), b.stride(0),
                       w.M, x["scale_a"], x["scale_b"])
        elif w.kind == "f8":
            dg.gemm_f8_tn(a, b, c, w.M, w.N, w.K, w.K, w.K, w.M, x["scale_a"], x["scale_b"])
        else:
            dg.gemm_batched_qkt(a, b, c, w.batch, w.M, w.N, w.K, w.K, w.K, w.M,
                                w.M * w.K, w.N * w.K, w.M * w.N)

    return x, sets, launch, R


CLOCK_WORDS = 10   # uint64 words per block record (see gemm_clock_record)


def clock_summary(rec) -> dict | None:
    """Per-block clock records (see gemm_clock_record: shader-clock ticks and
    100 MHz real-time ticks at the block's start, K-loop start, K-loop end and
    end, and its XCD) -> the clock the blocks ran at: time-weighted MHz overall
    and per XCD, the median and range of per-block MHz, the median block
    duration and, for kernels with a pipelined K loop, the median prologue,
    loop and epilogue durations (microseconds) and the loop's own clock."""
    import numpy as np

    rec = np.asarray(rec, dtype=np.uint64).reshape(-1, CLOCK_WORDS)
    t = (rec[:, 6] - rec[:, 0]).astype(np.float64)
    r = (rec[:, 7] - rec[:, 1]).astype(np.float64)
    ok = (rec[:, 6] > rec[:, 0]) & (rec[:, 7] > rec[:, 1]) & (rec[:, 0] > 0)
    if not ok.any():
        return None
    rec, t, r = rec[ok], t[ok], r[ok]
    xcd = rec[:, 8].astype(np.int64)
    mhz = t / r * 100.0                       # real-time counter: 100 MHz
    per_xcd = {int(x): float(t[xcd == x].sum() / r[xcd == x].sum() * 100.0)
               for x in np.unique(xcd)}
    out = {
        "blocks": int(ok.sum()),
        "sclk_mhz": float(t.sum() / r.sum() * 100.0),
        "sclk_mhz_block_median": float(np.median(mhz)),
        "sclk_mhz_block_min": float(mhz.min()),
        "sclk_mhz_block_max": float(mhz.max()),
        "sclk_mhz_per_xcd": per_xcd,
        "block_us_median": float(np.median(r) / 100.0),
    }
    looped = (rec[:, 2] >= rec[:, 0]) & (rec[:, 4] >= rec[:, 2]) & (rec[:, 6] >= rec[:, 4]) & \
        (rec[:, 3] > 0) & (rec[:, 5] > 0)
    if looped.all():
        rr = rec[:, 1::2].astype(np.float64)       # real-time ticks at the four points
        tt = rec[:, 0::2][:, :4].astype(np.float64)
        out["prologue_us_median"] = float(np.median(rr[:, 1] - rr[:, 0]) / 100.0)
        out["loop_us_median"] = float(np.median(rr[:, 2] - rr[:, 1]) / 100.0)
        out["epilogue_us_median"] = float(np.median(rr[:, 3] - rr[:, 2]) / 100.0)
        out["loop_sclk_mhz"] = float((tt[:, 2] - tt[:, 1]).sum() / (rr[:, 2] - rr[:, 1]).sum()
                                     * 100.0)
    return out


def launch_spans_us(rec, blocks: int) -> dict | None:
    """Per-launch durations from clock records taken in launch order: for each
    launch, the first block's start to the last block's end on the 100 MHz
    counter (microseconds) -> median, min, max and count."""
    import numpy as np

    rec = np.asarray(rec, dtype=np.uint64).reshape(-1, CLOCK_WORDS)
    n = rec.shape[0] // blocks if blocks > 0 else 0
    spans = []
    for j in range(n):
        r = rec[j * blocks:(j + 1) * blocks]
        ok = (r[:, 7] > r[:, 1]) & (r[:, 1] > 0)
        if ok.all():
            spans.append(float(r[:, 7].max() - r[:, 1].min()) / 100.0)
    if not spans:
        return None
    spans.sort()
    return {"median": float(np.median(spans)), "min": spans[0], "max": spans[-1],
            "launches": len(spans)}


def sample_check(w, x, out):
    """The GPU output of set 0 against the oracle on sampled entries: corners,
    tile edges and seeded random entries (attention: sampled query rows of the
    first and last head).  Returns {"entries", "max_rel_err" or "inexact",
    "ok"} -- +-1 data must be exact, other data within the output format's bar
    relative to the largest sampled reference value."""
    import numpy as np
    import torch

    import oracle

    rng = np.random.default_rng(7)
    if w.kind == "attn":
        D, scale = w.K, 1.0 / w.K ** 0.5
        worst, n = 0.0, 0
        for h in sorted({0, w.batch - 1}):
            rows = np.unique(np.concatenate([[0, w.M - 1], rng.integers(0, w.M, 6)]))
            ref = oracle.attention_rows(x["Q"][h], x["K"][h], x["Vt"][h], w.N, D, rows, scale)
            got = out[h][torch.from_numpy(rows).to(out.device)].float().cpu().numpy()
            bound = 1e-3 * np.abs(x["Vt"][h].astype(np.float64)).max() + 2e-3 * np.abs(ref) + 1e-5
            worst = max(worst, float(np.max(np.abs(got - ref) / bound)))
            n += ref.size
        return {"entries": n, "max_err_over_bound": worst, "ok": worst <= 1.0}
    edges_m = sorted({0, 1, 15, 16, 127, 128, 255, 256, w.M // 2, w.M - 1} & set(range(w.M)))
    edges_n = sorted({0, 1, 15, 16, 127, 128, 255, 256, w.N // 2, w.N - 1} & set(range(w.N)))
    ms = np.array([m for m in edges_m for _ in edges_n] + list(rng.integers(0, w.M, 256)))
    ns = np.array([n for _ in edges_m for n in edges_n] + list(rng.integers(0, w.N, 256)))
    if w.kind == "qkt":
        pairs = [(x["Q"][h], x["K"][h], out[h]) for h in sorted({0, w.batch - 1})]
        fmt_in, fmt_out, scale = oracle.FMT_F16, oracle.FMT_F16, 1.0
    else:
        pairs = [(x["A"], x["B"], out)]
        fmt_in = oracle.FMT_E4M3FN if w.kind == "f8" else oracle.FMT_F16
        fmt_out = oracle.FMT_BF16 if w.kind == "f8" else oracle.FMT_F16
        scale = float(x["scale_a"]) * float(x["scale_b"]) if w.kind == "f8" else 1.0
    err, top, inexact, n = 0.0, 0.0, 0, 0
    idx_n = torch.from_numpy(ns).to(out.device)
    idx_m = torch.from_numpy(ms).to(out.device)
    for A, B, c in pairs:
        ref = oracle.gemm_tn_entries(A, B, fmt_in, w.K, ms, ns, scale=scale)
        codes = c.view(torch.int16)[idx_n, idx_m].cpu().numpy().view(np.uint16)
        got = oracle.decode(codes, fmt_out)
        err = max(err, float(np.max(np.abs(got - ref))))
        top = max(top, float(np.max(np.abs(ref))))
        want = oracle.decode(oracle.encode(ref, fmt_out), fmt_out)
        inexact += int(np.sum(got != want))
        n += ref.size
    if w.dist == "pm1":
        return {"entries": n, "inexact": inexact, "ok": inexact == 0}
    rel = err / top if top > 0 else err
    bar = 1e-2 if w.kind == "f8" else 4e-3
    return {"entries": n, "max_rel_err": rel, "ok": rel <= bar}


def time_workload(w, steps, warmup, dev, check=True, settle_s=0.25):
    import statistics as st

    import torch

    import dense_gemm_tn_amd as dg

    x, sets, launch, R = make_launcher(w, dev)
    # Parity before timing: every set is launched once (its buffers are then
    # in use before the timed region), set 0's output is checked and kept.
    for i in range(R):
        launch(i)
    torch.cuda.synchronize()
    out0 = sets[0][-1]
    before = sample_check(w, x, out0) if check else None
    ref_bits = out0.clone()
    # Settle: back-to-back launches for a fixed time before the warm-up steps,
    # so the timed steps start at the clock the load sustains, not on the ramp
    # up from idle (the MI355X FP8 GEMM page warms up with 1000 launches).
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < settle_s:
        for _ in range(4):
            launch(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        launch(i)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Second pass: the same K launches back to back with per-block clock
    # records (one launch first, to learn its block count).  Each launch's
    # span, first block start to last block end on the 100 MHz counter, gives
    # the per-launch distribution without host-side gaps between launches.
    probe = torch.zeros(CLOCK_WORDS, dtype=torch.int64, device=dev)
    dg.clock_record(probe, 1)
    launch(0)
    torch.cuda.synchronize()
    blocks = dg.clock_records_used()
    n_rec = min(steps, max(1, (256 << 20) // (8 * CLOCK_WORDS * blocks)))
    recs = torch.zeros((n_rec * blocks, CLOCK_WORDS), dtype=torch.int64, device=dev)
    dg.clock_record(recs, n_rec * blocks)
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record()
    for i in range(steps):
        launch(i)
    r1.record()
    torch.cuda.synchronize()
    dg.clock_record(None, 0)
    rec_np = recs.cpu().numpy().view("uint64")
    clock = clock_summary(rec_np)
    spans = launch_spans_us(rec_np, blocks)
    if clock is not None:
        clock["launches_recorded"] = n_rec
        clock["ms_per_step_recorded_pass"] = r0.elapsed_time(r1) / steps
    del recs, probe
    # Third pass: each launch bracketed by its own event pair.  The event
    # packets leave the GPU idle for some microseconds between launches, and
    # launches that start from idle run measurably slower than back-to-back
    # ones, so this distribution is reported beside the others, not as the
    # per-launch figure.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        launch(i)
        e1.record()
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)   # microseconds
    # Parity after timing: set 0 again, bit for bit the output checked before.
    launch(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(out0, ref_bits))
    del ref_bits
    ev_ms = start.elapsed_time(stop)
    kernel_s = ev_ms / 1e3 / steps
    tflops = w.flops / kernel_s / 1e12
    res = {
        "M": w.M, "N": w.N, "K": w.K, "batch": w.batch, "kind": w.kind, "seed": w.seed,
        "dist": w.dist, "rotating_sets": R,
        "settle_launches": n_settle,
        "ms_per_step": ev_ms / steps,
        "wall_ms_per_step": wall * 1e3 / steps,
        "per_launch_us": spans,
        "per_launch_us_isolated": {"median": st.median(per), "min": per[0], "max": per[-1],
                                   "launches": len(per)},
        "tflops": tflops,
        "frac_of_peak": tflops / PEAK_TFLOPS[w.kind],
        "hbm_gbs_algorithmic": algorithmic_bytes(w) / kernel_s / 1e9,
        "clock": clock,
        "parity": {"before": before, "after_bitwise_equal": same},
    }
    return res, x, sets


def traffic_for(name, w, kernel_s):
    """HBM bytes per launch from stored counter runs, if taken on this kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
    except ValueError:
        return None
    ent = t.get("workloads", {}).get(name)
    if not ent or ent.get("source_sha256_16", t.get("source_sha256_16")) != source_hash(w.kind):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(w, x, sets, target_s=10.0):
    """The CPU oracle on a bounded sample: all M rows, full K, the first Ns columns,
    Ns doubling from 64 until one run takes at least target_s seconds or covers
    all N columns.  Also reports the GPU's normwise error on that sample."""
    import numpy as np
    import torch

    import oracle

    threads = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        threads = min(threads, int(env))
    fmt = oracle.FMT_E4M3FN if w.kind == "f8" else oracle.FMT_F16
    scale = float(x["scale_a"]) * float(x["scale_b"]) if w.kind == "f8" else 1.0
    A = x["A"] if w.kind != "qkt" else x["Q"][0]
    B = x["B"] if w.kind != "qkt" else x["K"][0]
    ns = min(64, w.N)
    while True:
        t0 = time.perf_counter()
        ref = oracle.gemm_tn(A, B[:ns], fmt, w.M, ns, w.K, scale=scale, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s or ns >= w.N:
            break
        ns = min(w.N, ns * 2)
    c = sets[0][2] if w.kind != "qkt" else sets[0][2][0]
    got_codes = c[:ns].view(torch.int16).cpu().numpy().view(np.uint16)
    got = oracle.decode(got_codes, oracle.FMT_BF16 if w.kind == "f8" else oracle.FMT_F16)
    err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": 2.0 * w.M * ns * w.K / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%s: all %d rows x first %d of %d columns, full K=%d (%.1f%% of the work)%s; "
                  "%.1f s" % (w.name, w.M, ns, w.N, w.K, 100.0 * ns / w.N,
                              ", head 0 of %d" % w.batch if w.kind == "qkt" else "", dt),
        "cpu_model": model,
        "gpu_max_rel_err_on_sample": err,
    }


def strip_processes(argv):
    """argv without any --processes option (the children get --processes 1)."""
    out, skip = [], False
    for a in argv:
        if skip:
            skip = False
        elif a == "--processes":
            skip = True
        elif not a.startswith("--processes="):
            out.append(a)
    return out


def merge_processes(lines):
    """One line from the lines of several processes (the timing protocol's
    independent processes): each workload as measured by the process with the
    median ms_per_step, plus every process's mean and per-launch median, the
    median of those medians and their range; the CPU baseline from the first
    process (the others skip it)."""
    import statistics

    P = len(lines)
    first = lines[0]
    merged = {}
    for name in first["workloads"]:
        recs = [ln["workloads"][name] for ln in lines]
        ms = [r["ms_per_step"] for r in recs]
        mid = sorted(range(P), key=lambda i: ms[i])[P // 2]
        r = dict(recs[mid])
        meds = [rr["per_launch_us"]["median"] for rr in recs if rr.get("per_launch_us")]
        r["processes"] = {
            "count": P,
            "reported_process": mid,
            "ms_per_step": ms,
            "per_launch_median_us": meds,
            "median_of_medians_us": statistics.median(meds) if meds else None,
            "range_of_medians_us": [min(meds), max(meds)] if meds else None,
        }
        merged[name] = r
    head = first["config"]["workload"]
    hr = merged[head]
    line = dict(first)
    line.update({
        "value": hr["tflops"],
        "ms_per_step": hr["ms_per_step"],
        "frac_of_peak": hr["frac_of_peak"],
        "roofline": {k: hr["roofline"][k] for k in
                     ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "clock": hr.get("clock"),
        "parity_ok": all(ln["parity_ok"] for ln in lines),
        "processes": P,
        "workloads": merged,
        "cpu_baseline": first.get("cpu_baseline"),
    })
    return line


def run_processes(P, argv):
    """Run the measurement in P child processes, one after another on the one
    GPU, and merge their lines."""
    import subprocess

    base = [sys.executable, os.path.abspath(__file__)] + strip_processes(argv) + ["--processes", "1"]
    lines = []
    for i in range(P):
        cmd = base + (["--no-cpu"] if i > 0 and "--no-cpu" not in base else [])
        print("bench: process %d of %d" % (i + 1, P), file=sys.stderr, flush=True)
        out = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        if out.returncode != 0:
            sys.stderr.write(out.stdout[-2000:])
            sys.exit(out.returncode)
        js = [ln for ln in out.stdout.splitlines() if ln.startswith("{")]
        lines.append(json.loads(js[-1]))
    return merge_processes(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", action="append", default=None,
                    help="workload names (default: DEFAULT_WORKLOADS: the five configurations "
                         "f16_4096, f8_8192, f16_256_pm1, f16_1920x13900x4096, "
                         "qkt_64x4096x4096x128, then attn_64x4096x4096x128, f16_2048, the "
                         "NN/TT/NT layouts of f16_4096 and f8_8192, 512 x 512 x 32768 without "
                         "and with split-K, and the ping-pong kernel on f16_4096 and f8_8192)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the sampled oracle checks before timing (profiling runs)")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="back-to-back launches for this long before the warm-up steps")
    ap.add_argument("--processes", type=int, default=3,
                    help="independent processes, run one after another; the line reports "
                         "each workload from the process with the median time, plus every "
                         "process's per-launch median and their median and range")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (a known-size kernel for "
                         "scaling HBM byte counters), then exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch

        n = args.calibrate_copy * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                          "copies": 5}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this GEMM build runs on a single MI355X; "
              "--gpus %d is not supported (a multi-GPU run would shard N across GPUs with no "
              "exchange, see the design notes)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.processes > 1:
        # The parent only starts the children and merges their lines: it never
        # touches the GPU itself.
        print(json.dumps(run_processes(args.processes, sys.argv[1:])), flush=True)
        return

    import torch

    from dense_gemm_tn_amd import inputs

    dev = torch.device("cuda:0")
    names = args.workload or list(DEFAULT_WORKLOADS)
    head = "f16_4096" if "f16_4096" in names else names[0]
    results = {}
    keep = {}
    for name in names:
        w = inputs.WORKLOADS[name]
        # A workload may force a tile configuration (the library reads
        # DG_GEMM_TILE on every call); it is set only while that workload runs.
        saved = os.environ.pop("DG_GEMM_TILE", None)
        if "tile" in w.extra:
            os.environ["DG_GEMM_TILE"] = w.extra["tile"]
        elif saved is not None:
            os.environ["DG_GEMM_TILE"] = saved
        print("bench: %s" % name, file=sys.stderr, flush=True)
        res, x, sets = time_workload(w, args.steps, args.warmup, dev, check=not args.no_check,
                                     settle_s=args.settle_ms / 1e3)
        kname = kernel_name(w)
        os.environ.pop("DG_GEMM_TILE", None)
        if saved is not None:
            os.environ["DG_GEMM_TILE"] = saved
        kernel_s = res["ms_per_step"] / 1e3
        tb = traffic_for(name, w, kernel_s)
        if w.kind == "qkt":
            res["hbm_frac_of_peak"] = res["hbm_gbs_algorithmic"] / HBM_PEAK_GBS
        res["roofline"] = {
            "bound": "hbm" if w.kind == "qkt" else "mfma",
            "achieved": res["hbm_gbs_algorithmic"] if w.kind == "qkt" else res["tflops"],
            "peak": HBM_PEAK_GBS if w.kind == "qkt" else PEAK_TFLOPS[w.kind],
            "unit": "GB/s" if w.kind == "qkt" else "TFLOP/s",
            "traffic": tb,
            "kernel": kname,
        }
        r = res["roofline"]
        r["frac"] = r["achieved"] / r["peak"]
        results[name] = res
        if name == head:
            keep = {"w": w, "x": x, "sets": sets}
        else:
            del sets, x
        torch.cuda.empty_cache()

    hw = inputs.WORKLOADS[head]
    hr = results[head]
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(keep["w"], keep["x"], keep["sets"])
    line = {
        "metric": METRIC,
        "value": hr["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hr["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if hw.kind != "f8" else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": head, "M": hw.M, "N": hw.N, "K": hw.K, "batch": hw.batch,
                   "layout": "TN (A row-major, B K-contiguous, C column-major ld=M)",
                   "accumulate": "fp32", "inputs": hw.dist, "seed": hw.seed},
        "frac_of_peak": hr["frac_of_peak"],
        "roofline": {k: hr["roofline"][k] for k in
                     ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "cpu_baseline": cpu,
        "clock": hr.get("clock"),
        "parity_ok": all((r["parity"]["before"] or {}).get("ok", True)
                         and r["parity"]["after_bitwise_equal"] for r in results.values()),
        "workloads": results,
        "kernel_source_sha256_16": {k: source_hash(k) for k in ("f16", "attn")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
