"""Stream ordering and graph capture of the C-ABI calls.

Every entry point enqueues its kernel on the stream it is given and touches
no other stream, allocates nothing and issues no memset, so its launches can be
ordered on a side stream and captured into a HIP graph.  The tests below check
both with +-1 inputs, whose products are small integers and must match the
oracle exactly: a GEMM on a side stream that also produces its inputs, and a
captured graph of eight different calls (fp16 TN, fp8 TN, fp16 NN, batched
QK^T, fused attention, split-K fp16 TN with its workspace, and two planned
calls of several launches each: QK^T heads whose columns run in two parts,
and a workspace plan with a split-K tail) replayed several times.  Between replays, eager copies
on the current stream put new inputs in place, and every replay is checked
against the oracle (the attention output within its tolerance of
test_gpu_attention).
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs
from test_gpu_attention import tol
from test_gpu_parity import DEV

pytestmark = pytest.mark.gpu


def exact(got_codes, ref, fmt):
    want = oracle.decode(oracle.encode(ref, fmt), fmt)
    got = oracle.decode(got_codes, fmt)
    assert np.array_equal(got, want), "%d mismatches" % int((got != want).sum())


def test_side_stream_orders_producer_and_gemm():
    """Inputs written by kernels on a side stream, the GEMM queued behind them on
    that stream, the result read after synchronising only that stream."""
    M, N, K = 520, 392, 264
    x = inputs.make_shape("f16", M, N, K, dist="pm1", seed=41)
    a_host = torch.from_numpy(x["A"]).pin_memory()
    b_host = torch.from_numpy(x["B"]).pin_memory()
    side = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(side):
        a = torch.empty((M, K), dtype=torch.float16, device=DEV)
        b = torch.empty((N, K), dtype=torch.float16, device=DEV)
        c = torch.full((N, M), 7.0, dtype=torch.float16, device=DEV)
        a.copy_(a_host, non_blocking=True)
        b.copy_(b_host, non_blocking=True)
        a.mul_(-1.0).mul_(-1.0)           # more producer kernels on the same stream
        dg.gemm_f16_tn(a, b, c, M, N, K, K, K, M, stream=side)
    side.synchronize()
    print("side stream %dx%dx%d" % (M, N, K), flush=True)
    exact(c.cpu().numpy().view(np.uint16), oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, M, N, K),
          oracle.FMT_F16)


def test_graph_capture_replays_match_oracle():
    shapes = {"f16": (264, 136, 200), "f8": (272, 144, 256), "nn": (136, 264, 200),
              "qkt": (3, 200, 300, 128)}
    M1, N1, K1 = shapes["f16"]
    M2, N2, K2 = shapes["f8"]
    M3, N3, K3 = shapes["nn"]
    H, M4, N4, D4 = shapes["qkt"]
    # Static device buffers the graph reads and writes.
    a1 = torch.empty((M1, K1), dtype=torch.float16, device=DEV)
    b1 = torch.empty((N1, K1), dtype=torch.float16, device=DEV)
    c1 = torch.empty((N1, M1), dtype=torch.float16, device=DEV)
    a2 = torch.empty((M2, K2), dtype=torch.uint8, device=DEV)
    b2 = torch.empty((N2, K2), dtype=torch.uint8, device=DEV)
    c2 = torch.empty((N2, M2), dtype=torch.int16, device=DEV)
    a3 = torch.empty((K3, M3), dtype=torch.float16, device=DEV)    # 'N': A[m + k*lda]
    b3 = torch.empty((N3, K3), dtype=torch.float16, device=DEV)    # 'N': B[k + n*ldb]
    c3 = torch.empty((N3, M3), dtype=torch.float16, device=DEV)
    q4 = torch.empty((H, M4, D4), dtype=torch.float16, device=DEV)
    k4 = torch.empty((H, N4, D4), dtype=torch.float16, device=DEV)
    s4 = torch.empty((H, N4, M4), dtype=torch.float16, device=DEV)
    H5, M5, N5, D5 = 2, 200, 328, 128
    q5 = torch.empty((H5, M5, D5), dtype=torch.float16, device=DEV)
    k5 = torch.empty((H5, N5, D5), dtype=torch.float16, device=DEV)
    vt5 = torch.empty((H5, D5, N5), dtype=torch.float16, device=DEV)
    o5 = torch.empty((H5, M5, D5), dtype=torch.float16, device=DEV)
    scale5 = 1.0 / D5 ** 0.5
    M6, N6, K6, S6 = 136, 200, 4096, 4
    a6 = torch.empty((M6, K6), dtype=torch.float16, device=DEV)
    b6 = torch.empty((N6, K6), dtype=torch.float16, device=DEV)
    c6 = torch.empty((N6, M6), dtype=torch.float16, device=DEV)
    ws6_bytes = dg.splitk_workspace_bytes(M6, N6, S6)
    ws6 = torch.empty(ws6_bytes // 4, dtype=torch.float32, device=DEV)
    # Planned launches: two QK^T heads with a 256-deep contraction whose
    # columns run in two launches, and a workspace plan (whole rounds of
    # columns, then split-K of the rest and its reduction: three launches).
    H7, M7, N7, D7 = 2, 4096, 4352, 256
    q7 = torch.empty((H7, M7, D7), dtype=torch.float16, device=DEV)
    k7 = torch.empty((H7, N7, D7), dtype=torch.float16, device=DEV)
    s7 = torch.empty((H7, N7, M7), dtype=torch.float16, device=DEV)
    M8, N8, K8 = 4096, 4352, 4096
    a8 = torch.empty((M8, K8), dtype=torch.float16, device=DEV)
    b8 = torch.empty((N8, K8), dtype=torch.float16, device=DEV)
    c8 = torch.empty((N8, M8), dtype=torch.float16, device=DEV)
    ws8_bytes = dg.tn_workspace_bytes(M8, N8, K8)
    ws8 = torch.empty(max(ws8_bytes, 16) // 4, dtype=torch.float32, device=DEV)
    print("plans: qkt %s, ws %s" % (dg.tn_plan(M7, N7, D7, batch=H7),
                                    dg.tn_plan(M8, N8, K8, workspace_bytes=ws8_bytes)), flush=True)

    def calls():
        dg.gemm_f16_tn(a1, b1, c1, M1, N1, K1, K1, K1, M1)
        dg.gemm_f8_tn(a2, b2, c2, M2, N2, K2, K2, K2, M2, 1.0, 1.0)
        dg.gemm_f16("N", "N", a3, b3, c3, M3, N3, K3, M3, K3, M3)
        dg.gemm_batched_qkt(q4, k4, s4, H, M4, N4, D4, D4, D4, M4, M4 * D4, N4 * D4, N4 * M4)
        dg.attention_fwd_f16(q5, k5, vt5, o5, H5, M5, N5, D5, D5, D5, N5, D5, M5 * D5, N5 * D5,
                             D5 * N5, M5 * D5, scale5)
        dg.gemm_f16_tn_splitk(a6, b6, c6, M6, N6, K6, K6, K6, M6, S6, ws6, ws6_bytes)
        dg.gemm_batched_qkt(q7, k7, s7, H7, M7, N7, D7, D7, D7, M7, M7 * D7, N7 * D7, N7 * M7)
        dg.gemm_f16_tn_ws(a8, b8, c8, M8, N8, K8, K8, K8, M8, ws8, ws8_bytes)

    def load(seed):
        x1 = inputs.make_shape("f16", M1, N1, K1, dist="pm1", seed=seed)
        x2 = inputs.make_shape("f8", M2, N2, K2, dist="pm1", seed=seed + 1)
        x3 = inputs.make_shape("f16", M3, N3, K3, dist="pm1", seed=seed + 2)
        x4 = inputs.make_shape("qkt", M4, N4, D4, dist="pm1", seed=seed + 3, batch=H)
        x5 = inputs.make_shape("attn", M5, N5, D5, seed=seed + 4, batch=H5)
        x6 = inputs.make_shape("f16", M6, N6, K6, dist="pm1", seed=seed + 5)
        x7 = inputs.make_shape("qkt", M7, N7, D7, dist="pm1", seed=seed + 6, batch=H7)
        x8 = inputs.make_shape("f16", M8, N8, K8, dist="pm1", seed=seed + 7)
        a1.copy_(torch.from_numpy(x1["A"]))
        b1.copy_(torch.from_numpy(x1["B"]))
        a2.copy_(torch.from_numpy(x2["A"]))
        b2.copy_(torch.from_numpy(x2["B"]))
        a3.copy_(torch.from_numpy(np.ascontiguousarray(x3["A"].T)))
        b3.copy_(torch.from_numpy(x3["B"]))
        q4.copy_(torch.from_numpy(x4["Q"]))
        k4.copy_(torch.from_numpy(x4["K"]))
        q5.copy_(torch.from_numpy(x5["Q"]))
        k5.copy_(torch.from_numpy(x5["K"]))
        vt5.copy_(torch.from_numpy(x5["Vt"]))
        a6.copy_(torch.from_numpy(x6["A"]))
        b6.copy_(torch.from_numpy(x6["B"]))
        q7.copy_(torch.from_numpy(x7["Q"]))
        k7.copy_(torch.from_numpy(x7["K"]))
        a8.copy_(torch.from_numpy(x8["A"]))
        b8.copy_(torch.from_numpy(x8["B"]))
        for t in (c1, c2, c3, s4, o5, c6, ws6, s7, c8, ws8):
            t.fill_(0)
        torch.cuda.synchronize()
        return x1, x2, x3, x4, x5, x6, x7, x8

    def check(x1, x2, x3, x4, x5, x6, x7, x8):
        exact(c1.cpu().numpy().view(np.uint16),
              oracle.gemm_tn(x1["A"], x1["B"], oracle.FMT_F16, M1, N1, K1), oracle.FMT_F16)
        exact(c2.cpu().numpy().view(np.uint16),
              oracle.gemm_tn(x2["A"], x2["B"], oracle.FMT_E4M3FN, M2, N2, K2), oracle.FMT_BF16)
        exact(c3.cpu().numpy().view(np.uint16),
              oracle.gemm_tn(x3["A"], x3["B"], oracle.FMT_F16, M3, N3, K3), oracle.FMT_F16)
        exact(s4.cpu().numpy().view(np.uint16),
              oracle.batched_qkt(x4["Q"], x4["K"], H, M4, N4, D4), oracle.FMT_F16)
        o = o5.cpu().numpy().astype(np.float64)
        rows = np.arange(M5)
        for h in range(H5):
            want = oracle.attention_rows(x5["Q"][h], x5["K"][h], x5["Vt"][h], N5, D5, rows, scale5)
            assert np.all(np.abs(o[h] - want) <= tol(want, x5["Vt"][h])), h
        exact(c6.cpu().numpy().view(np.uint16),
              oracle.gemm_tn(x6["A"], x6["B"], oracle.FMT_F16, M6, N6, K6), oracle.FMT_F16)
        exact(s7.cpu().numpy().view(np.uint16),
              oracle.batched_qkt(x7["Q"], x7["K"], H7, M7, N7, D7), oracle.FMT_F16)
        exact(c8.cpu().numpy().view(np.uint16),
              oracle.gemm_tn(x8["A"], x8["B"], oracle.FMT_F16, M8, N8, K8), oracle.FMT_F16)

    # Eager run first (also settles the library's one-time device queries).
    xs = load(100)
    calls()
    torch.cuda.synchronize()
    check(*xs)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):      # captures on its own (default-priority) stream
        calls()
    torch.cuda.synchronize()
    for r in range(4):
        print("graph replay %d" % r, flush=True)
        xs = load(200 + 10 * r)
        g.replay()
        torch.cuda.synchronize()
        check(*xs)
