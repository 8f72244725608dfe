"""GPU parity of the planned TN launches (grids with a ragged last round).

A plan runs the first dp_cols columns of C in whole rounds of the 256-row
kernel and the remaining columns as a second launch (see gemm_tn_plan):
  * without a workspace every element is computed as by the single launch of
    the selector's configuration (same products, same K order), so C equals
    that launch's C bit for bit, and +-1 inputs give the oracle's C exactly;
  * with a workspace the tail's K range may be cut into ranges summed through
    it: +-1 inputs still exact (integer partial sums below 2^24), N(0,1)
    inputs differ from the single launch by fp32 summation order only;
  * canaries around C, in its ldc padding and past the workspace's used bytes
    stay intact.
Shapes are ones the plan splits on a 256-CU device: 4096 x 4352 (16 tile
rows, 17 or 20 tile columns), a ragged M = 4000 with an odd ldc, and QK^T
heads with a 256-deep contraction.
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs
from test_gpu_parity import BF16_TOL, CANARY16, DEV, F16_TOL, assert_exact, out_fmt, reference

pytestmark = pytest.mark.gpu

WS_CANARY = -12345.0
TILE = {0: "256", 1: "224", 2: "128"}


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def launch(kind, x, M, N, K, ldc=None, ws_bytes=None, guard=64, ws_guard=256):
    """C as [N, M] 16-bit codes and the canary verdicts.  ws_bytes None: the
    plain call; else the *_ws call with that many workspace bytes."""
    ldc = M if ldc is None else ldc
    a = torch.from_numpy(x["A"].view(np.int16) if kind == "f16" else x["A"]).to(DEV)
    b = torch.from_numpy(x["B"].view(np.int16) if kind == "f16" else x["B"]).to(DEV)
    c = torch.full((guard * 2 + N * ldc,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    cp = c.data_ptr() + guard * 2
    ws = None
    if ws_bytes is not None:
        ws = torch.full((ws_bytes // 4 + ws_guard,), WS_CANARY, dtype=torch.float32, device=DEV)
    if kind == "f16":
        if ws is None:
            dg.gemm_f16_tn(a, b, cp, M, N, K, K, K, ldc)
        else:
            dg.gemm_f16_tn_ws(a, b, cp, M, N, K, K, K, ldc, ws, ws_bytes)
    else:
        if ws is None:
            dg.gemm_f8_tn(a, b, cp, M, N, K, K, K, ldc, x["scale_a"], x["scale_b"])
        else:
            dg.gemm_f8_tn_ws(a, b, cp, M, N, K, K, K, ldc, x["scale_a"], x["scale_b"], ws,
                             ws_bytes)
    torch.cuda.synchronize()
    host = c.cpu().numpy().view(np.uint16)
    body = host[guard:guard + N * ldc].reshape(N, ldc)
    canary = (np.all(host[:guard] == CANARY16) and np.all(host[guard + N * ldc:] == CANARY16)
              and np.all(body[:, M:] == CANARY16))
    ws_ok = True
    if ws is not None:
        ws_ok = bool(np.all(ws.cpu().numpy()[ws_bytes // 4:] == WS_CANARY))
    return np.ascontiguousarray(body[:, :M]), canary, ws_ok


def single_launch(monkeypatch, kind, x, M, N, K, ldc=None):
    """The selector's single launch (DG_GEMM_TILE turns plans off)."""
    cfg = dg.tn_config(M, N, K, fp8=(kind == "f8"))
    with monkeypatch.context() as m:
        m.setenv("DG_GEMM_TILE", TILE[cfg])
        got, canary, _ = launch(kind, x, M, N, K, ldc=ldc)
    assert canary
    return got


@pytest.mark.parametrize("kind,M,N,K,ldc", [("f16", 4096, 4352, 4096, None),
                                            ("f16", 4000, 4608, 4096, 4003),
                                            ("f8", 4096, 4608, 4096, None),
                                            ("f8", 4000, 4352, 4096, 4001)])
def test_plan_equals_single_launch_bitwise(monkeypatch, kind, M, N, K, ldc):
    plan = dg.tn_plan(M, N, K, fp8=(kind == "f8"))
    print("plan %s %dx%dx%d ldc %s: %s" % (kind, M, N, K, ldc, plan), flush=True)
    if _cus() == 256:
        assert plan["dp_cols"] > 0 and plan["splits"] == 1
    x = inputs.make_shape(kind, M, N, K, dist="normal", seed=M + N)
    got, canary, _ = launch(kind, x, M, N, K, ldc=ldc)
    assert canary
    one = single_launch(monkeypatch, kind, x, M, N, K, ldc=ldc)
    assert np.array_equal(got, one), "%d elements differ" % int((got != one).sum())


@pytest.mark.parametrize("kind,M,N,K", [("f16", 4000, 4352, 4096), ("f8", 4096, 4352, 4096)])
def test_plan_pm1_exact(kind, M, N, K):
    print("plan pm1 %s %dx%dx%d: %s" % (kind, M, N, K, dg.tn_plan(M, N, K, fp8=(kind == "f8"))),
          flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=7)
    got, canary, _ = launch(kind, x, M, N, K, ldc=M + 8)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


def test_ws_plan_split_tail_pm1_exact():
    """The workspace plan of 4096 x 4352 x 4096 fp16: 16 whole columns of
    256 x 256 tiles, the last 256 columns split-K through the workspace."""
    M, N, K = 4096, 4352, 4096
    nbytes = dg.tn_workspace_bytes(M, N, K)
    plan = dg.tn_plan(M, N, K, workspace_bytes=nbytes)
    print("ws plan f16 %dx%dx%d: %s" % (M, N, K, plan), flush=True)
    if _cus() == 256:
        assert plan["dp_cols"] > 0 and plan["splits"] > 1 and nbytes == plan["workspace_bytes"] > 0
    x = inputs.make_shape("f16", M, N, K, dist="pm1", seed=9)
    got, canary, ws_ok = launch("f16", x, M, N, K, ldc=M + 4, ws_bytes=nbytes)
    assert canary and ws_ok
    assert_exact("f16", got, reference("f16", x, M, N, K))


@pytest.mark.parametrize("kind,M,N,K", [("f16", 4608, 4096, 4096), ("f16", 2048, 9216, 8192)])
def test_ws_plan_normal_close_to_single_launch(monkeypatch, kind, M, N, K):
    nbytes = dg.tn_workspace_bytes(M, N, K)
    plan = dg.tn_plan(M, N, K, workspace_bytes=nbytes)
    print("ws plan normal %s %dx%dx%d: %s" % (kind, M, N, K, plan), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="normal", seed=5)
    got, canary, ws_ok = launch(kind, x, M, N, K, ws_bytes=nbytes)
    assert canary and ws_ok
    one = single_launch(monkeypatch, kind, x, M, N, K)
    g = oracle.decode(got, out_fmt(kind))
    u = oracle.decode(one, out_fmt(kind))
    assert np.all(np.isfinite(g))
    bar = F16_TOL if kind == "f16" else BF16_TOL
    # Summation order only: a couple of output ulps of the largest element.
    assert np.max(np.abs(g - u)) / np.max(np.abs(u)) <= bar / 4
    if plan["splits"] == 1:
        assert np.array_equal(got, one)


def test_ws_call_without_workspace_is_the_plain_call():
    M, N, K = 4096, 4352, 1024
    x = inputs.make_shape("f16", M, N, K, dist="normal", seed=2)
    a = torch.from_numpy(x["A"]).to(DEV)
    b = torch.from_numpy(x["B"]).to(DEV)
    c0 = torch.empty((N, M), dtype=torch.float16, device=DEV)
    c1 = torch.empty((N, M), dtype=torch.float16, device=DEV)
    dg.gemm_f16_tn(a, b, c0, M, N, K, K, K, M)
    dg.gemm_f16_tn_ws(a, b, c1, M, N, K, K, K, M, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(c0.view(torch.int16), c1.view(torch.int16))


def test_matmul_helper_auto_runs_the_workspace_plan():
    M, N, K = 4096, 4352, 4096
    x = inputs.make_shape("f16", M, N, K, dist="pm1", seed=9)
    a = torch.from_numpy(x["A"]).to(DEV)
    b = torch.from_numpy(x["B"]).to(DEV)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    c = dg.matmul_tn_f16(a, b, stream=side, splits="auto")
    side.synchronize()
    assert_exact("f16", c.cpu().numpy().view(np.uint16), reference("f16", x, M, N, K))


def test_batched_heads_plan(monkeypatch):
    """Two QK^T heads of 4096 x 4352 with a 256-deep contraction: the plan
    splits the columns of every head; bitwise equal to the single launch,
    +-1 exact against the oracle head by head, head gaps untouched."""
    H, M, N, D = 2, 4096, 4352, 256
    plan = dg.tn_plan(M, N, D, batch=H)
    print("batched plan %d x %dx%dx%d: %s" % (H, M, N, D, plan), flush=True)
    if _cus() == 256:
        assert plan["dp_cols"] > 0
    x = inputs.make_shape("qkt", M, N, D, dist="pm1", seed=4, batch=H)
    q = torch.from_numpy(x["Q"]).to(DEV)
    k = torch.from_numpy(x["K"]).to(DEV)
    ld, stride = M + 8, N * (M + 8) + 64

    def run():
        s = torch.full((H * stride,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
        dg.gemm_batched_qkt(q, k, s, H, M, N, D, D, D, ld, M * D, N * D, stride)
        torch.cuda.synchronize()
        return s.cpu().numpy().view(np.uint16)

    got = run()
    with monkeypatch.context() as m:
        m.setenv("DG_GEMM_TILE", TILE[dg.tn_config(M, N, D, batch=H)])
        one = run()
    assert np.array_equal(got, one)
    for h in range(H):
        blk = got[h * stride:(h + 1) * stride]
        body = blk[:N * ld].reshape(N, ld)
        assert np.all(body[:, M:] == CANARY16) and np.all(blk[N * ld:] == CANARY16)
        ref = oracle.gemm_tn(x["Q"][h], x["K"][h], oracle.FMT_F16, M, N, D)
        assert_exact("qkt", np.ascontiguousarray(body[:, :M]), ref)
