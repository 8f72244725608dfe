"""GPU parity of the split-K TN GEMM (gemm_f16_tn_splitk, gemm_f8_tn_splitk).

K is cut into ranges of whole K-steps, each multiplied into an fp32 partial
in the caller's workspace, then summed in range order and rounded once, so:
  * +-1 inputs: every partial and every sum is an integer below 2^24, exact in
    fp32, so C equals the oracle bit for bit (fp16 / bf16 of the exact sum);
  * N(0,1) inputs: within the bar of the unsplit call (fp16 4e-3, bf16 1e-2
    of max|C_ref|), the difference being fp32 summation order only;
  * splits = 1, or a K too short to split, is the unsplit call bit for bit
    and leaves the workspace untouched;
  * nothing outside C's logical extent and the workspace's needed bytes is
    written (canaries).
Shapes: uneven last ranges, K tails inside a K-step, more splits than K-steps
allow, ragged M / N below one tile, odd ldc, K = 0.
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs
from test_gpu_parity import BF16_TOL, CANARY16, DEV, F16_TOL

pytestmark = pytest.mark.gpu

WS_CANARY = -12345.0


def run(kind, x, M, N, K, splits, ldc=None, guard=64, ws_guard=256):
    """C as [N, M] 16-bit codes, C canaries intact, workspace guard intact."""
    ldc = M if ldc is None else ldc
    a = torch.from_numpy(x["A"].view(np.int16) if kind == "f16" else x["A"]).to(DEV)
    b = torch.from_numpy(x["B"].view(np.int16) if kind == "f16" else x["B"]).to(DEV)
    total = guard * 2 + max(N * ldc, 1)
    c = torch.full((total,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    need = dg.splitk_workspace_bytes(M, N, splits)
    assert need >= 0
    ws = torch.full((need // 4 + ws_guard,), WS_CANARY, dtype=torch.float32, device=DEV)
    cp = c.data_ptr() + guard * 2
    if kind == "f16":
        dg.gemm_f16_tn_splitk(a, b, cp, M, N, K, K, K, ldc, splits, ws, need)
    else:
        dg.gemm_f8_tn_splitk(a, b, cp, M, N, K, K, K, ldc, x["scale_a"], x["scale_b"], splits,
                             ws, need)
    torch.cuda.synchronize()
    host = c.cpu().numpy().view(np.uint16)
    body = host[guard:guard + N * ldc].reshape(N, ldc)
    canary = (np.all(host[:guard] == CANARY16) and np.all(host[guard + N * ldc:] == CANARY16)
              and np.all(body[:, M:] == CANARY16))
    ws_host = ws.cpu().numpy()
    ws_ok = bool(np.all(ws_host[need // 4:] == WS_CANARY))
    return np.ascontiguousarray(body[:, :M]), canary, ws_ok, ws_host[:need // 4]


def fmt_out(kind):
    return oracle.FMT_F16 if kind == "f16" else oracle.FMT_BF16


def fmt_in(kind):
    return oracle.FMT_F16 if kind == "f16" else oracle.FMT_E4M3FN


# (M, N, K, splits): even and uneven ranges, K tails, the 64-split maximum,
# more splits than 16-step ranges allow, tiny M / N, M not a multiple of 4
# (partial rows stored one by one, padded workspace columns).
CASES = {
    "f16": [(256, 256, 8192, 8), (200, 136, 4000, 7), (128, 128, 64 * 33, 4), (1, 8, 2048, 16),
            (512, 384, 16384, 64), (300, 260, 1024, 64), (136, 72, 65536, 32),
            (133, 45, 3000, 6)],
    "f8": [(256, 256, 16384, 8), (208, 144, 8000, 7), (16, 32, 4096, 16), (272, 160, 2048, 64),
           (131, 77, 4096, 8)],
}


@pytest.mark.parametrize("kind,M,N,K,splits",
                         [(k,) + c for k in ("f16", "f8") for c in CASES[k]])
def test_splitk_pm1_exact(kind, M, N, K, splits):
    print("splitk %s %dx%dx%d splits %d" % (kind, M, N, K, splits), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=M + 5 * N + K + splits)
    got, canary, ws_ok, _ = run(kind, x, M, N, K, splits)
    assert canary and ws_ok
    ref = oracle.gemm_tn(x["A"], x["B"], fmt_in(kind), M, N, K)
    want = oracle.decode(oracle.encode(ref, fmt_out(kind)), fmt_out(kind))
    g = oracle.decode(got, fmt_out(kind))
    assert np.array_equal(g, want), "%d mismatches" % int((g != want).sum())


@pytest.mark.parametrize("kind,M,N,K,splits", [("f16", 384, 200, 12288, 12),
                                               ("f8", 256, 320, 16384, 9)])
def test_splitk_normal_within_bar_and_close_to_unsplit(kind, M, N, K, splits):
    print("splitk normal %s %dx%dx%d" % (kind, M, N, K), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="normal", seed=3)
    got, canary, ws_ok, _ = run(kind, x, M, N, K, splits, ldc=M + 3)
    assert canary and ws_ok
    scale = 1.0 if kind == "f16" else float(x["scale_a"]) * float(x["scale_b"])
    ref = oracle.gemm_tn(x["A"], x["B"], fmt_in(kind), M, N, K, scale=scale)
    g = oracle.decode(got, fmt_out(kind))
    bar = F16_TOL if kind == "f16" else BF16_TOL
    assert np.all(np.isfinite(g))
    assert np.max(np.abs(g - ref)) / np.max(np.abs(ref)) <= bar
    one, _, _, _ = run(kind, x, M, N, K, 1, ldc=M + 3)
    u = oracle.decode(one, fmt_out(kind))
    # Summation order only: at most a couple of output ulps apart.
    assert np.max(np.abs(g - u)) / np.max(np.abs(ref)) <= bar / 4


@pytest.mark.parametrize("M,N,K,splits", [(256, 256, 4096, 1), (264, 200, 64, 8)])
def test_unsplit_cases_equal_plain_call_and_skip_workspace(M, N, K, splits):
    """splits = 1, or a K of a single K-step whatever the count asked for, is
    gemm_f16_tn itself and never touches the workspace."""
    x = inputs.make_shape("f16", M, N, K, dist="normal", seed=11)
    a = torch.from_numpy(x["A"]).to(DEV)
    b = torch.from_numpy(x["B"]).to(DEV)
    c0 = torch.empty((N, M), dtype=torch.float16, device=DEV)
    dg.gemm_f16_tn(a, b, c0, M, N, K, K, K, M)
    torch.cuda.synchronize()
    got, canary, ws_ok, ws = run("f16", x, M, N, K, splits)
    assert canary and ws_ok
    assert np.all(ws == WS_CANARY)
    assert np.array_equal(got, c0.cpu().numpy().view(np.uint16))


def test_k_zero_writes_zeros():
    M, N = 136, 72
    x = {"A": np.zeros((M, 8), np.float16), "B": np.zeros((N, 8), np.float16)}
    got, canary, ws_ok, _ = run("f16", x, M, N, 0, 8)
    assert canary and ws_ok
    assert np.all(oracle.decode(got, oracle.FMT_F16) == 0)


def test_choose_gives_every_cu_a_block():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = dg.splitk_choose(512, 512, 32768)
    assert 1 < s <= 64 and 16 * s >= cus
    assert dg.splitk_choose(4096, 4096, 4096) == 1
    assert dg.splitk_choose(512, 512, 1024) == 1


@pytest.mark.parametrize("splits", ["auto", 5])
def test_matmul_helper_splitk(splits):
    """The tensor helper allocates the workspace itself (auto: the chooser's count)."""
    M, N, K = 256, 192, 16384
    x = inputs.make_shape("f16", M, N, K, dist="pm1", seed=17)
    a = torch.from_numpy(x["A"]).to(DEV)
    b = torch.from_numpy(x["B"]).to(DEV)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    c = dg.matmul_tn_f16(a, b, stream=side, splits=splits)
    side.synchronize()
    ref = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, M, N, K)
    want = oracle.decode(oracle.encode(ref, oracle.FMT_F16), oracle.FMT_F16)
    assert np.array_equal(oracle.decode(c.cpu().numpy(), oracle.FMT_F16), want)


@pytest.mark.parametrize("kind,M,N,K", [("f16", 1024, 1024, 16384), ("f8", 1024, 1024, 32768)])
def test_splitk_chooser_doubled_configuration(kind, M, N, K):
    """The chooser's two-blocks-per-CU branch (1024^2 x 16384 fp16: 64 tiles,
    8 ranges of 32 K-steps on 256 CUs), run with the count it suggests: +-1
    data exact against the oracle, canaries around C and past the workspace."""
    splits = dg.splitk_choose(M, N, K, fp8=(kind == "f8"))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = (M // 128) * (N // 128)
    assert splits == 2 * (cus // tiles)   # the doubled branch on this device
    print("splitk chooser %s %dx%dx%d splits %d" % (kind, M, N, K, splits), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=23)
    got, canary, ws_ok, _ = run(kind, x, M, N, K, splits)
    assert canary and ws_ok
    ref = oracle.gemm_tn(x["A"], x["B"], fmt_in(kind), M, N, K)
    want = oracle.decode(oracle.encode(ref, fmt_out(kind)), fmt_out(kind))
    g = oracle.decode(got, fmt_out(kind))
    assert np.array_equal(g, want), "%d mismatches" % int((g != want).sum())


@pytest.mark.parametrize("kind,M,N,K", [("f16", 1536, 1536, 4096), ("f16", 1530, 1500, 4096 - 24),
                                        ("f16", 2048, 1024, 4096), ("f8", 1536, 1536, 8192)])
def test_splitk_chooser_medium_grid(kind, M, N, K):
    """The chooser's medium-grid branch (more than half of the CUs' worth of
    128 x 128 tiles, fewer than all): the count it suggests, two blocks per CU
    in one round (or one per CU at exactly half), +-1 data exact against the
    oracle, canaries around C and past the workspace."""
    splits = dg.splitk_choose(M, N, K, fp8=(kind == "f8"))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-M // 128) * -(-N // 128)
    print("splitk medium grid %s %dx%dx%d tiles %d splits %d" % (kind, M, N, K, tiles, splits),
          flush=True)
    if cus == 256:
        assert splits == (2 if 2 * tiles == cus else 3)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=29)
    got, canary, ws_ok, _ = run(kind, x, M, N, K, splits)
    assert canary and ws_ok
    ref = oracle.gemm_tn(x["A"], x["B"], fmt_in(kind), M, N, K)
    want = oracle.decode(oracle.encode(ref, fmt_out(kind)), fmt_out(kind))
    g = oracle.decode(got, fmt_out(kind))
    assert np.array_equal(g, want), "%d mismatches" % int((g != want).sum())


# Split ranges of 8 to 11 K-steps on a grid of one block per CU (the partial
# kernel's four-stage ring), the last range short, and 7 (two-stage ring).
# 57 K-steps in 8 splits: seven ranges of 8 and a last range of one step, whose
# block issues copies three steps past its range before its only step (whole
# K-steps: the fixed-offset form; with a K tail: the general form).
@pytest.mark.parametrize("kind,M,N,K,splits", [("f16", 300, 200, 64 * 8 * 6 - 40, 6),
                                               ("f16", 256, 256, 64 * 9 * 5, 5),
                                               ("f16", 130, 250, 64 * 10 * 4 + 64 * 3, 5),
                                               ("f16", 256, 128, 64 * 7 * 8, 8),
                                               ("f8", 256, 200, 128 * 11 * 3 - 16, 3),
                                               ("f16", 256, 256, 64 * 57, 8),
                                               ("f16", 250, 256, 64 * 57 - 24, 8),
                                               ("f8", 256, 200, 128 * 57, 8)])
def test_splitk_ring_ranges_exact(kind, M, N, K, splits):
    print("splitk ring %s %dx%dx%d splits %d" % (kind, M, N, K, splits), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=M + N + K)
    got, canary, ws_ok, _ = run(kind, x, M, N, K, splits)
    assert canary and ws_ok
    ref = oracle.gemm_tn(x["A"], x["B"], fmt_in(kind), M, N, K)
    want = oracle.decode(oracle.encode(ref, fmt_out(kind)), fmt_out(kind))
    g = oracle.decode(got, fmt_out(kind))
    assert np.array_equal(g, want), "%d mismatches" % int((g != want).sum())
