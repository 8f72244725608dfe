"""The no-allocation split-K entry point (gemm_f16_tn_splitk_noalloc) against
the workspace one (gemm_f16_tn_splitk), through the C ABI on the GPU.

The two run the same kernels with the same split count, so their outputs must
be equal bit for bit; +-1 data is also exact against the oracle (every
partial sum is an integer below 2^24) and N(0,1) data within the fp16 bar.
Two calls in a row, the second smaller than the first, so the second reads
nothing the first left in the shared device array; canaries around C."""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
CANARY16 = 0x7BCD
GUARD = 64


def _c_buffer(M, N, ldc):
    c = torch.full((GUARD * 2 + N * ldc,), CANARY16, dtype=torch.int32, device=DEV)
    return c.to(torch.int16)


def _body(c, M, N, ldc):
    host = c.cpu().numpy().view(np.uint16)
    body = host[GUARD:GUARD + N * ldc].reshape(N, ldc)
    ok = (np.all(host[:GUARD] == CANARY16) and np.all(host[GUARD + N * ldc:] == CANARY16)
          and np.all(body[:, M:] == CANARY16))
    return np.ascontiguousarray(body[:, :M]), ok


def _both(M, N, K, splits, dist, seed, ldc=None):
    ldc = M if ldc is None else ldc
    print("noalloc %dx%dx%d splits %d %s" % (M, N, K, splits, dist), flush=True)
    x = inputs.make_shape("f16", M, N, K, dist=dist, seed=seed)
    a = torch.from_numpy(x["A"]).to(DEV)
    b = torch.from_numpy(x["B"]).to(DEV)
    c_ws, c_na = _c_buffer(M, N, ldc), _c_buffer(M, N, ldc)
    need = dg.splitk_workspace_bytes(M, N, splits)
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    L = dg.lib()
    assert L.gemm_f16_tn_splitk(a.data_ptr(), b.data_ptr(), c_ws.data_ptr() + 2 * GUARD, M, N, K,
                                K, K, ldc, splits, ws.data_ptr(), need, stream) == dg.DG_OK
    assert L.gemm_f16_tn_splitk_noalloc(a.data_ptr(), b.data_ptr(), c_na.data_ptr() + 2 * GUARD,
                                        M, N, K, K, K, ldc, splits, stream) == dg.DG_OK
    torch.cuda.synchronize()
    got_ws, ok_ws = _body(c_ws, M, N, ldc)
    got_na, ok_na = _body(c_na, M, N, ldc)
    assert ok_ws and ok_na
    return x, got_ws, got_na


def test_noalloc_equals_workspace_call_then_smaller_call():
    # First: 16 ranges of 512 x 512 x 32768 (16 MiB of partials), N(0,1).
    x, got_ws, got_na = _both(512, 512, 32768, 16, "normal", 3)
    assert np.array_equal(got_na, got_ws)
    ref = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, 512, 512, 32768)
    got = oracle.decode(got_na, oracle.FMT_F16)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) <= 4e-3
    # Second, smaller (ragged M, N; uneven ranges; odd ldc): +-1, exact.
    M, N, K = 200, 136, 4000
    x, got_ws, got_na = _both(M, N, K, 7, "pm1", 4, ldc=M + 3)
    assert np.array_equal(got_na, got_ws)
    ref = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, M, N, K)
    want = oracle.decode(oracle.encode(ref, oracle.FMT_F16), oracle.FMT_F16)
    assert np.array_equal(oracle.decode(got_na, oracle.FMT_F16), want)


def test_noalloc_at_the_size_limit():
    # 8 ranges of 1024 x 1024 x 16384 need exactly the array's 32 MiB.
    assert dg.splitk_workspace_bytes(1024, 1024, 8) == 32 << 20
    x, got_ws, got_na = _both(1024, 1024, 16384, 8, "pm1", 5)
    assert np.array_equal(got_na, got_ws)
    ref = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, 1024, 1024, 16384)
    want = oracle.decode(oracle.encode(ref, oracle.FMT_F16), oracle.FMT_F16)
    assert np.array_equal(oracle.decode(got_na, oracle.FMT_F16), want)
