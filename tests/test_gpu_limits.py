"""GPU parity at the sizes where the library's address arithmetic is stretched.

Every block reads its operands through buffer descriptors with 32-bit byte
offsets, so a TN call is accepted only while 256 rows of an operand span less
than 2^31 bytes (the library rejects one vector more: CPU-tested in
test_abi.py).  Block, head and column bases are 64-bit.  Here, on the GPU:

  * the largest accepted row strides (about 8 MiB per row), ragged M and N, the
    library's choice and every tile configuration forced, with NaN in the
    padding between rows (never read into a stored element): +-1 data
    bit-exact against the oracle;
  * a product whose A spans more than 2 GiB (about 2^20 rows), so block bases
    pass 2^31 bytes: +-1 invariants on all of C, the oracle on sampled rows;
  * a batched QK^T whose output spans more than 4 GiB (head offsets past 32
    bits): the first, a middle and the last head against the oracle, the
    memory past the last head untouched.
Inputs are seeded +-1 (every partial sum an exact integer), so the bar is bit
equality ("hello-gpu, chapter 11 (GEMM-like)", section 11.4: edge shapes and
sizes; "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", step 4: buffer
descriptors for bounded loads).
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs
from test_gpu_parity import CANARY16, DEV, assert_exact, in_fmt, out_fmt, reference

pytestmark = pytest.mark.gpu

NAN16 = 0x7E00          # fp16 quiet NaN
NAN8 = 0x7F             # E4M3FN NaN


def max_ld(es):
    """The largest row stride (elements) the TN calls accept: 256 rows of it,
    plus one 128-byte K row, below 2^31 bytes, rounded down to the 16-byte
    vector (one vector more is rejected: test_abi.py)."""
    vec = 16 // es
    return ((2 ** 31 - 128 - 1) // (256 * es)) // vec * vec


def strided_operand(logical, ld, nan_code):
    """A device buffer of rows at stride ld (elements) holding `logical` (rows x K
    codes), NaN everywhere else."""
    rows, K = logical.shape
    n = (rows - 1) * ld + K
    dt = torch.int16 if logical.dtype == np.float16 else torch.uint8
    buf = torch.full((n,), nan_code, dtype=dt, device=DEV)   # both codes fit the type
    src = torch.from_numpy(np.ascontiguousarray(logical).view(np.int16 if dt == torch.int16 else np.uint8))
    buf.as_strided((rows, K), (ld, 1)).copy_(src.to(DEV))
    return buf


def run(kind, a, b, x, M, N, K, lda, ldb, guard=64):
    ldc = M
    c = torch.full((guard * 2 + N * ldc,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    cp = c.data_ptr() + guard * 2
    if kind == "f16":
        rc = dg.lib().gemm_f16_tn(a.data_ptr(), b.data_ptr(), cp, M, N, K, lda, ldb, ldc, None)
    else:
        rc = dg.lib().gemm_f8_tn(a.data_ptr(), b.data_ptr(), cp, M, N, K, lda, ldb, ldc,
                                 float(x["scale_a"]), float(x["scale_b"]), None)
    torch.cuda.synchronize()
    assert rc == 0, dg.status_string(rc)
    host = c.cpu().numpy().view(np.uint16)
    body = host[guard:guard + N * ldc].reshape(N, ldc)
    ok = np.all(host[:guard] == CANARY16) and np.all(host[guard + N * ldc:] == CANARY16)
    return np.ascontiguousarray(body[:, :M]), ok


@pytest.mark.parametrize("tile", [None, "256", "224", "128"])
@pytest.mark.parametrize("kind,M,N,K", [("f16", 300, 280, 520), ("f8", 290, 300, 528)])
def test_largest_row_strides_exact(monkeypatch, tile, kind, M, N, K):
    es = 2 if kind == "f16" else 1
    ld = max_ld(es)
    print("limit strides %s %dx%dx%d ld %d tile %s" % (kind, M, N, K, ld, tile), flush=True)
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    if tile:
        monkeypatch.setenv("DG_GEMM_TILE", tile)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=M + N + K + es)
    nan = NAN16 if kind == "f16" else NAN8
    a = strided_operand(x["A"], ld, nan)
    b = strided_operand(x["B"], ld, nan)
    got, canary = run(kind, a, b, x, M, N, K, ld, ld)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))
    del a, b
    torch.cuda.empty_cache()


def test_operand_past_2gib_block_bases():
    """A with 2^20 + 7 rows of 1024 fp16 (2 GiB + 14 KiB): the last blocks'
    bases lie past 2^31 bytes."""
    M, N, K = (1 << 20) + 7, 136, 1024
    print("A past 2 GiB: %dx%dx%d config %d" % (M, N, K, dg.tn_config(M, N, K)), flush=True)
    x = inputs.make_shape("f16", M, N, K, dist="pm1", seed=11)
    a = torch.from_numpy(x["A"].view(np.int16)).to(DEV)
    b = torch.from_numpy(x["B"].view(np.int16)).to(DEV)
    got, canary = run("f16", a, b, x, M, N, K, K, K)
    assert canary
    del a, b
    torch.cuda.empty_cache()
    C = oracle.decode(got, out_fmt("f16"))
    # +-1 invariants on every element: integer, |C| <= K, C = K (mod 2).
    assert np.all(np.abs(C) <= K) and np.all(np.mod(C, 2) == K % 2)
    # Oracle on the first, a middle and the last 512 rows (all N columns).
    for r0 in (0, (M // 2) // 256 * 256 + 3, M - 512):
        rows = slice(r0, r0 + 512)
        ref = oracle.gemm_tn(np.ascontiguousarray(x["A"][rows]), x["B"], in_fmt("f16"), 512, N, K)
        assert_exact("f16", np.ascontiguousarray(got[:, rows]), ref)


def test_batched_qkt_output_past_4gib():
    """130 heads of 4096 x 4096 (D = 64): S spans 4.06 GiB, head bases pass 2^32
    bytes."""
    H, M, N, D = 130, 4096, 4096, 64
    x = inputs.make_shape("qkt", M, N, D, dist="pm1", seed=13, batch=H)
    q = torch.from_numpy(x["Q"]).to(DEV)
    k = torch.from_numpy(x["K"]).to(DEV)
    stride = N * M
    tail = 4096
    s = torch.empty((H * stride + tail,), dtype=torch.int16, device=DEV)
    s[H * stride:].fill_(int(np.int16(np.uint16(CANARY16).view(np.int16))))
    print("qkt past 4 GiB: %d heads, %.2f GiB" % (H, H * stride * 2 / 2 ** 30), flush=True)
    dg.gemm_batched_qkt(q, k, s, H, M, N, D, D, D, M, M * D, N * D, stride)
    torch.cuda.synchronize()
    assert np.all(s[H * stride:].cpu().numpy().view(np.uint16) == CANARY16)
    for h in (0, 65, H - 1):
        got = s[h * stride:(h + 1) * stride].cpu().numpy().view(np.uint16).reshape(N, M)
        ref = oracle.gemm_tn(x["Q"][h], x["K"][h], oracle.FMT_F16, M, N, D)
        assert_exact("qkt", got, ref)
