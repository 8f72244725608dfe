"""GPU parity of the FP8 GEMM in all four op-code layouts (gemm_f8) against the oracle.

The FP8 product of "AMD ROCm 4-wave interleave FP8 GEMM for Instinct MI355X
(CDNA 4)" (E4M3FN operands, per-tensor fp32 scales, fp32 accumulation, bf16
output) with the operands read as they lie, as for the fp16 layouts
("FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we compute"):
A 'T' = A[m*lda + k], 'N' = A[m + k*lda]; B 'N' = B[k + n*ldb], 'T' = B[k*ldb + n].
Expected values come from ``oracle.gemm`` on the same stored bytes.

Bars: +-1 inputs (codes 0x38 / 0xB8, scales 1) bit-exact in bf16 (every partial
sum is an integer of magnitude <= K); N(0,1) inputs quantised per tensor within
max|C - C_ref| / max|C_ref| <= 1e-2; canaries around C intact; operand padding
(the E4M3FN NaN code) never read into a stored element.  Every shape runs under
the library's choice and with each tile configuration forced (DG_GEMM_TILE).
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs
from test_gpu_parity import BF16_TOL, CANARY16, DEV

pytestmark = pytest.mark.gpu

LAYOUTS = [("T", "N"), ("N", "N"), ("T", "T"), ("N", "T")]
F8_NAN = np.uint8(0x7F)

# Multiples of 16 everywhere: one tile, ragged tiles, K tails inside a 128-deep
# step, many steps, skinny grids.
COMMON = [(16, 16, 16), (16, 32, 16), (128, 128, 128), (144, 272, 208), (256, 384, 1008),
          (528, 400, 144), (1008, 1008, 272), (64, 1200, 3984), (1200, 64, 400)]
# Extents only some layouts accept (see the fp16 layout tests).
EXTRA = {
    ("T", "N"): [(131, 133, 208)],
    ("N", "N"): [(144, 131, 208), (272, 1, 144)],
    ("T", "T"): [(131, 144, 208), (1, 272, 144)],
    ("N", "T"): [(144, 272, 203), (128, 128, 1), (256, 144, 129)],
}
CASES = [(ta, tb) + s for ta, tb in LAYOUTS for s in COMMON + EXTRA[(ta, tb)]]


def _pad(src, ld):
    rows, cols = src.shape
    out = np.full((rows, ld), F8_NAN, dtype=np.uint8)
    out[:, :cols] = src
    return np.ascontiguousarray(out)


def store(x, ta, tb, lda, ldb):
    As = _pad(x["A"] if ta == "T" else np.ascontiguousarray(x["A"].T), lda)
    Bs = _pad(x["B"] if tb == "N" else np.ascontiguousarray(x["B"].T), ldb)
    return As, Bs


def run_layout(ta, tb, As, Bs, M, N, K, lda, ldb, sa, sb, ldc=None, guard=64):
    """C (as [N, M] bf16 codes) from gemm_f8 with canaries around it."""
    ldc = M if ldc is None else ldc
    a = torch.from_numpy(As).to(DEV)
    b = torch.from_numpy(Bs).to(DEV)
    total = guard * 2 + max(N * ldc, 1)
    c = torch.full((total,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    dg.gemm_f8(ta, tb, a, b, c.data_ptr() + guard * 2, M, N, K, lda, ldb, ldc, sa, sb)
    torch.cuda.synchronize()
    host = c.cpu().numpy().view(np.uint16)
    body = host[guard:guard + N * ldc].reshape(N, ldc)
    canary = (np.all(host[:guard] == CANARY16) and np.all(host[guard + N * ldc:] == CANARY16)
              and np.all(body[:, M:] == CANARY16))
    return np.ascontiguousarray(body[:, :M]), canary


def lds(ta, tb, M, N, K, pad_a=0, pad_b=0):
    return (K if ta == "T" else M) + pad_a, (K if tb == "N" else N) + pad_b


def exact(got_codes, ref):
    got = oracle.decode(got_codes, oracle.FMT_BF16)
    want = oracle.decode(oracle.encode(ref, oracle.FMT_BF16), oracle.FMT_BF16)
    bad = got != want
    assert not bad.any(), "%d of %d differ; first [n,m]=%s got %r want %r" % (
        bad.sum(), bad.size, np.argwhere(bad)[0], got[bad][0], want[bad][0])


@pytest.fixture(params=[None, "256", "128"], ids=["auto", "tile256", "tile128"])
def tile(request, monkeypatch):
    if request.param is None:
        monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    else:
        monkeypatch.setenv("DG_GEMM_TILE", request.param)
    return request.param


@pytest.mark.parametrize("ta,tb,M,N,K", CASES)
def test_f8_layout_pm1_exact(tile, ta, tb, M, N, K):
    cfg = dg.f8_config(ta, tb, M, N, K)
    if tile == "256" and K > 256:
        assert cfg == 0
    if tile == "128" and not (ta == "T" and tb == "N" and K <= 256):
        assert cfg == 2
    print("f8 layout %s%s %dx%dx%d config %d" % (ta, tb, M, N, K, cfg), flush=True)
    x = inputs.make_shape("f8", M, N, K, dist="pm1", seed=M + 3 * N + 7 * K)
    lda, ldb = lds(ta, tb, M, N, K)
    As, Bs = store(x, ta, tb, lda, ldb)
    got, canary = run_layout(ta, tb, As, Bs, M, N, K, lda, ldb, 1.0, 1.0)
    assert canary
    exact(got, oracle.gemm(As, Bs, oracle.FMT_E4M3FN, M, N, K, ta, tb, lda, ldb))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_f8_layout_padding_and_odd_ldc(tile, ta, tb):
    M, N, K = 272, 304, 528
    print("f8 layout padding %s%s" % (ta, tb), flush=True)
    x = inputs.make_shape("f8", M, N, K, dist="pm1", seed=5)
    lda, ldb = lds(ta, tb, M, N, K, pad_a=48, pad_b=80)
    As, Bs = store(x, ta, tb, lda, ldb)
    got, canary = run_layout(ta, tb, As, Bs, M, N, K, lda, ldb, 1.0, 1.0, ldc=M + 1)
    assert canary
    exact(got, oracle.gemm(As, Bs, oracle.FMT_E4M3FN, M, N, K, ta, tb, lda, ldb))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_f8_layout_k_zero_writes_zeros(ta, tb):
    """K = 0: the empty sum, +0 in bf16 at every logical element and nothing else
    written, whatever the scales."""
    M, N = 144, 80
    print("f8 layout K=0 %s%s" % (ta, tb), flush=True)
    lda = 16 if ta == "T" else M
    ldb = 16 if tb == "N" else N
    As = np.zeros((M if ta == "T" else 1, lda), np.uint8)
    Bs = np.zeros((N if tb == "N" else 1, ldb), np.uint8)
    got, canary = run_layout(ta, tb, As, Bs, M, N, 0, lda, ldb, 3.0, 0.5)
    assert canary
    assert np.all(got == 0)


@pytest.mark.parametrize("force", ["128", "256"])
def test_f8_layouts_scaled_normal_agree(monkeypatch, force):
    """Per-tensor-scaled N(0,1) data: every layout within the bf16 tolerance of the
    binary64 oracle, and the transposed-read layouts equal to TN bit for bit on the
    same tiles."""
    M, N, K = 528, 400, 1552
    x = inputs.make_shape("f8", M, N, K, dist="normal", seed=9)
    sa, sb = x["scale_a"], x["scale_b"]
    ref = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_E4M3FN, M, N, K, scale=float(sa) * float(sb))
    monkeypatch.setenv("DG_GEMM_TILE", force)
    results = {}
    for ta, tb in LAYOUTS:
        print("f8 layout normal %s%s" % (ta, tb), flush=True)
        lda, ldb = lds(ta, tb, M, N, K)
        As, Bs = store(x, ta, tb, lda, ldb)
        got, canary = run_layout(ta, tb, As, Bs, M, N, K, lda, ldb, sa, sb)
        assert canary
        g = oracle.decode(got, oracle.FMT_BF16)
        assert np.all(np.isfinite(g))
        assert np.max(np.abs(g - ref)) / np.max(np.abs(ref)) <= BF16_TOL
        results[ta + tb] = got
    for key in ("NN", "TT", "NT"):
        assert np.array_equal(results[key], results["TN"]), key


@pytest.mark.parametrize("ta,tb", [("N", "N"), ("N", "T")])
def test_f8_layout_full_8192_sampled(monkeypatch, ta, tb):
    """8192^3 in a transposed layout on the 256 x 256 tiles: +-1 data exact on
    sampled entries, scaled N(0,1) data within the bf16 tolerance."""
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    M = N = K = 8192
    assert dg.f8_config(ta, tb, M, N, K) == 0
    rng = np.random.default_rng(23)
    ms = np.concatenate([[0, M - 1, 255, 256], rng.integers(0, M, 1200)])
    ns = np.concatenate([[0, N - 1, 256, 255], rng.integers(0, N, 1200)])
    for dist in ("pm1", "normal"):
        print("f8 layout full %s%s %s" % (ta, tb, dist), flush=True)
        x = inputs.make_shape("f8", M, N, K, dist=dist, seed=2)
        sa, sb = x["scale_a"], x["scale_b"]
        lda, ldb = lds(ta, tb, M, N, K)
        As, Bs = store(x, ta, tb, lda, ldb)
        a = torch.from_numpy(As).to(DEV)
        b = torch.from_numpy(Bs).to(DEV)
        del As, Bs
        c = torch.empty((N, M), dtype=torch.int16, device=DEV)
        dg.gemm_f8(ta, tb, a, b, c, M, N, K, lda, ldb, M, sa, sb)
        torch.cuda.synchronize()
        got = oracle.decode(c.cpu().numpy().view(np.uint16)[ns, ms], oracle.FMT_BF16)
        ref = oracle.gemm_entries(x["A"], x["B"], oracle.FMT_E4M3FN, K, ms, ns, M, N,
                                  scale=float(sa) * float(sb))
        del a, b, c
        torch.cuda.empty_cache()
        if dist == "pm1":
            assert np.array_equal(got, oracle.decode(oracle.encode(ref, oracle.FMT_BF16),
                                                     oracle.FMT_BF16))
        else:
            assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) <= BF16_TOL
