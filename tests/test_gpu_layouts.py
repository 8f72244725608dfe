"""GPU parity of the fp16 GEMM in all four op-code layouts (gemm_f16) against the oracle.

Data in another layout would otherwise have to be transposed before the TN
kernel ("FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we
compute"); gemm_f16 reads each operand as it lies: A 'T' = A[m*lda + k],
A 'N' = A[m + k*lda], B 'N' = B[k + n*ldb], B 'T' = B[k*ldb + n] (the
row-major NN indexing of section 11.1 of the hello-gpu chapter is the 'N','N'
case on swapped operands).  The expected values come from ``oracle.gemm``,
which reads the same stored buffers through the layout's own strides.

Bars (as for the TN path): +-1 inputs bit-exact; N(0,1) inputs within
max|C - C_ref| / max|C_ref| <= 4e-3; memory around C and the ldc padding never
written; operand padding (NaN) never read into a stored element.  The non-TN
layouts run the TN kernels (256 x 256 or 128 x 128 tiles) with only the staging
and fragment reads changed, so on the same logical operands, with the same
configuration forced, all four give the same bits.  Every shape runs under the
library's own choice and with each configuration forced (DG_GEMM_TILE).
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs
from test_gpu_parity import CANARY16, DEV, F16_TOL

pytestmark = pytest.mark.gpu

LAYOUTS = [("T", "N"), ("N", "N"), ("T", "T"), ("N", "T")]
F16_NAN = np.uint16(0x7E00)

# Shapes every layout accepts (M, N, K multiples of 8): one tile and one K-step,
# ragged tiles, K tails inside a 64-element step, many steps, skinny grids.
COMMON = [(8, 8, 8), (16, 24, 8), (128, 128, 64), (136, 264, 200), (256, 384, 1000),
          (520, 392, 72), (1000, 1000, 136), (64, 1200, 3976), (1200, 64, 392)]
# Extents only some layouts accept: M (N) need not be a multiple of 8 when A (B)
# is K-contiguous, and K need not be one when neither operand is.
EXTRA = {
    ("T", "N"): [(131, 133, 200), (1, 1, 8)],
    ("N", "N"): [(136, 131, 200), (264, 1, 72)],
    ("T", "T"): [(131, 136, 200), (1, 264, 72)],
    ("N", "T"): [(136, 264, 203), (128, 128, 1), (256, 136, 65), (8, 8, 3)],
}
CASES = [(ta, tb) + s for ta, tb in LAYOUTS for s in COMMON + EXTRA[(ta, tb)]]


def store_a(a_logical, ta, ld):
    """op(A) (M x K) laid out for op code ta with leading dimension ld, padding NaN:
    'T' -> [M, ld] rows along K; 'N' -> [K, ld] rows along M."""
    src = a_logical if ta == "T" else a_logical.T
    return _pad(src, ld)


def store_b(b_rows, tb, ld):
    """op(B) given as [N, K] (row n = column n of op(B)) laid out for op code tb:
    'N' -> [N, ld] rows along K; 'T' -> [K, ld] rows along N."""
    src = b_rows if tb == "N" else b_rows.T
    return _pad(src, ld)


def _pad(src, ld):
    rows, cols = src.shape
    out = np.full((rows, ld), F16_NAN, dtype=np.uint16).view(np.float16)
    out[:, :cols] = src
    return np.ascontiguousarray(out)


def run_layout(ta, tb, As, Bs, M, N, K, lda, ldb, ldc=None, guard=64):
    """C (as [N, M] fp16 codes) from gemm_f16 with canaries around it."""
    ldc = M if ldc is None else ldc
    a = torch.from_numpy(As.view(np.int16)).to(DEV)
    b = torch.from_numpy(Bs.view(np.int16)).to(DEV)
    total = guard * 2 + max(N * ldc, 1)
    c = torch.full((total,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    dg.gemm_f16(ta, tb, a, b, c.data_ptr() + guard * 2, M, N, K, lda, ldb, ldc)
    torch.cuda.synchronize()
    host = c.cpu().numpy().view(np.uint16)
    body = host[guard:guard + N * ldc].reshape(N, ldc)
    canary = (np.all(host[:guard] == CANARY16) and np.all(host[guard + N * ldc:] == CANARY16)
              and np.all(body[:, M:] == CANARY16))
    return np.ascontiguousarray(body[:, :M]), canary


def case(ta, tb, M, N, K, dist, seed, pad_a=0, pad_b=0):
    x = inputs.make_shape("f16", M, N, K, dist=dist, seed=seed)
    lda = (K if ta == "T" else M) + pad_a
    ldb = (K if tb == "N" else N) + pad_b
    As = store_a(x["A"], ta, lda)
    Bs = store_b(x["B"], tb, ldb)
    return x, As, Bs, lda, ldb


def exact(got_codes, ref):
    got = oracle.decode(got_codes, oracle.FMT_F16)
    want = oracle.decode(oracle.encode(ref, oracle.FMT_F16), oracle.FMT_F16)
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
def test_layout_pm1_exact(tile, ta, tb, M, N, K):
    cfg = dg.f16_config(ta, tb, M, N, K)
    if tile == "256" and K > 128:
        assert cfg == 0
    if tile == "128" and not (ta == "T" and tb == "N" and K <= 128):
        assert cfg == 2
    print("layout %s%s %dx%dx%d config %d" % (ta, tb, M, N, K, cfg), flush=True)
    x, As, Bs, lda, ldb = case(ta, tb, M, N, K, "pm1", seed=M + 3 * N + 7 * K)
    got, canary = run_layout(ta, tb, As, Bs, M, N, K, lda, ldb)
    assert canary
    exact(got, oracle.gemm(As, Bs, oracle.FMT_F16, M, N, K, ta, tb, lda, ldb))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_layout_padding_and_odd_ldc(tile, ta, tb):
    """Padded rows (NaN-filled) on both operands and an odd ldc (narrow stores)."""
    M, N, K = 272, 296, 520
    print("layout padding %s%s" % (ta, tb), flush=True)
    x, As, Bs, lda, ldb = case(ta, tb, M, N, K, "pm1", seed=5, pad_a=24, pad_b=40)
    got, canary = run_layout(ta, tb, As, Bs, M, N, K, lda, ldb, ldc=M + 1)
    assert canary
    exact(got, oracle.gemm(As, Bs, oracle.FMT_F16, M, N, K, ta, tb, lda, ldb))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_layout_k_zero_writes_zeros(ta, tb):
    M, N = 136, 72
    print("layout K=0 %s%s" % (ta, tb), flush=True)
    lda = 8 if ta == "T" else M
    ldb = 8 if tb == "N" else N
    As = np.zeros((M if ta == "T" else 1, lda), np.float16)
    Bs = np.zeros((N if tb == "N" else 1, ldb), np.float16)
    got, canary = run_layout(ta, tb, As, Bs, M, N, 0, lda, ldb)
    assert canary
    assert np.all(oracle.decode(got, oracle.FMT_F16) == 0)


@pytest.mark.parametrize("force", ["128", "256"])
def test_layouts_agree_bit_for_bit(monkeypatch, force):
    """N(0,1) data: every layout within the tolerance of the binary64 oracle, and the
    three transposed-read layouts equal to TN on the same tiles bit for bit."""
    M, N, K = 520, 392, 1544
    x = inputs.make_shape("f16", M, N, K, dist="normal", seed=9)
    ref = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, M, N, K)
    monkeypatch.setenv("DG_GEMM_TILE", force)
    results = {}
    for ta, tb in LAYOUTS:
        print("layout normal %s%s" % (ta, tb), flush=True)
        lda = K if ta == "T" else M
        ldb = K if tb == "N" else N
        got, canary = run_layout(ta, tb, store_a(x["A"], ta, lda), store_b(x["B"], tb, ldb),
                                 M, N, K, lda, ldb)
        assert canary
        g = oracle.decode(got, oracle.FMT_F16)
        assert np.all(np.isfinite(g))
        assert np.max(np.abs(g - ref)) / np.max(np.abs(ref)) <= F16_TOL
        results[ta + tb] = got
    for key in ("NN", "TT", "NT"):
        assert np.array_equal(results[key], results["TN"]), key


@pytest.mark.parametrize("ta,tb", [("N", "N"), ("T", "T"), ("N", "T")])
def test_layout_full_4096_sampled(monkeypatch, ta, tb):
    """The 4096^3 product in each transposed layout, in the configuration the library
    picks (256 x 256 tiles): +-1 data exact on sampled entries (every entry an
    integer), N(0,1) data on sampled entries within the tolerance."""
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    M = N = K = 4096
    assert dg.f16_config(ta, tb, M, N, K) == 0
    rng = np.random.default_rng(17)
    ms = np.concatenate([[0, M - 1, 127, 128], rng.integers(0, M, 1500)])
    ns = np.concatenate([[0, N - 1, 128, 127], rng.integers(0, N, 1500)])
    for dist in ("pm1", "normal"):
        print("layout full %s%s %s" % (ta, tb, dist), flush=True)
        x, As, Bs, lda, ldb = case(ta, tb, M, N, K, dist, seed=1)
        a = torch.from_numpy(As.view(np.int16)).to(DEV)
        b = torch.from_numpy(Bs.view(np.int16)).to(DEV)
        c = torch.empty((N, M), dtype=torch.int16, device=DEV)
        dg.gemm_f16(ta, tb, a, b, c, M, N, K, lda, ldb, M)
        torch.cuda.synchronize()
        got = oracle.decode(c.cpu().numpy().view(np.uint16)[ns, ms], oracle.FMT_F16)
        ref = oracle.gemm_entries(As, Bs, oracle.FMT_F16, K, ms, ns, M, N, ta, tb, lda, ldb)
        if dist == "pm1":
            assert np.array_equal(got, ref)
        else:
            assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) <= F16_TOL


def test_matmul_f16_helper_shapes():
    """The tensor helper reads each operand's shape from its op code."""
    M, N, K = 136, 72, 96
    x = inputs.make_shape("f16", M, N, K, dist="pm1", seed=2)
    ref = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, M, N, K)
    for ta, tb in LAYOUTS:
        a = torch.from_numpy(np.ascontiguousarray(x["A"] if ta == "T" else x["A"].T)).to(DEV)
        b = torch.from_numpy(np.ascontiguousarray(x["B"] if tb == "N" else x["B"].T)).to(DEV)
        out = dg.matmul_f16(a, b, ta, tb)
        torch.cuda.synchronize()
        exact(out.cpu().numpy().view(np.uint16), ref)
