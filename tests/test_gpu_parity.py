"""GPU path vs CPU oracle, element by element (gfx950, through the C ABI).

Bars:
  * +-1 inputs: bit-exact.  Every partial sum is an integer of magnitude <= K, so
    the fp32 accumulation is exact in any order and the single rounding to the
    output format is the oracle's ("FP16 GEMM optimisation on AMD RDNA 3 and
    RDNA 4", section "What we compute", exact comparison on +-1 inputs).
  * normal inputs: max|C - C_ref| / max|C_ref| <= 4e-3 for fp16 output and
    <= 1e-2 for bf16 output (FP8 path), C_ref the unrounded binary64 oracle.
  * memory around C and in the ldc padding is never written (section 11.4 of the
    hello-gpu chapter: invalid C is not written).
Shapes: the edge shapes of section 11.4 (K rounded up to the 16-byte vector),
multi-tile ragged shapes, K tails, and the five full-size workloads compared
over every output element (N(0,1) data within the bar, +-1 data exact, plus
the +-1 invariants |C| <= K and C = K mod 2).
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
CANARY16 = 0x7BCD  # a finite fp16 / bf16 pattern no kernel writes by accident
F16_TOL = 4e-3
BF16_TOL = 1e-2


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _padded(src: np.ndarray, ld: int) -> np.ndarray:
    """Rows of src placed in a wider row stride ld; the padding holds a nonzero
    value (7.0 or the E4M3FN code of 1.0) that must never enter the sum."""
    rows, cols = src.shape
    fill = np.float16(7.0) if src.dtype == np.float16 else np.uint8(0x38)
    out = np.full((rows, ld), fill, dtype=src.dtype)
    out[:, :cols] = src
    return out


def run_gemm(kind, x, M, N, K, lda=None, ldb=None, ldc=None, guard=64):
    """Launch through the C ABI with C inside a canary-filled allocation.

    Returns (C as [N, M] uint16 codes, canary_ok)."""
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = M if ldc is None else ldc
    A = x["A"] if lda == K else _padded(x["A"], lda)
    B = x["B"] if ldb == K else _padded(x["B"], ldb)
    a = _dev(A.view(np.int16) if A.dtype == np.float16 else A)
    b = _dev(B.view(np.int16) if B.dtype == np.float16 else B)
    total = guard * 2 + max(N * ldc, 1)
    c = torch.full((total,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    cptr = c.data_ptr() + guard * 2
    if kind == "f16":
        dg.gemm_f16_tn(a, b, cptr, M, N, K, lda, ldb, ldc)
    else:
        dg.gemm_f8_tn(a, b, cptr, M, N, K, lda, ldb, ldc, x["scale_a"], x["scale_b"])
    torch.cuda.synchronize()
    host = c.cpu().numpy().view(np.uint16)
    body = host[guard:guard + N * ldc].reshape(N, ldc) if N else np.zeros((0, ldc), np.uint16)
    ok = (np.all(host[:guard] == CANARY16) and np.all(host[guard + N * ldc:] == CANARY16)
          and np.all(body[:, M:] == CANARY16))
    return np.ascontiguousarray(body[:, :M]), ok


def out_fmt(kind):
    return oracle.FMT_F16 if kind in ("f16", "qkt") else oracle.FMT_BF16


def in_fmt(kind):
    return oracle.FMT_F16 if kind in ("f16", "qkt") else oracle.FMT_E4M3FN


def reference(kind, x, M, N, K):
    scale = float(x["scale_a"]) * float(x["scale_b"]) if kind == "f8" else 1.0
    return oracle.gemm_tn(x["A"], x["B"], in_fmt(kind), M, N, K, scale=scale)


def assert_exact(kind, got_codes, ref):
    got = oracle.decode(got_codes, out_fmt(kind))
    want = oracle.decode(oracle.encode(ref, out_fmt(kind)), out_fmt(kind))
    bad = got != want
    assert not bad.any(), "%d of %d elements differ; first at [n,m]=%s: got %r want %r" % (
        bad.sum(), bad.size, np.argwhere(bad)[0], got[bad][0], want[bad][0])


def normwise_error(kind, got_codes, ref):
    got = oracle.decode(got_codes, out_fmt(kind))
    assert np.all(np.isfinite(got))
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / denom) if denom > 0 else float(np.max(np.abs(got)))


# Edge shapes of section 11.4 (1x1x1, 3x5x7, 15x17x19, 17x19x23, 31x33x29) with K
# rounded up to the 16-byte vector, plus multi-tile ragged shapes and K tails.
# K rows of at most 256 bytes take the skinny-K kernel (fp16 K <= 128, fp8
# K <= 256); longer ones, on grids this small, the 128 x 128 kernel (the
# library's selector).  The 256-row kernels get ragged shapes of their own in
# test_gpu_tiles.py (forced configuration) and below (large grids).
EDGE = [(1, 1, 8), (3, 5, 8), (15, 17, 24), (17, 19, 24), (31, 33, 32)]
EDGE8 = [(1, 1, 16), (3, 5, 16), (15, 17, 32), (17, 19, 32), (31, 33, 32)]
RAGGED = [(256, 256, 256), (300, 290, 200), (257, 255, 72), (513, 260, 136), (64, 700, 64),
          (700, 64, 1000), (1000, 1000, 8), (260, 300, 128), (129, 131, 136), (383, 385, 264)]
RAGGED8 = [(256, 256, 256), (300, 290, 208), (257, 255, 144), (513, 260, 112), (64, 700, 64),
           (700, 64, 1008), (1000, 1000, 16), (300, 290, 272), (513, 260, 400),
           (256, 256, 512), (129, 131, 528)]


@pytest.mark.parametrize("M,N,K", EDGE + RAGGED)
@pytest.mark.parametrize("dist", ["pm1", "normal"])
def test_f16_shapes(M, N, K, dist):
    x = inputs.make_shape("f16", M, N, K, dist=dist, seed=M + N + K)
    got, canary = run_gemm("f16", x, M, N, K)
    assert canary
    ref = reference("f16", x, M, N, K)
    if dist == "pm1":
        assert_exact("f16", got, ref)
    else:
        assert normwise_error("f16", got, ref) <= F16_TOL


@pytest.mark.parametrize("M,N,K", EDGE8 + RAGGED8)
@pytest.mark.parametrize("dist", ["pm1", "normal"])
def test_f8_shapes(M, N, K, dist):
    x = inputs.make_shape("f8", M, N, K, dist=dist, seed=M + N + K)
    got, canary = run_gemm("f8", x, M, N, K)
    assert canary
    ref = reference("f8", x, M, N, K)
    if dist == "pm1":
        assert_exact("f8", got, ref)
    else:
        assert normwise_error("f8", got, ref) <= BF16_TOL


@pytest.mark.parametrize("kind", ["f16", "f8"])
def test_padded_leading_dimensions(kind):
    M, N, K = 270, 300, 160
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=9)
    got, canary = run_gemm(kind, x, M, N, K, lda=K + 32, ldb=K + 64, ldc=M + 10)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


@pytest.mark.parametrize("kind", ["f16", "f8"])
def test_odd_ldc_uses_narrow_stores(kind):
    M, N, K = 37, 41, 64
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=10)
    got, canary = run_gemm(kind, x, M, N, K, ldc=M + 3)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


@pytest.mark.parametrize("kind", ["f16", "f8"])
def test_k_zero_writes_zeros(kind):
    M, N = 40, 30
    x = {"A": np.zeros((M, 0), np.float16 if kind == "f16" else np.uint8),
         "B": np.zeros((N, 0), np.float16 if kind == "f16" else np.uint8),
         "scale_a": 1.0, "scale_b": 1.0}
    got, canary = run_gemm(kind, x, M, N, 0, lda=16, ldb=16)
    assert canary
    assert np.all(oracle.decode(got, out_fmt(kind)) == 0)


def test_identity_gives_exact_copy():
    """A = I: C holds B exactly; B = I: C holds A transposed (special cases of 11.1)."""
    n = 320
    I = np.eye(n, dtype=np.float16)
    rng = np.random.default_rng(0)
    Bm = rng.standard_normal((300, n)).astype(np.float16)
    got, ok = run_gemm("f16", {"A": I, "B": Bm}, n, 300, n)
    assert ok and np.array_equal(got, Bm.view(np.uint16))
    got, ok = run_gemm("f16", {"A": Bm, "B": I}, 300, n, n)
    assert ok and np.array_equal(got, np.ascontiguousarray(Bm.T).view(np.uint16))


def test_batched_qkt_small():
    H, M, N, D = 3, 100, 70, 128
    x = inputs.make_shape("qkt", M, N, D, dist="normal", seed=4, batch=H, std=128 ** -0.5)
    q = _dev(x["Q"])
    k = _dev(x["K"])
    s = dg.qkt(q, k)
    torch.cuda.synchronize()
    ref = oracle.batched_qkt(x["Q"], x["K"], H, M, N, D)
    got = s.view(torch.int16).cpu().numpy().view(np.uint16)
    for h in range(H):
        assert normwise_error("qkt", got[h], ref[h]) <= F16_TOL
    # +-1 exact, and the swapped call gives the transposed (row-major) result
    x = inputs.make_shape("qkt", M, N, D, dist="pm1", seed=5, batch=H)
    q, k = _dev(x["Q"]), _dev(x["K"])
    s = dg.qkt(q, k)
    st = dg.qkt(k, q)
    torch.cuda.synchronize()
    ref = oracle.batched_qkt(x["Q"], x["K"], H, M, N, D)
    got = s.view(torch.int16).cpu().numpy().view(np.uint16)
    gott = st.view(torch.int16).cpu().numpy().view(np.uint16)
    for h in range(H):
        assert_exact("qkt", got[h], ref[h])
        assert np.array_equal(gott[h], got[h].T)


@pytest.mark.parametrize("H,M,N,D,pad", [(12, 640, 520, 128, 0), (12, 640, 520, 64, 8),
                                         (2, 1024, 2048, 128, 0), (3, 136, 264, 32, 16)])
def test_batched_qkt_many_tiles(H, M, N, D, pad):
    """More 128 x 128 tiles than CUs, N tails, a padded lds, and a K shorter
    than the LDS row (grids this small give every block a single M tile)."""
    x = inputs.make_shape("qkt", M, N, D, dist="pm1", seed=H + M + D, batch=H)
    q, k = _dev(x["Q"]), _dev(x["K"])
    lds = M + pad
    s = torch.full((H, N, lds), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    dg.gemm_batched_qkt(q, k, s, H, M, N, D, D, D, lds, M * D, N * D, N * lds)
    torch.cuda.synchronize()
    got = s.cpu().numpy().view(np.uint16)
    ref = oracle.batched_qkt(x["Q"], x["K"], H, M, N, D)
    for h in range(H):
        assert_exact("qkt", np.ascontiguousarray(got[h, :, :M]), ref[h])
        assert np.all(got[h, :, M:] == CANARY16)


@pytest.mark.parametrize("H,M,N,D,pad", [(64, 4000, 3000, 128, 8), (8, 8152, 1000, 64, 0)])
def test_batched_qkt_walks(H, M, N, D, pad):
    """Grids of at least eight skinny-K blocks per CU, where each block walks
    several M tiles of one column (16 and 2 here) and the walk ends on a ragged
    M tile; +-1 data, so sampled entries are exact, and the lds padding keeps
    its canaries."""
    x = inputs.make_shape("qkt", M, N, D, dist="pm1", seed=H + M, batch=H)
    q, k = _dev(x["Q"]), _dev(x["K"])
    lds = M + pad
    s = torch.full((H, N, lds), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    dg.gemm_batched_qkt(q, k, s, H, M, N, D, D, D, lds, M * D, N * D, N * lds)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for h in sorted({0, H - 1} | set(rng.integers(0, H, 3).tolist())):
        ms, ns = sample_entries(M, N, 400, seed=h)
        ms = np.concatenate([ms, np.arange(M - 130, M)])  # the last, ragged M tile
        ns = np.concatenate([ns, np.full(130, N - 1)])
        ref = oracle.gemm_tn_entries(x["Q"][h], x["K"][h], oracle.FMT_F16, D, ms, ns)
        got = s[h].cpu().numpy().view(np.uint16)
        assert_exact("qkt", got[ns, ms], ref)
        if pad:
            assert np.all(got[:, M:] == CANARY16)
    del s
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind,M,N,K", [("f16", 4024, 3996, 3976), ("f8", 4024, 3996, 3856),
                                        ("f16", 1000, 700, 3976)])
def test_ragged_large_tiles(kind, M, N, K):
    """Grids large enough for 256-row tiles (the small ragged case takes the
    128 x 128 kernel),
    with M, N and K tails and an odd K-step count; +-1 data, sampled entries
    exact, the whole tail row and column exact, canaries intact."""
    assert dg.tn_config(M, N, K, fp8=(kind == "f8")) == (0 if M > 1000 else 2)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=M + N + K)
    got, canary = run_gemm(kind, x, M, N, K)
    assert canary
    ms, ns = sample_entries(M, N, 1500, seed=K)
    ms = np.concatenate([ms, np.arange(M), np.full(N, M - 1)])
    ns = np.concatenate([ns, np.full(M, N - 1), np.arange(N)])
    scale = float(x["scale_a"]) * float(x["scale_b"]) if kind == "f8" else 1.0
    ref = oracle.gemm_tn_entries(x["A"], x["B"], in_fmt(kind), K, ms, ns, scale=scale)
    assert_exact(kind, got[ns, ms], ref)


# ------------------------------------------------------------- full-size workloads

def sample_entries(M, N, count, seed):
    """Corners, tile edges and random entries of an M x N output."""
    rng = np.random.default_rng(seed)
    edges_m = sorted({0, 1, 15, 16, 127, 128, 255, 256, M // 2, M - 2, M - 1} & set(range(M)))
    edges_n = sorted({0, 1, 15, 16, 127, 128, 255, 256, N // 2, N - 2, N - 1} & set(range(N)))
    ms = [m for m in edges_m for _ in edges_n]
    ns = [n for _ in edges_m for n in edges_n]
    ms += list(rng.integers(0, M, count))
    ns += list(rng.integers(0, N, count))
    return np.asarray(ms, np.int64), np.asarray(ns, np.int64)


def _full_size(name, dist=None):
    """The workload through the C ABI, compared with the oracle's product over
    every element (the whole M x N output, unrounded binary64)."""
    w = inputs.WORKLOADS[name]
    print("full-size %s dist=%s" % (name, dist or w.dist), flush=True)
    x = inputs.make(w, dist=dist)
    got, canary = run_gemm(w.kind, x, w.M, w.N, w.K)
    assert canary
    ref = reference(w.kind, x, w.M, w.N, w.K)
    return w, x, got, ref


def _pm1_invariants(w, got):
    """+-1 inputs: every output is an integer of magnitude <= K and of K's parity
    (after rounding too: fp16 holds them exactly for K <= 4096, and every bf16
    value of magnitude >= 256 is even)."""
    vals = oracle.decode(got, out_fmt(w.kind))
    assert np.all(np.abs(vals) <= w.K) and np.all((vals - w.K) % 2 == 0)


def test_c1_f16_256_pm1_exact_full():
    w = inputs.WORKLOADS["f16_256_pm1"]
    x = inputs.make(w)
    got, canary = run_gemm("f16", x, w.M, w.N, w.K)
    assert canary
    assert_exact("f16", got, reference("f16", x, w.M, w.N, w.K))


def test_c2_f16_4096_normal_full():
    w, x, got, ref = _full_size("f16_4096")
    assert normwise_error("f16", got, ref) <= F16_TOL


def test_c2_f16_4096_pm1_exact_full():
    w, x, got, ref = _full_size("f16_4096", dist="pm1")
    assert_exact("f16", got, ref)
    _pm1_invariants(w, got)


def test_c3_f16_wide_ragged_normal_full():
    w, x, got, ref = _full_size("f16_1920x13900x4096")
    assert normwise_error("f16", got, ref) <= F16_TOL


def test_c3_f16_wide_ragged_pm1_exact_full():
    w, x, got, ref = _full_size("f16_1920x13900x4096_pm1")
    assert_exact("f16", got, ref)
    _pm1_invariants(w, got)


def test_c4_f8_8192_normal_full():
    w, x, got, ref = _full_size("f8_8192")
    assert normwise_error("f8", got, ref) <= BF16_TOL


def test_c4_f8_8192_pm1_exact_full():
    w, x, got, ref = _full_size("f8_8192", dist="pm1")
    assert_exact("f8", got, ref)
    _pm1_invariants(w, got)


def _c5_heads(dist):
    """The batched QK^T workload (64 heads of 4096 x 4096, K = 128), every head
    compared in full with the oracle, one head at a time.  Returns, over all
    heads, max|S - S_ref| and max|S_ref| (the normwise metric of the whole
    output) and the number of heads with an inexact element (+-1 data)."""
    w = inputs.WORKLOADS["qkt_64x4096x4096x128"]
    print("full-size %s dist=%s" % (w.name, dist), flush=True)
    x = inputs.make(w, dist=dist)
    q, k = _dev(x["Q"]), _dev(x["K"])
    s = dg.qkt(q, k)
    torch.cuda.synchronize()
    err = top = 0.0
    inexact = []
    for h in range(w.batch):
        got = s[h].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.gemm_tn(x["Q"][h], x["K"][h], oracle.FMT_F16, w.M, w.N, w.K)
        vals = oracle.decode(got, oracle.FMT_F16)
        assert np.all(np.isfinite(vals)), h
        err = max(err, float(np.max(np.abs(vals - ref))))
        top = max(top, float(np.max(np.abs(ref))))
        if dist == "pm1":
            want = oracle.decode(oracle.encode(ref, oracle.FMT_F16), oracle.FMT_F16)
            if not np.array_equal(vals, want):
                inexact.append(h)
    del s
    torch.cuda.empty_cache()
    return err, top, inexact


def test_c5_batched_qkt_normal_full():
    err, top, _ = _c5_heads("normal")
    assert err / top <= F16_TOL


def test_c5_batched_qkt_pm1_exact_full():
    _, _, inexact = _c5_heads("pm1")
    assert not inexact, "heads with inexact elements: %s" % inexact


@pytest.mark.parametrize("H,M,N,D,extra", [(3, 136, 264, 128, 4), (3, 136, 264, 128, 1),
                                           (2, 300, 260, 256, 4), (2, 300, 260, 256, 3)])
def test_batched_head_stride_not_16_byte_aligned(H, M, N, D, extra):
    """stride_s a multiple of 4 but not 8 (heads 8-byte aligned) or odd (2-byte
    aligned): S is stored in narrower pieces, exact on +-1, and the gaps
    between heads keep their canaries (skinny-K kernel for D = 128, the
    pipelined kernels for D = 256)."""
    x = inputs.make_shape("qkt", M, N, D, dist="pm1", seed=H + M + extra, batch=H)
    q, k = _dev(x["Q"]), _dev(x["K"])
    lds = M
    stride_s = N * lds + extra
    flat = torch.full((H * stride_s + 64,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    dg.gemm_batched_qkt(q, k, flat, H, M, N, D, D, D, lds, M * D, N * D, stride_s)
    torch.cuda.synchronize()
    host = flat.cpu().numpy().view(np.uint16)
    ref = oracle.batched_qkt(x["Q"], x["K"], H, M, N, D)
    for h in range(H):
        got = host[h * stride_s:h * stride_s + N * lds].reshape(N, lds)
        assert_exact("qkt", np.ascontiguousarray(got), ref[h])
        assert np.all(host[h * stride_s + N * lds:(h + 1) * stride_s] == CANARY16)
    assert np.all(host[H * stride_s:] == CANARY16)
