"""GPU parity of every GEMM tile configuration, including the 128 x 128 kernel.

The library picks a tile configuration per problem ("FP16 GEMM optimisation on
AMD RDNA 3 and RDNA 4", sections "Final results" and "Further tuning": one tile
shape is wrong for small or skinny products, so a set plus a selector is
needed).  Here each of the three K-pipelined configurations (256 x 256,
256 x 224, 128 x 128) is forced through DG_GEMM_TILE on the same ragged shapes
(M, N and K tails, a single row or column, one K-step and many), with +-1
inputs compared bit-exactly and canaries around C, plus padded leading
dimensions and an odd ldc.  The selector's own choice for the small-grid shapes
it sends to the 128 x 128 kernel is checked on the full 2048^3 problem.
"""
import numpy as np
import pytest

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs
from test_gpu_parity import (BF16_TOL, F16_TOL, assert_exact, normwise_error, reference,
                             run_gemm)

pytestmark = pytest.mark.gpu

# K rows longer than 256 bytes (shorter ones always take the skinny-K kernel).
SHAPES16 = [(1, 1, 136), (3, 5, 136), (31, 33, 264), (129, 131, 136), (257, 255, 520),
            (300, 290, 200), (513, 260, 1000), (64, 700, 3976), (700, 64, 392)]
SHAPES8 = [(1, 1, 272), (3, 5, 272), (31, 33, 528), (129, 131, 272), (257, 255, 1040),
           (513, 260, 400), (300, 290, 3856)]
FORCED = [("256", 0), ("224", 1), ("128", 2), ("pingpong", 4)]


@pytest.fixture
def force(monkeypatch):
    def _set(value):
        monkeypatch.setenv("DG_GEMM_TILE", value)
    yield _set


@pytest.mark.parametrize("tile,code", FORCED)
@pytest.mark.parametrize("kind,M,N,K", [("f16",) + s for s in SHAPES16] +
                         [("f8",) + s for s in SHAPES8])
def test_forced_tile_exact(force, tile, code, kind, M, N, K):
    force(tile)
    assert dg.tn_config(M, N, K, fp8=(kind == "f8")) == code
    print("forced tile %s %s %dx%dx%d" % (tile, kind, M, N, K), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=M * 7 + N + K)
    got, canary = run_gemm(kind, x, M, N, K)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


@pytest.mark.parametrize("tile", ["256", "224"])
@pytest.mark.parametrize("kind,M,N,K", [("f16",) + s for s in SHAPES16[3:]] +
                         [("f8",) + s for s in SHAPES8[3:]])
def test_two_stage_tn_kernel_exact(monkeypatch, tile, kind, M, N, K):
    """The TN calls' former 256-row kernel (two [A | B] LDS stages), kept for
    measurement behind DG_GEMM_RING=0: same shapes, same bits as the oracle."""
    monkeypatch.setenv("DG_GEMM_TILE", tile)
    monkeypatch.setenv("DG_GEMM_RING", "0")
    print("two-stage tn %s %s %dx%dx%d" % (tile, kind, M, N, K), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=M * 5 + N + K)
    got, canary = run_gemm(kind, x, M, N, K)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


@pytest.mark.parametrize("tile,code", FORCED)
@pytest.mark.parametrize("kind", ["f16", "f8"])
def test_forced_tile_padding_and_odd_ldc(force, tile, code, kind):
    force(tile)
    M, N, K = 270, 300, 528
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=11)
    vec = 8 if kind == "f16" else 16
    got, canary = run_gemm(kind, x, M, N, K, lda=K + vec, ldb=K + 3 * vec, ldc=M + 1)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


@pytest.mark.parametrize("tile", ["256", "128", "pingpong"])
def test_forced_tile_normal_data(force, tile):
    force(tile)
    M, N, K = 520, 390, 1544
    x = inputs.make_shape("f16", M, N, K, dist="normal", seed=5)
    got, canary = run_gemm("f16", x, M, N, K)
    assert canary
    assert normwise_error("f16", got, reference("f16", x, M, N, K)) <= F16_TOL


# The 128 x 128 kernel on N(0,1) data, every element against the oracle: both
# rings (7 K-steps: two stages; 12 or more on a 20-block grid: four), whole
# K-steps (the fixed-offset form) and K tails (the general form), fp16 and
# fp8; a second run must give the same bits.
MID_NORMAL = [("f16", 520, 390, 64 * 7), ("f16", 520, 390, 64 * 24),
              ("f16", 520, 390, 64 * 24 - 40), ("f8", 520, 390, 128 * 5),
              ("f8", 520, 390, 128 * 12), ("f8", 520, 390, 128 * 12 - 16)]


@pytest.mark.parametrize("kind,M,N,K", MID_NORMAL)
def test_mid_kernel_normal_data_both_forms(force, kind, M, N, K):
    force("128")
    ks = 64 if kind == "f16" else 128
    nk = -(-K // ks)
    print("mid normal %s %dx%dx%d (%d steps, ring %d)" % (kind, M, N, K, nk,
          dg.mid_stages(-(-M // 128) * -(-N // 128), nk)), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="normal", seed=M + K)
    got, canary = run_gemm(kind, x, M, N, K)
    assert canary
    tol = F16_TOL if kind == "f16" else BF16_TOL
    assert normwise_error(kind, got, reference(kind, x, M, N, K)) <= tol
    again, _ = run_gemm(kind, x, M, N, K)
    assert np.array_equal(got, again)


def test_selector_sends_2048_cube_to_128_tiles(monkeypatch):
    """The selector's choice on this device for the small-grid workload, run in
    full: +-1 data compared exactly everywhere, N(0,1) data on sampled entries."""
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    w = inputs.WORKLOADS["f16_2048"]
    assert dg.tn_config(w.M, w.N, w.K) == 2
    print("selector 2048^3", flush=True)
    x = inputs.make(w, dist="pm1")
    got, canary = run_gemm("f16", x, w.M, w.N, w.K)
    assert canary
    assert_exact("f16", got, reference("f16", x, w.M, w.N, w.K))
    x = inputs.make(w)
    got, canary = run_gemm("f16", x, w.M, w.N, w.K)
    rng = np.random.default_rng(3)
    ms = rng.integers(0, w.M, 2000)
    ns = rng.integers(0, w.N, 2000)
    ref = oracle.gemm_tn_entries(x["A"], x["B"], oracle.FMT_F16, w.K, ms, ns)
    g = oracle.decode(got[ns, ms], oracle.FMT_F16)
    assert np.max(np.abs(g - ref)) / np.max(np.abs(ref)) <= F16_TOL


# The 128 x 128 kernel's four-stage ring (grids of at most one block per CU
# with at least eight K-steps): step counts at and just past the floor, so the
# loop's last three steps take each of its waits (no, one, two later steps in
# flight), with a K tail inside the last step; and one count below the floor
# (the two-stage ring).  fp16 K-steps are 64 elements, fp8 128.  The same
# counts with whole K-steps (no tail) run the fixed-offset form of both rings,
# whose copies past the last step read an empty descriptor; 1 and 2 steps put
# those copies in the prologue.
RING = [("f16", 300, 260, 64 * n - 8) for n in (7, 8, 9, 10, 11, 33)] + \
       [("f8", 257, 300, 128 * n - 16) for n in (7, 8, 9, 10, 21)] + \
       [("f16", 300, 260, 64 * n) for n in (1, 2, 7, 8, 9, 10, 33)] + \
       [("f8", 257, 300, 128 * n) for n in (1, 7, 8, 9, 10)]


@pytest.mark.parametrize("kind,M,N,K", RING)
def test_mid_ring_step_counts_exact(force, kind, M, N, K):
    force("128")
    print("mid ring %s %dx%dx%d" % (kind, M, N, K), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=M + N + K)
    got, canary = run_gemm(kind, x, M, N, K, ldc=M + 4)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


def test_mid_ring_batched_heads_exact(force):
    """Strided heads through the four-stage ring (three 300 x 300 heads, a
    1024-deep contraction: 27 blocks of 16 K-steps), head gaps untouched."""
    import torch
    from test_gpu_parity import CANARY16, DEV
    force("128")
    H, M, N, D = 3, 300, 300, 1024
    assert dg.mid_stages(H * 9, D // 64) == 4 or torch.cuda.get_device_properties(0).multi_processor_count < 27
    x = inputs.make_shape("qkt", M, N, D, dist="pm1", seed=17, batch=H)
    q = torch.from_numpy(x["Q"]).to(DEV)
    k = torch.from_numpy(x["K"]).to(DEV)
    ld, stride = M + 4, N * (M + 4) + 40
    s = torch.full((H * stride,), CANARY16, dtype=torch.int32, device=DEV).to(torch.int16)
    dg.gemm_batched_qkt(q, k, s, H, M, N, D, D, D, ld, M * D, N * D, stride)
    torch.cuda.synchronize()
    host = s.cpu().numpy().view(np.uint16)
    for h in range(H):
        blk = host[h * stride:(h + 1) * stride]
        body = blk[:N * ld].reshape(N, ld)
        assert np.all(body[:, M:] == CANARY16) and np.all(blk[N * ld:] == CANARY16)
        ref = oracle.gemm_tn(x["Q"][h], x["K"][h], oracle.FMT_F16, M, N, D)
        assert_exact("qkt", np.ascontiguousarray(body[:, :M]), ref)
