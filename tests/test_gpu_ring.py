"""GPU parity of the TN kernel's LDS ring (three A strips, two B strips).

Each K-step's A strip lands in stage t mod 3 and its B strip in stage t mod 2,
A's copies are issued two steps ahead and B's one, and an odd step count is led
by an all-zero step.  So the step counts 3 .. 10 (both parities, every phase of
the mod-3 rotation against the two-step loop; fewer steps take the skinny-K
kernel) are run with K a multiple of the K-step (the kernel form with fixed
copy offsets and empty descriptors for the steps outside the matrix) and with
a K tail (per-lane zero-fill), for fp16 and fp8, 256- and 224-wide tiles,
ragged M and N: +-1 data compared exactly with the oracle, canaries around C.
Normal data on a many-step product checks the tolerance and bit-equality with
the two-stage kernel (the same products in the same K order).
"""
import numpy as np
import pytest

import dense_gemm_tn_amd as dg
from dense_gemm_tn_amd import inputs
from test_gpu_parity import assert_exact, normwise_error, reference, run_gemm, BF16_TOL, F16_TOL

pytestmark = pytest.mark.gpu

KSTEP = {"f16": 64, "f8": 128}


@pytest.mark.parametrize("tile", ["256", "224"])
@pytest.mark.parametrize("kind", ["f16", "f8"])
@pytest.mark.parametrize("steps", list(range(3, 11)))
@pytest.mark.parametrize("tail", [0, 1])
def test_ring_step_counts_exact(monkeypatch, tile, kind, steps, tail):
    monkeypatch.setenv("DG_GEMM_TILE", tile)
    monkeypatch.delenv("DG_GEMM_RING", raising=False)
    vec = 8 if kind == "f16" else 16
    K = steps * KSTEP[kind] - (vec if tail else 0)
    M, N = 300, 470
    assert dg.tn_config(M, N, K, fp8=(kind == "f8")) == (0 if tile == "256" else 1)
    print("ring %s %s steps %d K %d" % (kind, tile, steps, K), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=steps * 31 + tail * 7 + len(tile))
    got, canary = run_gemm(kind, x, M, N, K, ldc=M + 4)
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))


@pytest.mark.parametrize("kind", ["f16", "f8"])
def test_ring_normal_data_matches_two_stage_kernel(monkeypatch, kind):
    M, N, K = 600, 700, 40 * KSTEP[kind]
    x = inputs.make_shape(kind, M, N, K, dist="normal", seed=17)
    monkeypatch.setenv("DG_GEMM_TILE", "256")
    monkeypatch.delenv("DG_GEMM_RING", raising=False)
    print("ring normal %s" % kind, flush=True)
    ring, canary = run_gemm(kind, x, M, N, K)
    assert canary
    ref = reference(kind, x, M, N, K)
    tol = F16_TOL if kind == "f16" else BF16_TOL
    assert normwise_error(kind, ring, ref) <= tol
    monkeypatch.setenv("DG_GEMM_RING", "0")
    two, canary = run_gemm(kind, x, M, N, K)
    assert canary
    assert np.array_equal(ring, two)
