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


def _draw(n=48, seed=4242):
    """Seeded TN shapes with whole K-steps (the ring kernel's fixed-offset
    form), ragged M and N, padded leading dimensions and ldc, the tile width
    chosen or forced."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = "f16" if i % 2 == 0 else "f8"
        vec = 8 if kind == "f16" else 16
        big = rng.random() < 0.5
        M = int(rng.integers(200, 3000)) if big else int(rng.integers(1, 900))
        N = int(rng.integers(200, 3000)) if big else int(rng.integers(1, 900))
        steps = int(rng.integers(3, 40))
        while M * N * steps * KSTEP[kind] > 3e9:
            steps = max(3, steps // 2)
            if steps == 3:
                break
        out.append({"kind": kind, "M": M, "N": N, "K": steps * KSTEP[kind],
                    "pad_a": int(rng.integers(0, 3)) * vec, "pad_b": int(rng.integers(0, 3)) * vec,
                    "ldc_pad": int(rng.choice([0, 0, 1, 8])),
                    "tile": rng.choice([None, None, "256", "224"]), "seed": 7000 + i})
    return out


RANDOM = _draw()


@pytest.mark.parametrize("c", RANDOM, ids=["%s-%dx%dx%d-%s" % (c["kind"], c["M"], c["N"], c["K"],
                                                             c["tile"] or "auto") for c in RANDOM])
def test_ring_random_whole_steps_exact(monkeypatch, c):
    monkeypatch.delenv("DG_GEMM_RING", raising=False)
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    if c["tile"]:
        monkeypatch.setenv("DG_GEMM_TILE", str(c["tile"]))
    kind, M, N, K = c["kind"], c["M"], c["N"], c["K"]
    print("ring random %s %dx%dx%d tile %s" % (kind, M, N, K, c["tile"]), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="pm1", seed=c["seed"])
    got, canary = run_gemm(kind, x, M, N, K, lda=K + c["pad_a"], ldb=K + c["pad_b"],
                           ldc=M + c["ldc_pad"])
    assert canary
    assert_exact(kind, got, reference(kind, x, M, N, K))
