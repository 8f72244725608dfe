"""GPU parity of the fused attention forward (attention_fwd_f16) against the oracle.

The oracle (``oracle.attention_rows``) is binary64 softmax attention; the kernel
computes scores and sums in fp32 and rounds the probabilities to fp16 before the
second product, and the output to fp16.  Tolerance, per element:
    |O - O_ref| <= 1e-3 * max|V_h| + 2e-3 * |O_ref| + 1e-5
  * fp16 rounding of each probability (relative 2^-11) moves O by at most
    2^-11 * max|V| (a weighted mean of V with perturbed weights), and the sum of
    weights is taken before that rounding, another 2^-11 relative;
  * the output rounding to fp16 is 2^-11 relative;
  * fp32 scores and sums, and exp2 of fp32 arguments, add far less at these
    sizes.
Cases span several 128-query tiles and 64-key blocks with ragged tails in
both, keys that straddle a 16-byte chunk, strided and padded storage (padding
poisoned with NaN), heads sharing K and V, peaked and flat softmax, and the
full 64-head 4096 x 4096 x 128 workload on sampled query rows.
"""
import math

import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
import oracle
from dense_gemm_tn_amd import inputs

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module", autouse=True)
def _ready():
    oracle.build(force=False)
    dg.lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def tol(want, vt_h):
    return 1e-3 * float(np.abs(vt_h.astype(np.float64)).max()) + 2e-3 * np.abs(want) + 1e-5


def check_head(got_h, q_h, k_h, vt_h, N, rows, scale, what):
    want = oracle.attention_rows(q_h, k_h, vt_h, N, D, rows, scale)
    got = got_h[rows].astype(np.float64)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - want)
    bound = tol(want, vt_h)
    bad = err > bound
    assert not bad.any(), "%s: %d bad, worst err %.3g at %s (bound %.3g)" % (
        what, int(bad.sum()), float(err.max()), np.unravel_index(err.argmax(), err.shape),
        float(bound.reshape(-1)[err.argmax()]) if np.ndim(bound) else float(bound))


def padded_vt(vt_np):
    """Vt [H, D, N] on the GPU with its row stride rounded up to 8 keys (16-byte rows),
    the padding filled with NaN: keys past N must never reach the output."""
    H, Dv, N = vt_np.shape
    ldv = (N + 7) // 8 * 8
    buf = torch.full((H, Dv, ldv), float("nan"), dtype=torch.float16, device="cuda")
    buf[:, :, :N] = torch.from_numpy(vt_np).cuda()
    return buf[:, :, :N]


def run(inp, scale):
    q = torch.from_numpy(inp["Q"]).cuda()
    k = torch.from_numpy(inp["K"]).cuda()
    vt = padded_vt(inp["Vt"])
    out = dg.attention(q, k, vt, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("batch,M,N", [
    (1, 128, 64),       # one tile, one key block
    (2, 300, 333),      # ragged queries and keys (333 = 5 * 64 + 13: chunk straddle)
    (3, 1, 1),          # one query, one key
    (1, 17, 5),
    (2, 257, 1000),     # 1000 = 15 * 64 + 40 (whole chunks only)
    (1, 200, 127),
    (1, 64, 8195),      # many key blocks, straddling tail
    (1, 520, 2048),
])
def test_attention_matches_oracle(batch, M, N):
    print("attention parity batch=%d M=%d N=%d" % (batch, M, N), flush=True)
    inp = inputs.make_shape("attn", M, N, D, seed=batch * 1000 + N, batch=batch)
    scale = 1.0 / math.sqrt(D)
    got = run(inp, scale)
    for h in range(batch):
        check_head(got[h], inp["Q"][h], inp["K"][h], inp["Vt"][h], N, np.arange(M), scale,
                   "head %d" % h)


@pytest.mark.parametrize("std,scale", [
    (3.0, 1.0 / math.sqrt(D)),   # logits with std ~9: peaked rows, running max moves late
    (1.0, 1.0),                  # logits with std ~11
    (1.0, 0.0),                  # every weight equal: the mean of V
])
def test_attention_softmax_regimes(std, scale):
    print("attention regimes std=%g scale=%g" % (std, scale), flush=True)
    batch, M, N = 2, 192, 700
    inp = inputs.make_shape("attn", M, N, D, seed=7, batch=batch, std=std)
    got = run(inp, scale)
    for h in range(batch):
        check_head(got[h], inp["Q"][h], inp["K"][h], inp["Vt"][h], N, np.arange(M), scale,
                   "head %d" % h)


def test_attention_strided_padding_is_never_used():
    """Padded rows (ldq, ldk > D, ldv > N) and head gaps poisoned with NaN; O written
    only at its logical positions (sentinels around it survive)."""
    print("attention strided", flush=True)
    batch, M, N = 2, 150, 77
    ldq, ldk, ldv, ldo = D + 8, D + 16, N + 11 + 8 - (N + 11) % 8, D + 24
    sq, sk, sv, so = (M + 1) * ldq, (N + 2) * ldk, (D + 3) * ldv, (M + 2) * ldo
    inp = inputs.make_shape("attn", M, N, D, seed=11, batch=batch)
    nan = np.float16(np.nan)
    qb = np.full(batch * sq, nan, np.float16)
    kbuf = np.full(batch * sk, nan, np.float16)
    vb = np.full(batch * sv, nan, np.float16)
    for h in range(batch):
        for r in range(M):
            qb[h * sq + r * ldq: h * sq + r * ldq + D] = inp["Q"][h, r]
        for r in range(N):
            kbuf[h * sk + r * ldk: h * sk + r * ldk + D] = inp["K"][h, r]
        for d in range(D):
            vb[h * sv + d * ldv: h * sv + d * ldv + N] = inp["Vt"][h, d]
    sentinel = np.float16(-1234.0)
    ob = torch.full((batch * so,), float(sentinel), dtype=torch.float16, device="cuda")
    qd, kd, vd = (torch.from_numpy(a).cuda() for a in (qb, kbuf, vb))
    scale = 0.09
    dg.attention_fwd_f16(qd, kd, vd, ob, batch, M, N, D, ldq, ldk, ldv, ldo, sq, sk, sv, so,
                         scale)
    torch.cuda.synchronize()
    o = ob.cpu().numpy()
    mask = np.zeros(batch * so, bool)
    for h in range(batch):
        got = np.stack([o[h * so + r * ldo: h * so + r * ldo + D] for r in range(M)])
        for r in range(M):
            mask[h * so + r * ldo: h * so + r * ldo + D] = True
        check_head(got, inp["Q"][h], inp["K"][h], inp["Vt"][h], N, np.arange(M), scale,
                   "head %d" % h)
    assert np.all(o[~mask] == sentinel)


def test_attention_heads_sharing_kv():
    print("attention shared kv", flush=True)
    batch, M, N = 3, 130, 200
    inp = inputs.make_shape("attn", M, N, D, seed=5, batch=batch)
    q = torch.from_numpy(inp["Q"]).cuda()
    k = torch.from_numpy(inp["K"][0].copy()).cuda()
    vt = torch.from_numpy(inp["Vt"][0].copy()).cuda()      # N = 200: rows already 16-byte
    out = torch.empty((batch, M, D), dtype=torch.float16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    dg.attention_fwd_f16(q, k, vt, out, batch, M, N, D, D, D, N, D, M * D, 0, 0, M * D, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for h in range(batch):
        check_head(got[h], inp["Q"][h], inp["K"][0], inp["Vt"][0], N, np.arange(M), scale,
                   "head %d" % h)


def test_attention_is_deterministic_and_noop_cases():
    print("attention determinism", flush=True)
    inp = inputs.make_shape("attn", 256, 300, D, seed=3, batch=2)
    a = run(inp, 0.1)
    b = run(inp, 0.1)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    out = torch.full((2, 4, D), 7.0, dtype=torch.float16, device="cuda")
    q = torch.zeros((2, 4, D), dtype=torch.float16, device="cuda")
    dg.attention_fwd_f16(q, q, q, out, 2, 0, 4, D, D, D, 4, D, 4 * D, 4 * D, 4 * D, 4 * D, 0.1)
    dg.attention_fwd_f16(q, q, q, out, 0, 4, 4, D, D, D, 4, D, 4 * D, 4 * D, 4 * D, 4 * D, 0.1)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_attention_full_workload_sampled_rows():
    """64 heads x 4096 queries x 4096 keys x 128, the launch the benchmark times:
    sampled query rows of sampled heads against the oracle, and the whole output
    checked for finiteness and for lying inside the range of V per head and dim."""
    w = inputs.WORKLOADS["attn_64x4096x4096x128"]
    print("attention full workload", flush=True)
    inp = inputs.make(w)
    scale = 1.0 / math.sqrt(D)
    q = torch.from_numpy(inp["Q"]).cuda()
    k = torch.from_numpy(inp["K"]).cuda()
    vt = torch.from_numpy(inp["Vt"]).cuda()
    out = dg.attention(q, k, vt, scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    vmin = vt.float().amin(dim=2)          # [H, D]
    vmax = vt.float().amax(dim=2)
    of = out.float()
    assert bool((of >= vmin[:, None, :] - 1e-2).all()) and bool((of <= vmax[:, None, :] + 1e-2).all())
    rng = np.random.default_rng(42)
    heads = [0, 17, 38, 63]
    got = out.cpu().numpy()
    for h in heads:
        rows = np.unique(np.concatenate([[0, 127, 128, 4095], rng.integers(0, w.M, 28)]))
        check_head(got[h], inp["Q"][h], inp["K"][h], inp["Vt"][h], w.N, rows, scale,
                   "head %d" % h)


def test_attention_million_keys():
    """2^20 + 37 keys per head (16 385 key blocks, the last cut by N; K and Vt
    heads of 256 MiB, so each block's copy offsets span far past 2^24 bytes)
    and 300 queries over two heads: sampled rows of both heads against the
    oracle, every output inside the range of V."""
    batch, M, N = 2, 300, (1 << 20) + 37
    print("attention %d keys" % N, flush=True)
    inp = inputs.make_shape("attn", M, N, D, seed=21, batch=batch)
    scale = 1.0 / math.sqrt(D)
    got = run(inp, scale)
    assert np.all(np.isfinite(got))
    vt = inp["Vt"].astype(np.float32)
    assert np.all(got >= vt.min(axis=2)[:, None, :] - 1e-2)
    assert np.all(got <= vt.max(axis=2)[:, None, :] + 1e-2)
    rows = np.array([0, 1, 127, 128, 255, 256, 299])
    for h in range(batch):
        check_head(got[h], inp["Q"][h], inp["K"][h], inp["Vt"][h], N, rows, scale, "head %d" % h)
