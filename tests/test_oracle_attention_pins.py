"""Pins of the attention oracle (``oracle.attention_rows``) to facts it does not supply.

The pages name fusing the product with softmax as the next step (hello-gpu chapter
11, chapter summary) and motivate fused attention for QK^T (mlqm.cn TileLang
attention page) but print no formula or example, so every pin here is a fact of
the mathematics of O = softmax(scale * Q K^T) V:
  * closed forms: a zero query averages V; one key returns its row; two keys
    whose logits differ by ln 3 weigh 1/4 and 3/4; a dominant logit returns its row;
  * invariances: a constant added to every key, a permutation of keys and values;
  * linearity in V and the convex-hull bound on every output;
  * random inputs against scipy's softmax and a numpy product (a library route);
  * strided storage against packed storage.
A plausible slip -- a transposed V, a wrong sign of the max shift, a missing
normalisation, a scale applied twice, a dropped key -- breaks at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _f16(x):
    return np.asarray(x, dtype=np.float16)


def _run(q, k, v, scale, rows=None, **kw):
    """q [M, D], k [N, D], v [N, D] as float arrays exactly representable in fp16."""
    N, D = k.shape
    rows = np.arange(q.shape[0]) if rows is None else rows
    return oracle.attention_rows(_f16(q), _f16(k), _f16(np.ascontiguousarray(v.T)), N, D,
                                 rows, scale, **kw)


def test_zero_query_averages_values():
    rng = np.random.default_rng(1)
    N, D = 29, 16
    k = _f16(rng.standard_normal((N, D))).astype(np.float64)
    v = _f16(rng.standard_normal((N, D))).astype(np.float64)
    o = _run(np.zeros((3, D)), k, v, 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=0, atol=1e-14)


def test_single_key_returns_its_value_row():
    rng = np.random.default_rng(2)
    D = 8
    k = _f16(rng.standard_normal((1, D))).astype(np.float64)
    v = _f16(rng.standard_normal((1, D))).astype(np.float64)
    q = _f16(rng.standard_normal((4, D))).astype(np.float64)
    o = _run(q, k, v, 3.0)
    np.testing.assert_array_equal(o, np.broadcast_to(v[0], o.shape))


def test_two_keys_with_logit_gap_ln3_weigh_quarter_and_three_quarters():
    D = 4
    q = np.zeros((1, D)); q[0, 0] = 1.0
    k = np.zeros((2, D)); k[1, 0] = 1.0          # s = scale * [0, 1]
    v = np.array([[1.0, -2.0, 8.0, 0.5], [5.0, 2.0, 0.0, -0.5]])
    o = _run(q, k, v, math.log(3.0))
    np.testing.assert_allclose(o[0], (v[0] + 3.0 * v[1]) / 4.0, rtol=0, atol=1e-15)
    # V is used as given, not transposed: swapping the keys swaps the weights
    o2 = _run(q, k[::-1].copy(), v, math.log(3.0))
    np.testing.assert_allclose(o2[0], (3.0 * v[0] + v[1]) / 4.0, rtol=0, atol=1e-15)


def test_dominant_logit_returns_its_row_without_overflow():
    rng = np.random.default_rng(3)
    N, D = 50, 16
    k = _f16(rng.standard_normal((N, D)) * 0.1).astype(np.float64)
    k[17] = 1.0                                   # q . k_17 = 16, the others are far smaller
    v = _f16(rng.standard_normal((N, D))).astype(np.float64)
    q = np.ones((1, D))
    o = _run(q, k, v, 200.0)                      # logits near 3200: exp overflows without the max shift
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o[0], v[17], rtol=0, atol=1e-12)


def test_constant_added_to_every_key_changes_nothing():
    rng = np.random.default_rng(4)
    N, D = 40, 32
    k = rng.integers(-4, 5, (N, D)).astype(np.float64)
    c = rng.integers(-3, 4, (1, D)).astype(np.float64)
    v = _f16(rng.standard_normal((N, D))).astype(np.float64)
    q = rng.integers(-2, 3, (6, D)).astype(np.float64)
    a = _run(q, k, v, 0.0625)
    b = _run(q, k + c, v, 0.0625)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_permuting_keys_with_values_changes_nothing():
    rng = np.random.default_rng(5)
    N, D = 33, 16
    k = _f16(rng.standard_normal((N, D))).astype(np.float64)
    v = _f16(rng.standard_normal((N, D))).astype(np.float64)
    q = _f16(rng.standard_normal((5, D))).astype(np.float64)
    p = rng.permutation(N)
    np.testing.assert_allclose(_run(q, k, v, 0.3), _run(q, k[p], v[p], 0.3), rtol=0, atol=1e-14)


def test_linear_in_values_and_inside_their_hull():
    rng = np.random.default_rng(6)
    N, D = 45, 16
    k = _f16(rng.standard_normal((N, D))).astype(np.float64)
    q = _f16(rng.standard_normal((7, D))).astype(np.float64)
    v1 = rng.integers(-50, 51, (N, D)).astype(np.float64)
    v2 = rng.integers(-50, 51, (N, D)).astype(np.float64)
    o1, o2, o12 = _run(q, k, v1, 0.25), _run(q, k, v2, 0.25), _run(q, k, v1 + v2, 0.25)
    np.testing.assert_allclose(o12, o1 + o2, rtol=0, atol=1e-12)
    assert np.all(o1 >= v1.min(axis=0) - 1e-12) and np.all(o1 <= v1.max(axis=0) + 1e-12)
    # not a plain average: the weights depend on the logits
    assert np.abs(o1 - v1.mean(axis=0)).max() > 0.5


def test_random_against_library_softmax():
    rng = np.random.default_rng(7)
    N, D, M = 300, 128, 9
    k = _f16(rng.standard_normal((N, D))).astype(np.float64)
    v = _f16(rng.standard_normal((N, D))).astype(np.float64)
    q = _f16(rng.standard_normal((M, D))).astype(np.float64)
    scale = 1.0 / math.sqrt(D)
    want = scipy.special.softmax(scale * (q @ k.T), axis=1) @ v
    np.testing.assert_allclose(_run(q, k, v, scale), want, rtol=0, atol=1e-13)
    # a scale applied twice or not at all is far off
    assert np.abs(_run(q, k, v, scale * scale) - want).max() > 1e-3
    # selected rows only
    np.testing.assert_allclose(_run(q, k, v, scale, rows=[8, 0, 3]), want[[8, 0, 3]],
                               rtol=0, atol=1e-13)


def test_strided_storage_matches_packed():
    rng = np.random.default_rng(8)
    M, N, D = 6, 21, 16
    ldq, ldk, ldv = D + 8, D + 3, N + 5
    q = _f16(rng.standard_normal((M, D)))
    k = _f16(rng.standard_normal((N, D)))
    vt = _f16(rng.standard_normal((D, N)))
    qs = np.zeros((M, ldq), np.float16); qs[:, :D] = q
    ks = np.zeros((N, ldk), np.float16); ks[:, :D] = k
    vs = np.zeros((D, ldv), np.float16); vs[:, :N] = vt
    qs[:, D:] = 1e4; ks[:, D:] = -1e4; vs[:, N:] = 7e3      # padding must never be read
    rows = np.arange(M)
    a = oracle.attention_rows(q, k, vt, N, D, rows, 0.5)
    b = oracle.attention_rows(qs, ks, vs, N, D, rows, 0.5, ldq=ldq, ldk=ldk, ldv=ldv)
    np.testing.assert_array_equal(a, b)


def test_bad_arguments_raise():
    q = np.zeros((2, 8), np.float16)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, np.zeros((8, 2), np.float16), 2, 8, [2], 1.0)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, np.zeros((8, 1), np.float16), 2, 8, [0], 1.0)
