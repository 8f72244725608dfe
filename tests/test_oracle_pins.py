"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names the page passage or the mathematical fact it pins:
  * the worked 2x3 by 3x2 example (hello-gpu chapter 11, section 11.1) and its
    partial sums along K (Fig. 11.1; the rank-1 view of section 11.2);
  * closed forms (all-ones => C = K), identity special cases (transposed copy);
  * +-1 inputs against an exact integer matmul (a library routine on integers);
  * random inputs against exact rational sums (fractions.Fraction) within the
    recursive-summation error bound of binary64;
  * the codecs against the library casts of numpy and PyTorch, over every code.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_tn_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_gemm_like_11_1.json")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _tn_storage(A_rows, B_rows):
    """A row-major M x K, B column-major (rows of the returned array are columns of B)."""
    A = np.asarray(A_rows, dtype=np.float64)
    B = np.asarray(B_rows, dtype=np.float64)
    return A, np.ascontiguousarray(B.T)


# --------------------------------------------------------------- worked example

def test_worked_example_fp16_and_fp8():
    g = json.load(open(GOLDEN))
    A, Bt = _tn_storage(g["A_rows"], g["B_rows"])
    M, N, K = g["M"], g["N"], g["K"]
    want = np.asarray(g["C_rows"], dtype=np.float64)           # [M, N]
    for fmt in (oracle.FMT_F16, oracle.FMT_E4M3FN, oracle.FMT_BF16):
        a = oracle.encode(A, fmt)
        b = oracle.encode(Bt, fmt)
        C = oracle.gemm_tn(a, b, fmt, M, N, K)                  # [N, M] = column-major C
        np.testing.assert_array_equal(C.T, want)
        # column-major storage order of C is [5, 14, 8, 17]
        assert list(C.reshape(-1)) == [5.0, 14.0, 8.0, 17.0]


def test_worked_example_partial_sums_along_k():
    """Truncating K to k+1 gives the partial sums printed for C[0,0] and C[1,1]
    (Fig. 11.1) and the whole partial matrices of the rank-1 view (section 11.2)."""
    g = json.load(open(GOLDEN))
    A, Bt = _tn_storage(g["A_rows"], g["B_rows"])
    a = oracle.encode(A, oracle.FMT_F16)
    b = oracle.encode(Bt, oracle.FMT_F16)
    for k in range(1, 4):
        # Keep the full row strides, only the summation length changes.
        C = oracle.gemm_tn(a, b, oracle.FMT_F16, 2, 2, k, lda=3, ldb=3).T
        assert C[0, 0] == g["partial_sums_C00"][k - 1]
        assert C[1, 1] == g["partial_sums_C11"][k - 1]
        np.testing.assert_array_equal(C, np.asarray(g["rank1_partial_matrices"][k - 1]))


def test_worked_example_entries_and_batched():
    g = json.load(open(GOLDEN))
    A, Bt = _tn_storage(g["A_rows"], g["B_rows"])
    a = oracle.encode(A, oracle.FMT_F16)
    b = oracle.encode(Bt, oracle.FMT_F16)
    e = oracle.gemm_tn_entries(a, b, oracle.FMT_F16, 3, [0, 1, 0, 1], [0, 0, 1, 1])
    assert list(e) == [5.0, 14.0, 8.0, 17.0]
    # Batched QK^T: Q_h = A, K_h = B^T (row j of K_h is column j of B); head 1 is
    # the same problem negated.
    Q = np.stack([a.view(np.float16), (-A).astype(np.float16)])
    Kh = np.stack([b.view(np.float16), Bt.astype(np.float16)])
    S = oracle.batched_qkt(Q, Kh, 2, 2, 2, 3)
    np.testing.assert_array_equal(S[0].T, np.asarray(g["C_rows"]))
    np.testing.assert_array_equal(S[1].T, -np.asarray(g["C_rows"]))


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("K", [1, 7, 64, 2048, 4096])
def test_all_ones_gives_K(K):
    M, N = 5, 3
    ones = np.ones((M, K), dtype=np.float16)
    C = oracle.gemm_tn(ones, np.ones((N, K), dtype=np.float16), oracle.FMT_F16, M, N, K)
    assert np.all(C == K)


@pytest.mark.parametrize("K", [16, 256, 8192])
def test_all_ones_fp8_with_amax_scale(K):
    """Ones quantised per tensor: s = fp32(1/448), code 448; C = K * (448 s)^2, which is
    K to within a few fp32 ulps and rounds to exactly K in bf16 (K a power of two)."""
    codes, s = inputs.quantise_e4m3fn(np.ones((4, K), dtype=np.float32))
    assert np.all(codes == 0x7E)
    C = oracle.gemm_tn(codes, codes[:3], oracle.FMT_E4M3FN, 4, 3, K, scale=s * s)
    exact = K * (448.0 * s) ** 2
    assert np.all(C == exact)
    assert abs(exact / K - 1) < 2 ** -20
    bf = oracle.encode(C, oracle.FMT_BF16)
    assert np.all(oracle.decode(bf, oracle.FMT_BF16) == K)


def test_identity_special_cases():
    """A = I gives C = B (column-major C holds the columns of B); B = I gives the
    transposed copy of A -- special cases of the section 11.1 definition."""
    rng = np.random.default_rng(3)
    n = 24
    I = np.eye(n, dtype=np.float16)
    B = rng.standard_normal((5, n)).astype(np.float16)      # 5 columns of length n
    C = oracle.gemm_tn(I, B, oracle.FMT_F16, n, 5, n)       # [5, n]
    np.testing.assert_array_equal(C, B.astype(np.float64))
    A = rng.standard_normal((7, n)).astype(np.float16)
    C = oracle.gemm_tn(A, I, oracle.FMT_F16, 7, n, n)       # [n, 7] = A^T
    np.testing.assert_array_equal(C, A.T.astype(np.float64))


def test_pm1_against_exact_integer_matmul():
    """+-1 inputs: every partial sum is an integer; the integer matmul of numpy is exact.
    Also checks the parity and range invariants (C = K mod 2, |C| <= K)."""
    M, N, K = 37, 29, 301
    x = inputs.make_shape("f16", M, N, K, dist="pm1", seed=5)
    C = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, M, N, K)
    ia = x["A"].astype(np.int64)
    ib = x["B"].astype(np.int64)
    np.testing.assert_array_equal(C, (ia @ ib.T).T.astype(np.float64))
    assert np.all(np.abs(C) <= K) and np.all((C - K) % 2 == 0)


def test_scale_is_applied_once():
    """FP8 with power-of-two scales: the result is the exact integer sum times sa*sb."""
    M, N, K = 9, 11, 96
    x = inputs.make_shape("f8", M, N, K, dist="pm1", seed=2)
    C1 = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_E4M3FN, M, N, K)
    Cs = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_E4M3FN, M, N, K, scale=0.25 * 8.0)
    ia = np.where(x["A"] == 0x38, 1, -1).astype(np.int64)
    ib = np.where(x["B"] == 0x38, 1, -1).astype(np.int64)
    np.testing.assert_array_equal(C1, (ia @ ib.T).T.astype(np.float64))
    np.testing.assert_array_equal(Cs, 2.0 * C1)


def test_random_against_exact_rationals():
    """binary64 sums of exact fp16 products stay within gamma_K * sum|a b| of the
    exact rational result (standard recursive-summation bound, u = 2^-53)."""
    M, N, K = 6, 5, 200
    x = inputs.make_shape("f16", M, N, K, dist="normal", seed=11)
    C = oracle.gemm_tn(x["A"], x["B"], oracle.FMT_F16, M, N, K)
    A = x["A"].astype(np.float64)
    B = x["B"].astype(np.float64)
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    for n in range(N):
        for m in range(M):
            exact = sum(Fraction(A[m, k]) * Fraction(B[n, k]) for k in range(K))
            bound = gamma * float(sum(abs(Fraction(A[m, k]) * Fraction(B[n, k])) for k in range(K)))
            assert abs(Fraction(C[n, m]) - exact) <= Fraction(bound)


def test_strided_operands_and_degenerate_sizes():
    rng = np.random.default_rng(4)
    M, N, K, lda, ldb = 4, 3, 5, 9, 7
    A = rng.standard_normal((M, lda)).astype(np.float16)
    B = rng.standard_normal((N, ldb)).astype(np.float16)
    C = oracle.gemm_tn(A, B, oracle.FMT_F16, M, N, K, lda=lda, ldb=ldb)
    want = A[:, :K].astype(np.float64) @ B[:, :K].astype(np.float64).T
    np.testing.assert_allclose(C, want.T, rtol=1e-13, atol=1e-13)
    Z = oracle.gemm_tn(A, B, oracle.FMT_F16, M, N, 0, lda=lda, ldb=ldb)
    assert Z.shape == (N, M) and np.all(Z == 0)
    assert oracle.gemm_tn(A, B, oracle.FMT_F16, 0, N, K, lda=lda, ldb=ldb).shape == (N, 0)


# --------------------------------------------------------------------- codecs

def test_f16_decode_all_codes_vs_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(codes, oracle.FMT_F16)
    want = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_f16_encode_vs_numpy_rounding():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = codes.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    assert np.array_equal(oracle.encode(vals[finite], oracle.FMT_F16), codes[finite])
    rng = np.random.default_rng(0)
    # random magnitudes across the whole range, including subnormals and overflow
    x = rng.standard_normal(200000) * np.exp2(rng.uniform(-30, 17, 200000))
    # exact midpoints between neighbouring fp16 values (ties)
    lo = codes[finite & (vals > 0)][:-1].view(np.float16).astype(np.float64)
    hi = (codes[finite & (vals > 0)][:-1] + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2, -(lo + hi) / 2])
    with np.errstate(over="ignore"):        # the overflow to infinity is part of the check
        want = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.encode(x, oracle.FMT_F16), want)


def test_bf16_codec_vs_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(codes, oracle.FMT_BF16)
    want = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    rng = np.random.default_rng(1)
    with np.errstate(over="ignore"):        # values past the fp32 range are dropped below
        x32 = (rng.standard_normal(200000) * np.exp2(rng.uniform(-130, 127, 200000))).astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.encode(x32.astype(np.float64), oracle.FMT_BF16), want)


def test_e4m3fn_codec_vs_torch():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = oracle.decode(codes, oracle.FMT_E4M3FN)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(want)
    assert int(nan.sum()) == 2  # S.1111.111 only
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    # encoder: every finite code round-trips, and random fp32 values round like torch
    fin = ~nan
    np.testing.assert_array_equal(oracle.encode(got[fin], oracle.FMT_E4M3FN), codes[fin])
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(100000) * np.exp2(rng.uniform(-12, 9, 100000))).astype(np.float32)
    x32 = np.clip(x32, -448, 448)
    want = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode(x32.astype(np.float64), oracle.FMT_E4M3FN), want)
    # saturation beyond the largest finite value
    assert list(oracle.encode(np.array([500.0, -1e9]), oracle.FMT_E4M3FN)) == [0x7E, 0xFE]


def test_input_quantiser_matches_oracle_codec():
    """The generator's library cast and the oracle's own encoder agree on every element."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 512), dtype=np.float32)
    codes, s = inputs.quantise_e4m3fn(x)
    y = np.clip(x / np.float32(s), -448, 448).astype(np.float32)
    np.testing.assert_array_equal(oracle.encode(y.astype(np.float64), oracle.FMT_E4M3FN), codes)
    assert np.max(np.abs(oracle.decode(codes, oracle.FMT_E4M3FN))) == 448.0
    assert s == np.float32(np.float32(np.max(np.abs(x))) / np.float32(448))


# ------------------------------------------------------ other storage layouts

def test_row_major_worked_example_and_index_table():
    """Section 11.1 stores A, B and C row-major (A[m*K + k], B[k*N + n], C[m*N + n])
    and states that C[1,1] reads A at 3, 4, 5 and B at 1, 3, 5 (B's row stride is N)."""
    g = json.load(open(GOLDEN))
    M, N, K = g["M"], g["N"], g["K"]
    A = np.asarray(g["A_rows"], dtype=np.float16).reshape(-1)
    B = np.asarray(g["B_rows"], dtype=np.float16).reshape(-1)
    C = oracle.gemm_strided(A, K, 1, B, N, 1, oracle.FMT_F16, M, N, K, N, 1, M * N)
    np.testing.assert_array_equal(C.reshape(M, N), np.asarray(g["C_rows"], dtype=np.float64))
    # Only the elements the page names are nonzero: C[1,1] keeps its value, the rest is 0.
    A2 = np.zeros_like(A)
    A2[[3, 4, 5]] = A[[3, 4, 5]]
    B2 = np.zeros_like(B)
    B2[[1, 3, 5]] = B[[1, 3, 5]]
    C2 = oracle.gemm_strided(A2, K, 1, B2, N, 1, oracle.FMT_F16, M, N, K, N, 1, M * N)
    np.testing.assert_array_equal(C2.reshape(M, N), [[0.0, 0.0], [0.0, 17.0]])


@pytest.mark.parametrize("trans_a", ["T", "N"])
@pytest.mark.parametrize("trans_b", ["T", "N"])
def test_four_layouts_against_integer_matmul(trans_a, trans_b):
    """Each of the four op-code layouts, with padded leading dimensions whose
    padding is poisoned, against numpy's exact integer matmul of +-1 data."""
    rng = np.random.default_rng(17)
    M, N, K = 23, 19, 37
    a = rng.choice([-1, 1], size=(M, K)).astype(np.int64)
    b = rng.choice([-1, 1], size=(K, N)).astype(np.int64)
    want = a @ b                                     # [M, N]
    pad = 5
    # A storage: 'T' = rows of K (A[m*lda + k]), 'N' = rows of M (A[m + k*lda]).
    sa = a if trans_a == "T" else a.T
    Astore = np.full((sa.shape[0], sa.shape[1] + pad), 1000.0, np.float16)
    Astore[:, :sa.shape[1]] = sa
    # B storage: 'N' = rows of K per column n (B[k + n*ldb]), 'T' = rows of N (B[k*ldb + n]).
    sb = b.T if trans_b == "N" else b
    Bstore = np.full((sb.shape[0], sb.shape[1] + pad), -1000.0, np.float16)
    Bstore[:, :sb.shape[1]] = sb
    C = oracle.gemm(Astore, Bstore, oracle.FMT_F16, M, N, K, trans_a=trans_a, trans_b=trans_b,
                    lda=Astore.shape[1], ldb=Bstore.shape[1])
    np.testing.assert_array_equal(C.T, want.astype(np.float64))
    ms = rng.integers(0, M, 40)
    ns = rng.integers(0, N, 40)
    e = oracle.gemm_entries(Astore, Bstore, oracle.FMT_F16, K, ms, ns, M, N, trans_a=trans_a,
                            trans_b=trans_b, lda=Astore.shape[1], ldb=Bstore.shape[1])
    np.testing.assert_array_equal(e, want[ms, ns].astype(np.float64))


# E4M3FN codes of small dyadic values, from the format's definition
# (sign bit 7, 4 exponent bits with bias 7, 3 mantissa bits: 2^(e-7) * (1 + m/8)).
E4M3_TABLE = {0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0xC0: -2.0, 0x30: 0.5, 0xB0: -0.5,
              0x3C: 1.5, 0xBC: -1.5}


@pytest.mark.parametrize("trans_a", ["T", "N"])
@pytest.mark.parametrize("trans_b", ["T", "N"])
def test_four_layouts_fp8_against_exact_matmul(trans_a, trans_b):
    """The FP8 path of the strided oracle in each op-code layout: E4M3FN codes of
    dyadic values (every product and partial sum exact in binary64), padding holding
    the E4M3FN NaN code, a power-of-two scale; numpy's float64 matmul of the values
    the codes stand for is exact here."""
    rng = np.random.default_rng(29)
    M, N, K = 21, 17, 45
    codes = np.array(sorted(E4M3_TABLE), dtype=np.uint8)
    ca = rng.choice(codes, size=(M, K))
    cb = rng.choice(codes, size=(K, N))
    va = np.vectorize(E4M3_TABLE.get)(ca).astype(np.float64)
    vb = np.vectorize(E4M3_TABLE.get)(cb).astype(np.float64)
    want = (va @ vb) * 0.25                          # [M, N]
    pad = 3
    sa = ca if trans_a == "T" else ca.T
    Astore = np.full((sa.shape[0], sa.shape[1] + pad), 0x7F, np.uint8)
    Astore[:, :sa.shape[1]] = sa
    sb = cb.T if trans_b == "N" else cb
    Bstore = np.full((sb.shape[0], sb.shape[1] + pad), 0x7F, np.uint8)
    Bstore[:, :sb.shape[1]] = sb
    C = oracle.gemm(Astore, Bstore, oracle.FMT_E4M3FN, M, N, K, trans_a=trans_a,
                    trans_b=trans_b, lda=Astore.shape[1], ldb=Bstore.shape[1], scale=0.25)
    np.testing.assert_array_equal(C.T, want)
    ms = rng.integers(0, M, 30)
    ns = rng.integers(0, N, 30)
    e = oracle.gemm_entries(Astore, Bstore, oracle.FMT_E4M3FN, K, ms, ns, M, N,
                            trans_a=trans_a, trans_b=trans_b, lda=Astore.shape[1],
                            ldb=Bstore.shape[1], scale=0.25)
    np.testing.assert_array_equal(e, want[ms, ns])
