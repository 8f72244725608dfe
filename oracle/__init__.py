"""CPU oracle for the TN GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The product library (``dense_gemm_tn_amd``)
never imports it and shares no code with it: the arithmetic lives in
``oracle.c`` (plain C, binary64, k ascending), built with gcc into
``liboracle.so`` next to this file.

Definitions followed (page, section):
  * "hello-gpu, chapter 11 (GEMM-like)", section 11.1: C[m,n] = sum_k A[m,k] B[k,n]
    with the partial sum starting at zero and k ascending (Fig. 11.1); no scaling,
    transpose or addend.
  * "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we compute":
    A row-major M x K, B column-major (K contiguous per column), C column-major.
  * FP8 inputs carry per-tensor scales; the oracle applies scale_a * scale_b to
    the exact binary64 sum.
  * Other layouts (``gemm``, ``gemm_strided``): the same sum with A(m, k), B(k, n)
    and C(m, n) at arbitrary element strides -- the row-major storage and index
    table of section 11.1 of the hello-gpu chapter, and the BLAS-style 'T' / 'N'
    operand codes against a column-major C.
  * Attention (``attention_rows``): the hello-gpu chapter summary names joining the
    product with softmax as the next step, and the mlqm.cn TileLang attention page
    motivates fusing softmax with QK^T.  No page gives the formula, so the oracle is
    the textbook softmax attention O = softmax(scale * Q K^T) V, row by row, in
    binary64 (see oracle.c).

Every function here has at least one pin in ``tests/test_oracle_pins.py`` that
does not come from this code (the worked example of section 11.1, the rank-1
partial sums of section 11.2, closed forms, exact rational sums, and library
codecs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_F16 = 0
FMT_E4M3FN = 1
FMT_BF16 = 2

_ITEMSIZE = {FMT_F16: 2, FMT_BF16: 2, FMT_E4M3FN: 1}
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc into ``liboracle.so`` (no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        lib.oracle_decode.argtypes = [ctypes.c_int, vp, vp, i64]
        lib.oracle_encode.argtypes = [ctypes.c_int, vp, vp, i64]
        lib.oracle_gemm_tn.argtypes = [ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                       ctypes.c_double, ctypes.c_int]
        lib.oracle_gemm_tn_entries.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, vp, vp, i64,
                                               ctypes.c_double, vp]
        lib.oracle_attention_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp, i64,
                                              ctypes.c_double, vp, ctypes.c_int]
        lib.oracle_gemm_strided.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, i64, vp, i64,
                                            i64, i64, i64, i64, ctypes.c_double, ctypes.c_int]
        lib.oracle_gemm_strided_entries.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, i64,
                                                    i64, vp, vp, i64, ctypes.c_double, vp]
        for f in (lib.oracle_decode, lib.oracle_encode, lib.oracle_gemm_tn,
                  lib.oracle_gemm_tn_entries, lib.oracle_attention_rows,
                  lib.oracle_gemm_strided, lib.oracle_gemm_strided_entries):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _raw(arr: np.ndarray, fmt: int) -> np.ndarray:
    """View an array of element codes as contiguous raw storage for ``fmt``."""
    a = np.ascontiguousarray(arr)
    want = np.uint8 if _ITEMSIZE[fmt] == 1 else np.uint16
    if a.dtype == np.float16 and fmt == FMT_F16:
        return a.view(np.uint16)
    if a.dtype != want:
        raise TypeError("fmt %d expects %s codes, got %s" % (fmt, want, a.dtype))
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _default_threads() -> int:
    """Threads for the oracle's column ranges: the cores this process may run on,
    capped by OMP_NUM_THREADS when it is set (the host's share of a shared box)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def decode(codes: np.ndarray, fmt: int) -> np.ndarray:
    """Exact binary64 value of every element code."""
    raw = _raw(codes, fmt)
    out = np.empty(raw.shape, dtype=np.float64)
    rc = _load().oracle_decode(fmt, _ptr(raw), _ptr(out), raw.size)
    if rc:
        raise ValueError("oracle_decode: bad format %d" % fmt)
    return out


def encode(values: np.ndarray, fmt: int) -> np.ndarray:
    """Round binary64 values to ``fmt`` (nearest, ties to even); returns the codes."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8 if _ITEMSIZE[fmt] == 1 else np.uint16)
    rc = _load().oracle_encode(fmt, _ptr(v), _ptr(out), v.size)
    if rc:
        raise ValueError("oracle_encode: bad format %d" % fmt)
    return out


def gemm_tn(A: np.ndarray, B: np.ndarray, fmt: int, M: int, N: int, K: int,
            lda: int | None = None, ldb: int | None = None, scale: float = 1.0,
            nthreads: int | None = None) -> np.ndarray:
    """binary64 C (column-major, returned as an [N, M] array: row n is column n of C).

    A holds M rows of lda codes (row-major), B holds N columns of ldb codes
    (column-major, i.e. K contiguous per column), both flat or shaped.
    """
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ra = _raw(A, fmt).reshape(-1)
    rb = _raw(B, fmt).reshape(-1)
    if M and K and ra.size < (M - 1) * lda + K:
        raise ValueError("A is too small for M, K, lda")
    if N and K and rb.size < (N - 1) * ldb + K:
        raise ValueError("B is too small for N, K, ldb")
    C = np.zeros((N, M), dtype=np.float64)
    if nthreads is None:
        nthreads = _default_threads()
    rc = _load().oracle_gemm_tn(fmt, _ptr(ra), _ptr(rb), _ptr(C), M, N, K, lda, ldb, M,
                                float(scale), int(nthreads))
    if rc:
        raise RuntimeError("oracle_gemm_tn failed with %d" % rc)
    return C


def gemm_tn_entries(A: np.ndarray, B: np.ndarray, fmt: int, K: int, ms, ns,
                    lda: int | None = None, ldb: int | None = None,
                    scale: float = 1.0) -> np.ndarray:
    """binary64 values C[ms[i], ns[i]] of the same product, one by one."""
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ra = _raw(A, fmt).reshape(-1)
    rb = _raw(B, fmt).reshape(-1)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns differ in shape")
    if ms.size and (ms.min() < 0 or ns.min() < 0 or
                    (ms.max() * lda + K) > ra.size or (ns.max() * ldb + K) > rb.size):
        raise ValueError("entry index out of range")
    out = np.empty(ms.shape, dtype=np.float64)
    rc = _load().oracle_gemm_tn_entries(fmt, _ptr(ra), _ptr(rb), K, lda, ldb, _ptr(ms),
                                        _ptr(ns), ms.size, float(scale), _ptr(out))
    if rc:
        raise RuntimeError("oracle_gemm_tn_entries failed with %d" % rc)
    return out


def gemm_strided(A: np.ndarray, sam: int, sak: int, B: np.ndarray, sbk: int, sbn: int,
                 fmt: int, M: int, N: int, K: int, scm: int, scn: int, c_size: int,
                 scale: float = 1.0, nthreads: int | None = None) -> np.ndarray:
    """binary64 C(m, n) = scale * sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn], stored at
    C[m*scm + n*scn] of a flat array of c_size elements (other elements stay 0)."""
    ra = _raw(A, fmt).reshape(-1)
    rb = _raw(B, fmt).reshape(-1)
    if M and K and ra.size <= (M - 1) * sam + (K - 1) * sak:
        raise ValueError("A is too small for its strides")
    if N and K and rb.size <= (K - 1) * sbk + (N - 1) * sbn:
        raise ValueError("B is too small for its strides")
    if M and N and c_size <= (M - 1) * scm + (N - 1) * scn:
        raise ValueError("C is too small for its strides")
    C = np.zeros(c_size, dtype=np.float64)
    if nthreads is None:
        nthreads = _default_threads()
    rc = _load().oracle_gemm_strided(fmt, _ptr(ra), sam, sak, _ptr(rb), sbk, sbn, _ptr(C), scm,
                                     scn, M, N, K, float(scale), int(nthreads))
    if rc:
        raise RuntimeError("oracle_gemm_strided failed with %d" % rc)
    return C


def _op_strides(trans_a: str, trans_b: str, lda: int, ldb: int):
    """Element strides of A(m, k) and B(k, n) for the BLAS-style op codes of a
    column-major C: trans_a 'T' = A[m*lda + k] (K contiguous), 'N' = A[m + k*lda];
    trans_b 'N' = B[k + n*ldb] (K contiguous), 'T' = B[k*ldb + n]."""
    if trans_a not in ("T", "N") or trans_b not in ("T", "N"):
        raise ValueError("trans codes are 'T' or 'N'")
    sam, sak = (lda, 1) if trans_a == "T" else (1, lda)
    sbk, sbn = (1, ldb) if trans_b == "N" else (ldb, 1)
    return sam, sak, sbk, sbn


def gemm(A: np.ndarray, B: np.ndarray, fmt: int, M: int, N: int, K: int,
         trans_a: str = "T", trans_b: str = "N", lda: int | None = None,
         ldb: int | None = None, scale: float = 1.0, nthreads: int | None = None) -> np.ndarray:
    """binary64 C = op(A) op(B) for any of the four layouts, returned as [N, M] (row n is
    column n of the column-major C).  Default leading dimensions are the packed ones."""
    if lda is None:
        lda = K if trans_a == "T" else M
    if ldb is None:
        ldb = K if trans_b == "N" else N
    sam, sak, sbk, sbn = _op_strides(trans_a, trans_b, lda, ldb)
    return gemm_strided(A, sam, sak, B, sbk, sbn, fmt, M, N, K, 1, M, M * N, scale,
                        nthreads).reshape(N, M)


def gemm_entries(A: np.ndarray, B: np.ndarray, fmt: int, K: int, ms, ns, M: int, N: int,
                 trans_a: str = "T", trans_b: str = "N", lda: int | None = None,
                 ldb: int | None = None, scale: float = 1.0) -> np.ndarray:
    """binary64 entries C[ms[i], ns[i]] of gemm(...), one by one."""
    if lda is None:
        lda = K if trans_a == "T" else M
    if ldb is None:
        ldb = K if trans_b == "N" else N
    sam, sak, sbk, sbn = _op_strides(trans_a, trans_b, lda, ldb)
    ra = _raw(A, fmt).reshape(-1)
    rb = _raw(B, fmt).reshape(-1)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns differ in shape")
    if ms.size and (ms.min() < 0 or ns.min() < 0 or ms.max() >= M or ns.max() >= N):
        raise ValueError("entry index out of range")
    out = np.empty(ms.shape, dtype=np.float64)
    rc = _load().oracle_gemm_strided_entries(fmt, _ptr(ra), sam, sak, _ptr(rb), sbk, sbn, K,
                                             _ptr(ms), _ptr(ns), ms.size, float(scale),
                                             _ptr(out))
    if rc:
        raise RuntimeError("oracle_gemm_strided_entries failed with %d" % rc)
    return out


def batched_qkt(Q: np.ndarray, Kmat: np.ndarray, batch: int, M: int, N: int, D: int,
                nthreads: int | None = None) -> np.ndarray:
    """binary64 S_h = Q_h K_h^T per head, returned as [batch, N, M] (column-major S_h).

    Q is [batch, M, D] and Kmat is [batch, N, D] fp16 (packed); K_h row-major N x D is
    the K-contiguous B of the TN product, so S_h(i, j) = sum_d Q_h[i, d] K_h[j, d].
    Source: the QK^T sketch on the mlqm.cn TileLang attention page (K = head dim).
    """
    q = np.ascontiguousarray(Q).reshape(batch, M * D)
    k = np.ascontiguousarray(Kmat).reshape(batch, N * D)
    out = np.empty((batch, N, M), dtype=np.float64)
    for h in range(batch):
        out[h] = gemm_tn(q[h], k[h], FMT_F16, M, N, D, nthreads=nthreads)
    return out


def attention_rows(Q: np.ndarray, Kmat: np.ndarray, Vt: np.ndarray, N: int, D: int, rows,
                   scale: float, ldq: int | None = None, ldk: int | None = None,
                   ldv: int | None = None, nthreads: int | None = None) -> np.ndarray:
    """binary64 softmax attention of query rows `rows` of one head, shape [len(rows), D].

    Q holds query rows of ldq fp16 codes, Kmat key rows of ldk codes, Vt holds V
    column-major (D rows of ldv codes, row d = V[:, d]).  Definition in oracle.c.
    """
    ldq = D if ldq is None else ldq
    ldk = D if ldk is None else ldk
    ldv = N if ldv is None else ldv
    rq = _raw(Q, FMT_F16).reshape(-1)
    rk = _raw(Kmat, FMT_F16).reshape(-1)
    rv = _raw(Vt, FMT_F16).reshape(-1)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() * ldq + D > rq.size):
        raise ValueError("query row out of range")
    if (N - 1) * ldk + D > rk.size or (D - 1) * ldv + N > rv.size:
        raise ValueError("K or Vt too small")
    out = np.empty((rows.size, D), dtype=np.float64)
    if nthreads is None:
        nthreads = _default_threads()
    rc = _load().oracle_attention_rows(_ptr(rq), _ptr(rk), _ptr(rv), N, D, ldq, ldk, ldv,
                                       _ptr(rows), rows.size, float(scale), _ptr(out),
                                       int(nthreads))
    if rc:
        raise RuntimeError("oracle_attention_rows failed with %d" % rc)
    return out
