"""Python binding of libdense_gemm_tn.so (gfx950 TN GEMM and fused attention).

Argument marshalling only: every step runs in the HIP kernels of
``csrc/gemm_tn.hip`` and ``csrc/attention.hip`` behind the C ABI declared in
``include/dense_gemm_tn.h``.  PyTorch supplies device memory and the current HIP
stream.  If the library has not been built, every call raises -- there is no other code path.

Layouts (TN, "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we
compute"): A is row-major M x K (a [M, lda] tensor), B is column-major K x N,
i.e. a [N, ldb] tensor whose row n is column n of B, and C is column-major
M x N, i.e. a [N, ldc] tensor whose row n is column n of C.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdense_gemm_tn.so")

DG_OK = 0
DG_ERR_INVALID_ARGUMENT = 1
DG_ERR_UNSUPPORTED = 2
DG_ERR_HIP = 3

EXPORTS = (
    "gemm_f16_tn",
    "gemm_f16",
    "gemm_f8_tn",
    "gemm_batched_qkt",
    "attention_fwd_f16",
    "gemm_status_string",
    "gemm_tile_order",
    "gemm_block_tile",
    "gemm_tn_config",
    "gemm_mid_stages",
    "gemm_f16_config",
    "gemm_f8",
    "gemm_f8_config",
    "gemm_f16_tn_splitk",
    "gemm_f8_tn_splitk",
    "gemm_splitk_workspace_bytes",
    "gemm_splitk_choose",
    "gemm_clock_record",
    "gemm_clock_records_used",
    "gemm_f16_tn_splitk_noalloc",
    "gemm_f16_tn_ws",
    "gemm_f8_tn_ws",
    "gemm_tn_workspace_bytes",
    "gemm_tn_plan",
)

_lib = None


class GemmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libdense_gemm_tn.so is not built; run `python -m dense_gemm_tn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.gemm_f16_tn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
        L.gemm_f16.argtypes = [ctypes.c_char, ctypes.c_char, vp, vp, vp, i64, i64, i64, i64, i64,
                               i64, vp]
        L.gemm_f8_tn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32, vp]
        L.gemm_batched_qkt.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                       i64, vp]
        L.attention_fwd_f16.argtypes = [vp, vp, vp, vp] + [i64] * 12 + [f32, vp]
        L.gemm_status_string.argtypes = [ctypes.c_int]
        L.gemm_status_string.restype = ctypes.c_char_p
        L.gemm_tile_order.argtypes = [i64, i64, i64, vp]
        L.gemm_block_tile.argtypes = []
        L.gemm_tn_config.argtypes = [ctypes.c_int, i64, i64, i64, i64]
        L.gemm_mid_stages.argtypes = [i64, i64]
        L.gemm_f16_config.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64]
        L.gemm_f8.argtypes = [ctypes.c_char, ctypes.c_char, vp, vp, vp, i64, i64, i64, i64, i64,
                              i64, f32, f32, vp]
        L.gemm_f8_config.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64]
        L.gemm_f16_tn_splitk.argtypes = [vp, vp, vp] + [i64] * 7 + [vp, i64, vp]
        L.gemm_f8_tn_splitk.argtypes = [vp, vp, vp] + [i64] * 6 + [f32, f32, i64, vp, i64, vp]
        L.gemm_splitk_workspace_bytes.argtypes = [i64, i64, i64]
        L.gemm_splitk_workspace_bytes.restype = i64
        L.gemm_splitk_choose.argtypes = [ctypes.c_int, i64, i64, i64]
        L.gemm_splitk_choose.restype = i64
        L.gemm_clock_record.argtypes = [vp, i64]
        L.gemm_clock_record.restype = ctypes.c_int
        L.gemm_clock_records_used.argtypes = []
        L.gemm_clock_records_used.restype = i64
        L.gemm_f16_tn_splitk_noalloc.argtypes = [vp, vp, vp] + [i64] * 7 + [vp]
        L.gemm_f16_tn_splitk_noalloc.restype = ctypes.c_int
        L.gemm_f16_tn_ws.argtypes = [vp, vp, vp] + [i64] * 6 + [vp, i64, vp]
        L.gemm_f8_tn_ws.argtypes = [vp, vp, vp] + [i64] * 6 + [f32, f32, vp, i64, vp]
        L.gemm_tn_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64]
        L.gemm_tn_workspace_bytes.restype = i64
        L.gemm_tn_plan.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, vp]
        for f in (L.gemm_f16_tn, L.gemm_f16, L.gemm_f8_tn, L.gemm_batched_qkt, L.attention_fwd_f16,
                  L.gemm_tile_order, L.gemm_block_tile, L.gemm_tn_config, L.gemm_mid_stages,
                  L.gemm_f16_config,
                  L.gemm_f8, L.gemm_f8_config, L.gemm_f16_tn_splitk, L.gemm_f8_tn_splitk,
                  L.gemm_f16_tn_ws, L.gemm_f8_tn_ws, L.gemm_tn_plan):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gemm_status_string(int(status)).decode()


def _ptr(x) -> int | None:
    """Device address of a tensor, or an integer address passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != DG_OK:
        raise GemmError(fn, status)


def gemm_f16_tn(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                stream=None) -> None:
    """C[m + n*ldc] = sum_k A[m*lda + k] * B[n*ldb + k]   (fp16 in/out, fp32 accumulate)."""
    _check("gemm_f16_tn", lib().gemm_f16_tn(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                            _stream(stream)))


def gemm_f16(transa: str, transb: str, A, B, C, M: int, N: int, K: int, lda: int, ldb: int,
             ldc: int, stream=None) -> None:
    """C[m + n*ldc] = sum_k op(A)(m, k) op(B)(k, n) for BLAS op codes 'T' / 'N':
    A 'T' = A[m*lda + k], 'N' = A[m + k*lda]; B 'N' = B[k + n*ldb], 'T' = B[k*ldb + n]."""
    if transa not in "TtNn" or transb not in "TtNn" or len(transa) != 1 or len(transb) != 1:
        raise ValueError("op codes are 'T' or 'N'")
    _check("gemm_f16", lib().gemm_f16(transa.encode(), transb.encode(), _ptr(A), _ptr(B), _ptr(C),
                                      M, N, K, lda, ldb, ldc, _stream(stream)))


def gemm_f8(transa: str, transb: str, A, B, C, M: int, N: int, K: int, lda: int, ldb: int,
            ldc: int, scale_a: float, scale_b: float, stream=None) -> None:
    """bf16 C = fp32(scale_a*scale_b) * op(A) op(B) with E4M3FN A, B in any op-code layout
    (the index conventions of gemm_f16)."""
    if transa not in "TtNn" or transb not in "TtNn" or len(transa) != 1 or len(transb) != 1:
        raise ValueError("op codes are 'T' or 'N'")
    _check("gemm_f8", lib().gemm_f8(transa.encode(), transb.encode(), _ptr(A), _ptr(B), _ptr(C),
                                    M, N, K, lda, ldb, ldc, float(scale_a), float(scale_b),
                                    _stream(stream)))


def gemm_f8_tn(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
               scale_a: float, scale_b: float, stream=None) -> None:
    """C = bf16(fp32(scale_a*scale_b) * A x B) with E4M3FN A, B and fp32 accumulation."""
    _check("gemm_f8_tn", lib().gemm_f8_tn(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                          float(scale_a), float(scale_b), _stream(stream)))


CLOCK_RECORD_WORDS = 10  # uint64 words per block record (see gemm_clock_record)


def clock_record(buf, records: int) -> None:
    """Start per-block clock records into a device buffer of `records` records
    (a 64-bit tensor of 10 * records elements); clock_record(None, 0) stops."""
    _check("gemm_clock_record", lib().gemm_clock_record(_ptr(buf), records))


def clock_records_used() -> int:
    return int(lib().gemm_clock_records_used())


def splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    """Bytes of workspace the split-K calls need (-1 for invalid arguments)."""
    return int(lib().gemm_splitk_workspace_bytes(M, N, splits))


def splitk_choose(M: int, N: int, K: int, fp8: bool = False) -> int:
    """The library's suggested split count for an M x N x K TN product."""
    return int(lib().gemm_splitk_choose(1 if fp8 else 0, M, N, K))


def gemm_f16_tn_splitk(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                       splits: int, workspace, workspace_bytes: int, stream=None) -> None:
    """gemm_f16_tn with K cut into up to `splits` ranges summed through an fp32 workspace."""
    _check("gemm_f16_tn_splitk",
           lib().gemm_f16_tn_splitk(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc, splits,
                                    _ptr(workspace), workspace_bytes, _stream(stream)))


def gemm_f16_tn_ws(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int, workspace,
                   workspace_bytes: int, stream=None) -> None:
    """gemm_f16_tn by the library's plan within `workspace_bytes` of `workspace` (None, 0: none)."""
    _check("gemm_f16_tn_ws",
           lib().gemm_f16_tn_ws(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                _ptr(workspace), workspace_bytes, _stream(stream)))


def gemm_f8_tn_ws(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                  scale_a: float, scale_b: float, workspace, workspace_bytes: int,
                  stream=None) -> None:
    """gemm_f8_tn by the library's plan within `workspace_bytes` of `workspace`."""
    _check("gemm_f8_tn_ws",
           lib().gemm_f8_tn_ws(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc, scale_a,
                               scale_b, _ptr(workspace), workspace_bytes, _stream(stream)))


def tn_workspace_bytes(M: int, N: int, K: int, fp8: bool = False) -> int:
    """Workspace bytes the best plan for an M x N x K TN product uses (0: none)."""
    return int(lib().gemm_tn_workspace_bytes(1 if fp8 else 0, M, N, K))


def tn_plan(M: int, N: int, K: int, batch: int = 1, workspace_bytes: int = 0,
            fp8: bool = False) -> dict:
    """The library's plan: single-launch configuration, columns run in whole
    rounds first (dp_cols, 0: none) and their configuration, K ranges of the
    rest (splits) and workspace bytes used."""
    out = (ctypes.c_int64 * 5)()
    _check("gemm_tn_plan", lib().gemm_tn_plan(1 if fp8 else 0, M, N, K, batch, workspace_bytes,
                                              ctypes.addressof(out)))
    return {"config": out[0], "dp_cols": out[1], "dp_config": out[2], "splits": out[3],
            "workspace_bytes": out[4]}


def gemm_f16_tn_splitk_noalloc(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                               splits: int, stream=None) -> None:
    """gemm_f16_tn_splitk with the partials in the library's static 32 MiB device array."""
    _check("gemm_f16_tn_splitk_noalloc",
           lib().gemm_f16_tn_splitk_noalloc(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                            splits, _stream(stream)))


def gemm_f8_tn_splitk(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                      scale_a: float, scale_b: float, splits: int, workspace,
                      workspace_bytes: int, stream=None) -> None:
    """gemm_f8_tn with K cut into up to `splits` ranges summed through an fp32 workspace."""
    _check("gemm_f8_tn_splitk",
           lib().gemm_f8_tn_splitk(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                   float(scale_a), float(scale_b), splits, _ptr(workspace),
                                   workspace_bytes, _stream(stream)))


def gemm_batched_qkt(Q, Kmat, S, batch: int, M: int, N: int, D: int, ldq: int, ldk: int,
                     lds: int, stride_q: int, stride_k: int, stride_s: int,
                     stream=None) -> None:
    """S_h[i + j*lds] = sum_d Q_h[i*ldq + d] * K_h[j*ldk + d] for every head h."""
    _check("gemm_batched_qkt",
           lib().gemm_batched_qkt(_ptr(Q), _ptr(Kmat), _ptr(S), batch, M, N, D, ldq, ldk, lds,
                                  stride_q, stride_k, stride_s, _stream(stream)))


def attention_fwd_f16(Q, Kmat, Vt, O, batch: int, M: int, N: int, D: int, ldq: int, ldk: int,
                      ldv: int, ldo: int, stride_q: int, stride_k: int, stride_v: int,
                      stride_o: int, scale: float, stream=None) -> None:
    """O_h = softmax(scale * Q_h K_h^T) V_h with V_h passed as Vt_h (D x N, keys contiguous)."""
    _check("attention_fwd_f16",
           lib().attention_fwd_f16(_ptr(Q), _ptr(Kmat), _ptr(Vt), _ptr(O), batch, M, N, D, ldq,
                                   ldk, ldv, ldo, stride_q, stride_k, stride_v, stride_o,
                                   float(scale), _stream(stream)))


def tile_order(tiles_m: int, tiles_n: int, batch: int = 1):
    """(head, tile_m, tile_n) for every hardware block id, as a [G, 3] int64 numpy array."""
    import numpy as np

    out = np.empty((tiles_m * tiles_n * batch, 3), dtype=np.int64)
    _check("gemm_tile_order", lib().gemm_tile_order(tiles_m, tiles_n, batch, out.ctypes.data))
    return out


def block_tile() -> int:
    return lib().gemm_block_tile()


CONFIG_NAMES = {0: "256x256", 1: "256x224", 2: "128x128", 3: "skinny-K",
                4: "256x256 8-wave ping-pong"}


def mid_stages(blocks: int, ksteps: int) -> int:
    """LDS stages of the 128 x 128 kernel's ring for a grid (see gemm_mid_stages)."""
    return lib().gemm_mid_stages(blocks, ksteps)


def tn_config(M: int, N: int, K: int, batch: int = 1, fp8: bool = False) -> int:
    """Kernel configuration code the GEMM entry points choose (see gemm_tn_config)."""
    return lib().gemm_tn_config(1 if fp8 else 0, M, N, K, batch)


def f16_config(transa: str, transb: str, M: int, N: int, K: int) -> int:
    """Kernel configuration gemm_f16 chooses for a layout (see gemm_f16_config)."""
    return lib().gemm_f16_config(transa.encode(), transb.encode(), M, N, K)


def f8_config(transa: str, transb: str, M: int, N: int, K: int) -> int:
    """Kernel configuration gemm_f8 chooses for a layout (see gemm_f8_config)."""
    return lib().gemm_f8_config(transa.encode(), transb.encode(), M, N, K)


# ----------------------------------------------------------- tensor helpers
#
# The helpers check what the C ABI cannot see from raw pointers -- that every
# tensor lives on one GPU, that rows are contiguous, and that a caller's `out`
# has the shape, dtype and strides the product writes -- and raise ValueError
# before any launch.

def _check_tensors(fn: str, *ts) -> None:
    """Every tensor is a CUDA (HIP) tensor on one device with a contiguous last dimension."""
    for t in ts:
        if t.dim() == 0 or t.stride(-1) != 1:
            raise ValueError("%s: the last dimension must be contiguous" % fn)
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("%s: tensors must be on a GPU (got %s)" % (fn, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s: tensors on different devices (%s, %s)" % (fn, dev, t.device))


def _check_out(fn: str, out, shape, dtypes) -> None:
    if tuple(out.shape) != tuple(shape):
        raise ValueError("%s: out must have shape %s, got %s" % (fn, tuple(shape),
                                                                 tuple(out.shape)))
    if out.dtype not in dtypes:
        raise ValueError("%s: out dtype %s is not one of %s" % (fn, out.dtype, dtypes))
    if out.stride(-1) != 1:
        raise ValueError("%s: out's last dimension must be contiguous" % fn)
    for d in range(out.dim() - 1):
        if out.stride(d) < out.shape[d + 1] * out.stride(d + 1) and out.shape[d] > 1:
            raise ValueError("%s: out's rows overlap (stride %d)" % (fn, out.stride(d)))


def _empty_on(stream, shape, dtype, device):
    """A new tensor allocated on `stream` (or the current stream): the caching
    allocator then orders its reuse after the work queued on that stream."""
    import torch

    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def matmul_tn_f16(a, b, out=None, stream=None, splits=1):
    """a: [M, K] fp16 (row-major A), b: [N, K] fp16 (column-major B) -> C as [N, M] fp16.

    splits > 1 runs the split-K call with that many K ranges; "auto" runs the
    library's plan with the workspace it asks for (gemm_f16_tn_ws: split-K,
    a split tail of a ragged last round, or a single launch).  Workspaces are
    allocated on the launch stream (so the caching allocator hands them out
    only after earlier work on that stream).  A new `out` is allocated on the
    launch stream too; a caller's `out` must be [N, M] fp16 with contiguous
    rows."""
    import torch

    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("matmul_tn_f16 expects 2-D tensors")
    M, K = a.shape
    N, Kb = b.shape
    if K != Kb or a.dtype != torch.float16 or b.dtype != torch.float16:
        raise ValueError("matmul_tn_f16 expects fp16 [M, K] and [N, K]")
    if out is not None:
        _check_out("matmul_tn_f16", out, (N, M), (torch.float16,))
    _check_tensors("matmul_tn_f16", a, b, *(() if out is None else (out,)))
    if stream is not None and not isinstance(stream, torch.cuda.Stream):
        if splits != 1 or out is None:
            raise ValueError("matmul_tn_f16: pass a torch.cuda.Stream (or None) when the "
                             "helper allocates")
    if out is None:
        out = _empty_on(stream, (N, M), torch.float16, a.device)
    if splits == "auto":
        nbytes = tn_workspace_bytes(M, N, K)
        ws = _empty_on(stream, (max(nbytes, 16) // 4,), torch.float32, a.device) if nbytes else None
        gemm_f16_tn_ws(a, b, out, M, N, K, a.stride(0), b.stride(0), out.stride(0), ws, nbytes,
                       stream)
        return out
    if splits == 1:
        gemm_f16_tn(a, b, out, M, N, K, a.stride(0), b.stride(0), out.stride(0), stream)
        return out
    nbytes = splitk_workspace_bytes(M, N, int(splits))
    if nbytes < 0:
        raise ValueError("splits must be 1 .. 64 or 'auto'")
    ws = _empty_on(stream, (max(nbytes, 16) // 4,), torch.float32, a.device)
    gemm_f16_tn_splitk(a, b, out, M, N, K, a.stride(0), b.stride(0), out.stride(0), int(splits),
                       ws, nbytes, stream)
    return out


def matmul_f16(a, b, transa: str = "T", transb: str = "N", out=None, stream=None):
    """fp16 C = op(A) op(B) as [N, M] (column-major C) from operands as they lie in memory:
    a is [M, K] for transa 'T' and [K, M] for 'N'; b is [N, K] for transb 'N' and
    [K, N] for 'T' (each with a contiguous last dimension)."""
    import torch

    if a.dtype != torch.float16 or b.dtype != torch.float16 or a.dim() != 2 or b.dim() != 2:
        raise ValueError("matmul_f16 expects 2-D fp16 tensors")
    if transa not in ("T", "t", "N", "n") or transb not in ("T", "t", "N", "n"):
        raise ValueError("op codes are 'T' or 'N'")
    M, K = a.shape if transa in "Tt" else a.shape[::-1]
    N, Kb = b.shape if transb in "Nn" else b.shape[::-1]
    if K != Kb:
        raise ValueError("matmul_f16: K differs")
    if out is not None:
        _check_out("matmul_f16", out, (N, M), (torch.float16,))
    _check_tensors("matmul_f16", a, b, *(() if out is None else (out,)))
    if out is None:
        out = _empty_on(stream if isinstance(stream, torch.cuda.Stream) else None, (N, M),
                        torch.float16, a.device)
    gemm_f16(transa, transb, a, b, out, M, N, K, a.stride(0), b.stride(0), out.stride(0), stream)
    return out


def matmul_tn_f8(a, b, scale_a: float, scale_b: float, out=None, stream=None):
    """a: [M, K] uint8 E4M3FN codes, b: [N, K] codes -> C as [N, M] bf16."""
    import torch

    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("matmul_tn_f8 expects 2-D tensors")
    M, K = a.shape
    N, Kb = b.shape
    if K != Kb or a.element_size() != 1 or b.element_size() != 1:
        raise ValueError("matmul_tn_f8 expects 1-byte [M, K] and [N, K]")
    if out is not None:
        _check_out("matmul_tn_f8", out, (N, M), (torch.bfloat16,))
    _check_tensors("matmul_tn_f8", a, b, *(() if out is None else (out,)))
    if out is None:
        out = _empty_on(stream if isinstance(stream, torch.cuda.Stream) else None, (N, M),
                        torch.bfloat16, a.device)
    gemm_f8_tn(a, b, out, M, N, K, a.stride(0), b.stride(0), out.stride(0), scale_a, scale_b,
               stream)
    return out


def qkt(q, k, out=None, stream=None):
    """q: [H, M, D], k: [H, N, D] fp16 -> S as [H, N, M] fp16 (S_h column-major)."""
    import torch

    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("qkt expects [H, M, D] and [H, N, D]")
    H, M, D = q.shape
    Hk, N, Dk = k.shape
    if H != Hk or D != Dk or q.dtype != torch.float16 or k.dtype != torch.float16:
        raise ValueError("qkt expects fp16 [H, M, D] and [H, N, D]")
    if out is not None:
        _check_out("qkt", out, (H, N, M), (torch.float16,))
    _check_tensors("qkt", q, k, *(() if out is None else (out,)))
    if out is None:
        out = _empty_on(stream if isinstance(stream, torch.cuda.Stream) else None, (H, N, M),
                        torch.float16, q.device)
    gemm_batched_qkt(q, k, out, H, M, N, D, q.stride(1), k.stride(1), out.stride(1),
                     q.stride(0), k.stride(0), out.stride(0), stream)
    return out


def attention(q, k, vt, scale: float | None = None, out=None, stream=None):
    """q: [H, M, D], k: [H, N, D], vt: [H, D, N] fp16 -> O as [H, M, D] fp16.

    scale defaults to 1/sqrt(D).  Row strides are taken from the tensors (the last
    dimension must be contiguous, and every row stride a multiple of 8 elements:
    for N % 8 != 0 pass a slice of a [H, D, N rounded up to 8] buffer as vt).
    """
    import math

    import torch

    if q.dim() != 3 or k.dim() != 3 or vt.dim() != 3:
        raise ValueError("attention expects [H, M, D], [H, N, D] and [H, D, N]")
    H, M, D = q.shape
    Hk, N, Dk = k.shape
    Hv, Dv, Nv = vt.shape
    if (H, D) != (Hk, Dk) or (H, D, N) != (Hv, Dv, Nv):
        raise ValueError("attention expects [H, M, D], [H, N, D] and [H, D, N]")
    if any(t.dtype != torch.float16 for t in (q, k, vt)):
        raise ValueError("attention expects fp16 tensors")
    if out is not None:
        _check_out("attention", out, (H, M, D), (torch.float16,))
    _check_tensors("attention", q, k, vt, *(() if out is None else (out,)))
    if out is None:
        out = _empty_on(stream if isinstance(stream, torch.cuda.Stream) else None, (H, M, D),
                        torch.float16, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    attention_fwd_f16(q, k, vt, out, H, M, N, D, q.stride(1), k.stride(1), vt.stride(1),
                      out.stride(1), q.stride(0), k.stride(0), vt.stride(0), out.stride(0),
                      scale, stream)
    return out
