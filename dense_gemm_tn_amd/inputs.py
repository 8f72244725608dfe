"""Seeded synthetic inputs for the TN GEMM and attention workloads.

This module only draws and encodes input elements (numpy PCG64 streams, the
fp16 cast, the per-tensor FP8 quantiser); it contains none of the GEMM's
arithmetic.  Both the GPU path and the CPU oracle receive exactly the bytes
made here.

Recipe (one numpy ``default_rng(seed)`` per workload, drawing A then B, Q then
K, or Q, K then Vt for attention):
  * "pm1"    elements uniform on {-1, +1} (the exact-comparison inputs of
             "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we
             compute": every product is +-1 and every partial sum an integer);
  * "normal" i.i.d. N(0, std^2) drawn in float32 and rounded to fp16 (nearest
             even);
  * FP8      i.i.d. N(0, 1) in float32, per-tensor scale s = fp32(amax) / 448,
             codes = E4M3FN(round-nearest-even(x / s)) clamped to +-448 (the
             largest finite E4M3FN value).  The library cast of PyTorch is used
             for the rounding; the oracle has its own codec to check it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "f16", "f8", "qkt" or "attn"
    M: int
    N: int
    K: int               # contraction length (head dim D for "qkt")
    dist: str            # "pm1" or "normal"
    seed: int = 0
    batch: int = 1
    std: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        """Algorithmic work: 2*M*N*K per head (section 11.1 of the hello-gpu chapter);
        attention does two such products per head (Q K^T and P V, K = head dim)."""
        products = 2 if self.kind == "attn" else 1
        return products * 2 * self.M * self.N * self.K * self.batch


# The five workloads (sizes and distributions as stated for this GEMM).
WORKLOADS = {
    w.name: w
    for w in (
        Workload("f16_256_pm1", "f16", 256, 256, 256, "pm1", seed=0),
        Workload("f16_4096", "f16", 4096, 4096, 4096, "normal", seed=0),
        Workload("f16_2048", "f16", 2048, 2048, 2048, "normal", seed=0),
        Workload("f16_1920x13900x4096", "f16", 1920, 13900, 4096, "normal", seed=0),
        Workload("f16_1920x13900x4096_pm1", "f16", 1920, 13900, 4096, "pm1", seed=1),
        Workload("f8_8192", "f8", 8192, 8192, 8192, "normal", seed=0),
        # The other op-code layouts (A 'T' = K-contiguous rows, 'N' = M-contiguous;
        # B 'N' = K-contiguous, 'T' = N-contiguous), same values as f16_4096 and
        # f8_8192.
        Workload("f16_nn_4096", "f16", 4096, 4096, 4096, "normal", seed=0,
                 extra={"layout": "NN"}),
        Workload("f16_tt_4096", "f16", 4096, 4096, 4096, "normal", seed=0,
                 extra={"layout": "TT"}),
        Workload("f16_nt_4096", "f16", 4096, 4096, 4096, "normal", seed=0,
                 extra={"layout": "NT"}),
        Workload("f8_nn_8192", "f8", 8192, 8192, 8192, "normal", seed=0,
                 extra={"layout": "NN"}),
        Workload("f8_tt_8192", "f8", 8192, 8192, 8192, "normal", seed=0,
                 extra={"layout": "TT"}),
        Workload("f8_nt_8192", "f8", 8192, 8192, 8192, "normal", seed=0,
                 extra={"layout": "NT"}),
        # Few output tiles, long K: 16 tiles of 128 x 128 over K = 32768, one
        # block per tile, and the same product split along K over a workspace.
        Workload("f16_512x512x32768", "f16", 512, 512, 32768, "normal", seed=0),
        Workload("f16_512x512x32768_splitk", "f16", 512, 512, 32768, "normal", seed=0,
                 extra={"splitk": True}),
        # The 8-wave ping-pong form of the 256 x 256 tile, forced (a measured
        # counter-design; the library never picks it by itself).
        Workload("f16_4096_pingpong", "f16", 4096, 4096, 4096, "normal", seed=0,
                 extra={"tile": "pingpong"}),
        Workload("f8_8192_pingpong", "f8", 8192, 8192, 8192, "normal", seed=0,
                 extra={"tile": "pingpong"}),
        # A ragged last round (288 tiles of 256 x 256 on 256 CUs): the library's
        # plan (whole rounds of columns, then the rest), the same product as a
        # single launch of the selector's configuration, and a plan whose tail
        # is split along K through a workspace.
        Workload("f16_4096x4608x4096", "f16", 4096, 4608, 4096, "normal", seed=0),
        Workload("f16_4096x4608x4096_single", "f16", 4096, 4608, 4096, "normal", seed=0,
                 extra={"tile": "128"}),
        Workload("f8_4096x4608x4096", "f8", 4096, 4608, 4096, "normal", seed=0),
        Workload("f8_4096x4608x4096_single", "f8", 4096, 4608, 4096, "normal", seed=0,
                 extra={"tile": "128"}),
        Workload("f16_4096x4352x4096_ws", "f16", 4096, 4352, 4096, "normal", seed=0,
                 extra={"ws": True}),
        Workload("f16_4096x4352x4096_single", "f16", 4096, 4352, 4096, "normal", seed=0,
                 extra={"tile": "128"}),
        Workload("qkt_64x4096x4096x128", "qkt", 4096, 4096, 128, "normal", seed=0, batch=64,
                 std=1.0 / math.sqrt(128.0)),
        Workload("attn_64x4096x4096x128", "attn", 4096, 4096, 128, "normal", seed=0, batch=64),
    )
}


def pm1_f16(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform {-1, +1} as fp16."""
    bits = rng.integers(0, 2, size=shape, dtype=np.int8)
    return (bits.astype(np.float16) * np.float16(2) - np.float16(1)).astype(np.float16)


def normal_f16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) drawn in float32, rounded to fp16 (nearest even)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return x.astype(np.float16)


def quantise_e4m3fn(x: np.ndarray):
    """Per-tensor FP8 quantiser: returns (uint8 E4M3FN codes, fp32 scale = amax/448)."""
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    y = np.clip(x / scale, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, float(scale)


def normal_e4m3fn(rng: np.random.Generator, shape):
    """N(0, 1) in float32 quantised per tensor: (codes, scale)."""
    return quantise_e4m3fn(rng.standard_normal(size=shape, dtype=np.float32))


def pm1_e4m3fn(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform {-1, +1} encoded directly as E4M3FN codes 0x38 / 0xB8 (scale 1)."""
    bits = rng.integers(0, 2, size=shape, dtype=np.uint8)
    return np.where(bits == 1, np.uint8(0x38), np.uint8(0xB8)).astype(np.uint8)


def make(w: Workload | str, dist: str | None = None, seed: int | None = None):
    """Host inputs of a workload.

    Returns a dict with
      f16:  A [M, K] fp16, B [N, K] fp16 (row n = column n of B)
      f8:   A [M, K] uint8, B [N, K] uint8, scale_a, scale_b (fp32 values)
      qkt:  Q [batch, M, D] fp16, K [batch, N, D] fp16
      attn: Q [batch, M, D], K [batch, N, D], Vt [batch, D, N] fp16 (Vt row d =
            column d of V), all N(0, std^2)
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    dist = w.dist if dist is None else dist
    seed = w.seed if seed is None else seed
    return make_shape(w.kind, w.M, w.N, w.K, dist=dist, seed=seed, batch=w.batch, std=w.std)


def make_shape(kind: str, M: int, N: int, K: int, dist: str = "normal", seed: int = 0,
               batch: int = 1, std: float = 1.0):
    rng = np.random.default_rng(seed)
    if kind == "f16":
        if dist == "pm1":
            return {"A": pm1_f16(rng, (M, K)), "B": pm1_f16(rng, (N, K))}
        return {"A": normal_f16(rng, (M, K), std), "B": normal_f16(rng, (N, K), std)}
    if kind == "f8":
        if dist == "pm1":
            return {"A": pm1_e4m3fn(rng, (M, K)), "B": pm1_e4m3fn(rng, (N, K)),
                    "scale_a": 1.0, "scale_b": 1.0}
        a, sa = normal_e4m3fn(rng, (M, K))
        b, sb = normal_e4m3fn(rng, (N, K))
        return {"A": a, "B": b, "scale_a": sa, "scale_b": sb}
    if kind == "qkt":
        if dist == "pm1":
            return {"Q": pm1_f16(rng, (batch, M, K)), "K": pm1_f16(rng, (batch, N, K))}
        return {"Q": normal_f16(rng, (batch, M, K), std), "K": normal_f16(rng, (batch, N, K), std)}
    if kind == "attn":
        if dist != "normal":
            raise ValueError("attention inputs are normal only")
        return {"Q": normal_f16(rng, (batch, M, K), std), "K": normal_f16(rng, (batch, N, K), std),
                "Vt": normal_f16(rng, (batch, K, N), std)}
    raise ValueError("unknown kind %r" % kind)
