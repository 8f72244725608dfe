"""Host-side checks of the C ABI (no kernel launches: runs without a GPU).

  * the library loads and exports every function declared in include/dense_gemm_tn.h;
  * argument validation returns the documented status before any HIP call;
  * the block -> tile order is a bijection onto all (head, tile_m, tile_n) for
    every workload's grid and for ragged grids, and each XCD receives a
    contiguous run of logical tiles;
  * the tile-configuration selector picks the documented kernel for each
    workload shape (with the 256-CU count the library assumes without a device).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import dense_gemm_tn_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dense_gemm_tn.h")


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(dg.LIB_PATH):
        from dense_gemm_tn_amd import build

        build.build()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(dg.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = dg.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name


def test_status_strings():
    assert dg.status_string(0) == "ok"
    assert dg.status_string(1) == "invalid argument"
    assert dg.status_string(2) == "unsupported argument"
    assert dg.status_string(3) == "HIP launch error"
    assert dg.status_string(99) == "unknown status"
    assert dg.block_tile() == 256


# Fake, well-aligned, non-overlapping device addresses: validation never dereferences.
A_ADDR, B_ADDR, C_ADDR = 0x10000000, 0x40000000, 0x70000000


def f16(*args, **kw):
    L = dg.lib()
    return L.gemm_f16_tn(*args, None)


@pytest.mark.parametrize("args,status", [
    ((A_ADDR, B_ADDR, C_ADDR, -1, 8, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),
    ((A_ADDR, B_ADDR, C_ADDR, 8, -1, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),
    ((A_ADDR, B_ADDR, C_ADDR, 8, 8, -8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),
    ((A_ADDR, B_ADDR, C_ADDR, 8, 8, 16, 8, 16, 8), dg.DG_ERR_INVALID_ARGUMENT),   # lda < K
    ((A_ADDR, B_ADDR, C_ADDR, 8, 8, 16, 16, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),   # ldb < K
    ((A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 4), dg.DG_ERR_INVALID_ARGUMENT),     # ldc < M
    ((None, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),       # null A
    ((A_ADDR, B_ADDR, None, 8, 8, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),       # null C
    ((A_ADDR, B_ADDR, A_ADDR + 64, 8, 8, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),  # C overlaps A
    ((A_ADDR, B_ADDR, C_ADDR, 8, 8, 12, 16, 16, 8), dg.DG_ERR_UNSUPPORTED),       # K % 8
    ((A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 12, 8, 8), dg.DG_ERR_UNSUPPORTED),         # lda % 8
    ((A_ADDR + 2, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 8), dg.DG_ERR_UNSUPPORTED),      # misaligned
    ((1 << 44, 2 << 44, 3 << 44, 300, 8, 8 << 20, 8 << 20, 8 << 20, 300),
     dg.DG_ERR_UNSUPPORTED),                                                      # strip >= 2 GiB
    ((None, None, None, 0, 8, 8, 8, 8, 8), dg.DG_OK),                             # M = 0: no-op
    ((None, None, None, 8, 0, 8, 8, 8, 8), dg.DG_OK),                             # N = 0: no-op
])
def test_f16_validation(args, status):
    assert f16(*args) == status


def f16_any(ta, tb, *args):
    return dg.lib().gemm_f16(ta, tb, *args, None)


@pytest.mark.parametrize("codes,args,status", [
    ((b"X", b"N"), (A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),
    ((b"N", b"Q"), (A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),
    ((b"N", b"N"), (A_ADDR, B_ADDR, C_ADDR, 16, 8, 8, 8, 8, 16), dg.DG_ERR_INVALID_ARGUMENT),  # lda < M
    ((b"T", b"T"), (A_ADDR, B_ADDR, C_ADDR, 8, 16, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),  # ldb < N
    ((b"n", b"t"), (A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 4), dg.DG_ERR_INVALID_ARGUMENT),   # ldc < M
    ((b"N", b"N"), (A_ADDR, B_ADDR, A_ADDR + 32, 8, 8, 8, 8, 8, 8),
     dg.DG_ERR_INVALID_ARGUMENT),                                                     # C overlaps A
    ((b"N", b"T"), (None, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 8), dg.DG_ERR_INVALID_ARGUMENT),
    ((b"N", b"N"), (A_ADDR, B_ADDR, C_ADDR, 12, 8, 8, 16, 8, 12), dg.DG_ERR_UNSUPPORTED),  # M % 8
    ((b"T", b"T"), (A_ADDR, B_ADDR, C_ADDR, 8, 12, 8, 8, 16, 8), dg.DG_ERR_UNSUPPORTED),   # N % 8
    ((b"N", b"N"), (A_ADDR, B_ADDR, C_ADDR, 8, 8, 12, 8, 16, 8), dg.DG_ERR_UNSUPPORTED),   # K % 8, B K-major
    ((b"N", b"T"), (A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 12, 8, 8), dg.DG_ERR_UNSUPPORTED),    # lda % 8
    ((b"N", b"T"), (A_ADDR, B_ADDR + 2, C_ADDR, 8, 8, 8, 8, 8, 8), dg.DG_ERR_UNSUPPORTED),  # misaligned
    ((b"N", b"N"), (1 << 44, 2 << 44, 3 << 44, 8, 8, 8, 16 << 20, 8, 8),
     dg.DG_ERR_UNSUPPORTED),                                                          # 64 rows >= 2 GiB
    ((b"T", b"N"), (A_ADDR, B_ADDR, C_ADDR, 8, 8, 12, 16, 16, 8), dg.DG_ERR_UNSUPPORTED),  # TN rules
    ((b"N", b"T"), (None, None, None, 0, 8, 8, 8, 8, 8), dg.DG_OK),                    # M = 0: no-op
    ((b"T", b"T"), (None, None, None, 8, 0, 8, 8, 8, 8), dg.DG_OK),                    # N = 0: no-op
])
def test_f16_any_layout_validation(codes, args, status):
    assert f16_any(*codes, *args) == status


def test_f16_layout_selector(monkeypatch):
    """Layouts with an M/N-contiguous operand take 256 x 256 or 128 x 128 tiles only;
    TN keeps gemm_tn_config's choice."""
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    for M, N, K in [(4096, 4096, 4096), (2048, 2048, 2048), (1920, 13900, 4096),
                    (256, 256, 64), (8192, 8192, 8192), (1000, 1000, 136)]:
        tn = dg.lib().gemm_tn_config(0, M, N, K, 1)
        assert dg.f16_config("T", "N", M, N, K) == tn
        for ta, tb in [("N", "N"), ("T", "T"), ("N", "T")]:
            c = dg.f16_config(ta, tb, M, N, K)
            assert c in (0, 2)
            if tn in (0, 2):
                assert c == tn
            if K <= 128:
                assert c == 2
    assert dg.f16_config("N", "T", 4096, 4096, 4096) == 0
    assert dg.lib().gemm_f16_config(b"X", b"N", 8, 8, 8) == -1
    assert dg.lib().gemm_f16_config(b"N", b"N", -1, 8, 8) == -1
    monkeypatch.setenv("DG_GEMM_TILE", "224")
    assert dg.f16_config("N", "N", 512, 512, 512) == 0
    assert dg.f16_config("T", "N", 512, 512, 512) == 1
    monkeypatch.setenv("DG_GEMM_TILE", "pingpong")     # TN only: layouts keep their choice
    assert dg.f16_config("N", "N", 4096, 4096, 4096) == 0
    assert dg.f16_config("T", "N", 4096, 4096, 4096) == 4


@pytest.mark.parametrize("codes,args,status", [
    ((b"X", b"N"), (A_ADDR, B_ADDR, C_ADDR, 16, 16, 16, 16, 16, 16), dg.DG_ERR_INVALID_ARGUMENT),
    ((b"N", b"N"), (A_ADDR, B_ADDR, C_ADDR, 32, 16, 16, 16, 16, 32), dg.DG_ERR_INVALID_ARGUMENT),
    ((b"N", b"N"), (A_ADDR, B_ADDR, C_ADDR, 24, 16, 16, 32, 16, 24), dg.DG_ERR_UNSUPPORTED),  # M % 16
    ((b"T", b"T"), (A_ADDR, B_ADDR, C_ADDR, 16, 24, 16, 16, 32, 16), dg.DG_ERR_UNSUPPORTED),  # N % 16
    ((b"N", b"N"), (A_ADDR, B_ADDR, C_ADDR, 16, 16, 24, 16, 32, 16), dg.DG_ERR_UNSUPPORTED),  # K % 16
    ((b"N", b"T"), (A_ADDR, B_ADDR, C_ADDR, 16, 16, 16, 24, 16, 16), dg.DG_ERR_UNSUPPORTED),  # lda % 16
    ((b"N", b"T"), (A_ADDR, B_ADDR, C_ADDR, 16, 16, 8, 8, 16, 16), dg.DG_ERR_INVALID_ARGUMENT),
    ((b"T", b"N"), (A_ADDR, B_ADDR, C_ADDR, 16, 16, 8, 16, 16, 16), dg.DG_ERR_UNSUPPORTED),   # TN rules
    ((b"N", b"N"), (1 << 44, 2 << 44, 3 << 44, 16, 16, 16, 16 << 20, 16, 16),
     dg.DG_ERR_UNSUPPORTED),                                                  # 128 K-rows >= 2 GiB
    ((b"T", b"T"), (1 << 44, 2 << 44, 3 << 44, 16, 16, 16, 16, 16 << 20, 16),
     dg.DG_ERR_UNSUPPORTED),                                                  # the same for B
    ((b"N", b"T"), (None, None, None, 0, 16, 16, 16, 16, 16), dg.DG_OK),
])
def test_f8_any_layout_validation(codes, args, status):
    assert dg.lib().gemm_f8(*codes, *args, 1.0, 1.0, None) == status


def test_f8_layout_selector(monkeypatch):
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    for M, N, K in [(8192, 8192, 8192), (2048, 2048, 2048), (1024, 1024, 256)]:
        tn = dg.lib().gemm_tn_config(1, M, N, K, 1)
        assert dg.f8_config("T", "N", M, N, K) == tn
        for ta, tb in [("N", "N"), ("T", "T"), ("N", "T")]:
            c = dg.f8_config(ta, tb, M, N, K)
            assert c in (0, 2)
            if K <= 256:
                assert c == 2
    assert dg.f8_config("N", "N", 8192, 8192, 8192) == 0
    assert dg.lib().gemm_f8_config(b"Q", b"N", 16, 16, 16) == -1


def test_f16_binding_rejects_bad_codes():
    with pytest.raises(ValueError):
        dg.gemm_f16("X", "N", A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 8)
    with pytest.raises(ValueError):
        dg.gemm_f16("NN", "N", A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 8, 8, 8)


def test_f8_validation():
    L = dg.lib()
    assert L.gemm_f8_tn(A_ADDR, B_ADDR, C_ADDR, 8, 8, 8, 16, 16, 8, 1.0, 1.0, None) == \
        dg.DG_ERR_UNSUPPORTED  # K must be a multiple of 16 bytes = 16 fp8 elements
    assert L.gemm_f8_tn(A_ADDR, B_ADDR, C_ADDR, 8, 8, 16, 16, 24, 8, 1.0, 1.0, None) == \
        dg.DG_ERR_UNSUPPORTED
    assert L.gemm_f8_tn(A_ADDR, B_ADDR, C_ADDR, 8, 8, 16, 8, 16, 8, 1.0, 1.0, None) == \
        dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_f8_tn(None, None, None, 0, 0, 16, 16, 16, 0, 1.0, 1.0, None) == dg.DG_OK


def test_batched_validation():
    L = dg.lib()
    # heads of S overlap (stride_s < lds * N)
    assert L.gemm_batched_qkt(A_ADDR, B_ADDR, C_ADDR, 2, 64, 64, 128, 128, 128, 64,
                              64 * 128, 64 * 128, 64 * 63, None) == dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_batched_qkt(A_ADDR, B_ADDR, C_ADDR, -1, 64, 64, 128, 128, 128, 64,
                              0, 0, 0, None) == dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_batched_qkt(None, None, None, 0, 64, 64, 128, 128, 128, 64,
                              0, 0, 0, None) == dg.DG_OK
    # S of head 1 runs into Q
    assert L.gemm_batched_qkt(A_ADDR, B_ADDR, A_ADDR - 64 * 64 * 2, 2, 64, 64, 128, 128, 128,
                              64, 64 * 128, 64 * 128, 64 * 64, None) == \
        dg.DG_ERR_INVALID_ARGUMENT


def attn(Q=A_ADDR, K=B_ADDR, V=C_ADDR, O=0x7C000000, batch=2, M=64, N=64, D=128, ldq=128,
         ldk=128, ldv=64, ldo=128, sq=8192, sk=8192, sv=8192, so=8192, scale=0.088):
    return dg.lib().attention_fwd_f16(Q, K, V, O, batch, M, N, D, ldq, ldk, ldv, ldo, sq, sk, sv,
                                      so, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), dg.DG_ERR_INVALID_ARGUMENT),
    (dict(N=0), dg.DG_ERR_INVALID_ARGUMENT),                   # softmax over no keys
    (dict(sq=-8), dg.DG_ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), dg.DG_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), dg.DG_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), dg.DG_ERR_INVALID_ARGUMENT),
    (dict(Q=None), dg.DG_ERR_INVALID_ARGUMENT),
    (dict(O=None), dg.DG_ERR_INVALID_ARGUMENT),
    (dict(ldq=64), dg.DG_ERR_INVALID_ARGUMENT),                # ldq < D
    (dict(ldv=56), dg.DG_ERR_INVALID_ARGUMENT),                # ldv < N
    (dict(ldo=120), dg.DG_ERR_INVALID_ARGUMENT),               # ldo < D
    (dict(so=64 * 128 - 8), dg.DG_ERR_INVALID_ARGUMENT),       # heads of O overlap
    (dict(O=A_ADDR + 4096), dg.DG_ERR_INVALID_ARGUMENT),       # O overlaps Q
    (dict(O=C_ADDR - 8192 * 2), dg.DG_ERR_INVALID_ARGUMENT),   # head 1 of O runs into Vt
    (dict(D=64, ldq=64, ldk=64, ldo=64), dg.DG_ERR_UNSUPPORTED),
    (dict(ldk=132), dg.DG_ERR_UNSUPPORTED),                    # ld % 8
    (dict(sv=8196), dg.DG_ERR_UNSUPPORTED),                    # stride % 8
    (dict(K=B_ADDR + 8), dg.DG_ERR_UNSUPPORTED),               # misaligned
    (dict(Q=1 << 44, K=2 << 44, V=3 << 44, O=4 << 44, N=1 << 23, ldv=1 << 23,
          sq=0, sk=0, sv=0, so=1 << 24), dg.DG_ERR_UNSUPPORTED),  # Vt head >= 2 GiB
    (dict(Q=None, K=None, V=None, O=None, batch=0), dg.DG_OK),   # no-op
    (dict(Q=None, K=None, V=None, O=None, M=0), dg.DG_OK),       # no-op
])
def test_attention_validation(kw, status):
    assert attn(**kw) == status


def test_attention_shared_kv_heads_are_allowed():
    # stride 0 for K and Vt (one K/V for every head) passes validation; checked
    # with M = 0 so nothing launches, and with an O overlap to prove the path
    # reaches the checks after the stride rules.
    assert attn(sk=0, sv=0, M=0) == dg.DG_OK
    assert attn(sk=0, sv=0, O=B_ADDR) == dg.DG_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("tiles_m,tiles_n,batch", [
    (1, 1, 1), (16, 16, 1), (8, 55, 1), (32, 32, 1), (16, 16, 64), (3, 5, 1), (9, 1, 1),
    (1, 13, 3), (7, 11, 2),
])
def test_tile_order_is_a_bijection(tiles_m, tiles_n, batch):
    t = dg.tile_order(tiles_m, tiles_n, batch)
    assert t.shape == (tiles_m * tiles_n * batch, 3)
    assert t[:, 0].min() >= 0 and t[:, 0].max() < batch
    assert t[:, 1].min() >= 0 and t[:, 1].max() < tiles_m
    assert t[:, 2].min() >= 0 and t[:, 2].max() < tiles_n
    key = (t[:, 0] * tiles_m + t[:, 1]) * tiles_n + t[:, 2]
    assert len(np.unique(key)) == len(key)


def test_tile_order_groups_per_xcd():
    """4096^2 with 256x256 tiles: the 32 blocks dealt to one XCD form an 8 x 4 patch."""
    t = dg.tile_order(16, 16, 1)
    for x in range(8):
        mine = t[x::8]
        rows = set(mine[:, 1])
        cols = set(mine[:, 2])
        assert len(mine) == 32 and len(rows) == 8 and len(cols) == 4


@pytest.mark.parametrize("M,N,K,batch,fp8,want", [
    (4096, 4096, 4096, 1, False, 0),      # one full round of 256 x 256 tiles
    (8192, 8192, 8192, 1, True, 0),
    (1920, 13900, 4096, 1, False, 1),     # 224-column tiles pack the grid
    (2048, 2048, 2048, 1, False, 2),      # 64 wide tiles would leave 3/4 of the CUs idle
    (256, 256, 256, 1, False, 2),
    (1000, 700, 3976, 1, False, 2),
    (4096, 4096, 128, 64, False, 3),      # QK^T: K row of 256 bytes
    (1024, 1024, 256, 1, True, 3),        # fp8 K of 256 bytes
    (-1, 4, 4, 1, False, -1),
])
def test_tile_config_selector(M, N, K, batch, fp8, want, monkeypatch):
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    if torch_device_count() > 0:
        pytest.skip("selector expectations assume the 256-CU default of a device-less host")
    assert dg.tn_config(M, N, K, batch, fp8) == want


def test_mid_ring_stages():
    """Ring depth of the 128 x 128 kernel: four stages for grids of at most one
    block per CU (the 256-CU default of a device-less host) with at least
    eight K-steps per block, else two."""
    if torch_device_count() > 0:
        pytest.skip("expectations assume the 256-CU default of a device-less host")
    assert dg.mid_stages(256, 8) == 4 and dg.mid_stages(1, 512) == 4
    assert dg.mid_stages(257, 64) == 2 and dg.mid_stages(256, 7) == 2
    assert dg.mid_stages(0, 0) == 2
    assert dg.mid_stages(-1, 8) == -1 and dg.mid_stages(8, -1) == -1


def test_tile_config_override(monkeypatch):
    for force, code in (("256", 0), ("224", 1), ("128", 2), ("pingpong", 4)):
        monkeypatch.setenv("DG_GEMM_TILE", force)
        assert dg.tn_config(2048, 2048, 2048) == code
        assert dg.tn_config(4096, 4096, 128, 64) == 3   # skinny-K is never forced
    monkeypatch.setenv("DG_GEMM_TILE", "64")            # unknown values are ignored
    assert dg.tn_config(4096, 4096, 4096) in (0, 1, 2)


def torch_device_count():
    try:
        import torch

        return torch.cuda.device_count()
    except Exception:
        return 0


def splitk(*args):
    return dg.lib().gemm_f16_tn_splitk(*args, None)


# 128 x 128 x 8192: 128 K-steps, so any split count >= 2 really splits and the
# workspace checks run (with these fake addresses nothing may be launched).
SK = (A_ADDR, B_ADDR, C_ADDR, 128, 128, 8192, 8192, 8192, 128)
SK_NEED = 4 * 128 * 128 * 4


@pytest.mark.parametrize("tail,status", [
    ((0, 0x20000000, SK_NEED), dg.DG_ERR_INVALID_ARGUMENT),               # splits < 1
    ((65, 0x20000000, 65 * 128 * 128 * 4), dg.DG_ERR_INVALID_ARGUMENT),   # splits > 64
    ((4, None, SK_NEED), dg.DG_ERR_INVALID_ARGUMENT),                     # no workspace
    ((4, 0x20000000, SK_NEED - 4), dg.DG_ERR_INVALID_ARGUMENT),           # too small
    ((4, 0x20000000, -1), dg.DG_ERR_INVALID_ARGUMENT),                    # negative size
    ((4, A_ADDR + 4096, SK_NEED), dg.DG_ERR_INVALID_ARGUMENT),            # overlaps A
    ((4, C_ADDR, SK_NEED), dg.DG_ERR_INVALID_ARGUMENT),                   # overlaps C
    ((4, 0x20000008, SK_NEED), dg.DG_ERR_UNSUPPORTED),                    # misaligned
])
def test_splitk_validation(tail, status):
    assert splitk(*SK, *tail) == status


def test_splitk_validation_keeps_tn_rules():
    # K % 8 and a null A fail as for gemm_f16_tn, before the workspace is looked at.
    assert splitk(A_ADDR, B_ADDR, C_ADDR, 128, 128, 8188, 8192, 8192, 128, 4, None, 0) == \
        dg.DG_ERR_UNSUPPORTED
    assert splitk(None, B_ADDR, C_ADDR, 128, 128, 8192, 8192, 8192, 128, 4, None, 0) == \
        dg.DG_ERR_INVALID_ARGUMENT
    assert splitk(None, None, None, 0, 128, 8192, 8192, 8192, 128, 4, None, 0) == dg.DG_OK
    assert dg.lib().gemm_f8_tn_splitk(A_ADDR, B_ADDR, C_ADDR, 128, 128, 8192, 8192, 8192, 128,
                                      1.0, 1.0, 4, None, 0, None) == dg.DG_ERR_INVALID_ARGUMENT


def test_splitk_workspace_and_choice():
    assert dg.splitk_workspace_bytes(130, 7, 3) == 3 * 7 * 132 * 4
    assert dg.splitk_workspace_bytes(1, 1, 64) == 64 * 4 * 4
    assert dg.splitk_workspace_bytes(8, 8, 0) == -1
    assert dg.splitk_workspace_bytes(8, 8, 65) == -1
    assert dg.splitk_workspace_bytes(-1, 8, 2) == -1
    # Few tiles and a long K split; a full grid or a short K does not.
    assert dg.splitk_choose(512, 512, 32768) > 1
    assert dg.splitk_choose(256, 256, 1 << 20) == 64
    assert dg.splitk_choose(4096, 4096, 4096) == 1
    assert dg.splitk_choose(512, 512, 1024) == 1
    assert dg.splitk_choose(512, 512, 0) == 1
    assert dg.splitk_choose(-1, 512, 4096) == -1


def test_splitk_choose_doubling_rule():
    # One block per CU gives S = CUs / tiles; the count doubles when those
    # ranges are >= 64 K-steps, so the doubled ranges are >= 32 steps
    # (1024^2 x 16384 fp16: 64 tiles, 256 K-steps -> 4 ranges of 64 -> 8 of 32).
    assert dg.splitk_choose(1024, 1024, 16384) == 8
    assert dg.splitk_choose(1024, 1024, 16384, fp8=True) == 4   # 128 steps: 4 ranges of 32
    assert dg.splitk_choose(1024, 512, 16384) == 8              # 256 steps / 8 = 32: no doubling
    assert dg.splitk_choose(512, 512, 32768) == 16
    assert dg.splitk_choose(768, 768, 8192) == 7                # 36 tiles: floor(256 / 36)
    assert dg.splitk_choose(256, 256, 65536) == 64


def test_splitk_choose_medium_grids():
    # Between half and all of 256 CUs' worth of 128 x 128 tiles: two blocks per
    # CU in one round when that cuts the busiest CU's block-steps to <= 0.8 of
    # the unsplit K-steps.
    assert dg.splitk_choose(2048, 1024, 4096) == 2              # 128 tiles: one block per CU
    assert dg.splitk_choose(1536, 1536, 4096) == 3              # 144 tiles: 2 x 22 <= 0.8 x 64
    assert dg.splitk_choose(1536, 1536, 8192) == 3
    assert dg.splitk_choose(1536, 1536, 8192, fp8=True) == 3    # 64 fp8 steps
    assert dg.splitk_choose(1792, 1792, 4096) == 1              # 196 tiles: S = 2 gives 2 x 32
    assert dg.splitk_choose(1536, 1536, 2048) == 1              # 32 steps: S <= 2, no gain
    assert dg.splitk_choose(2048, 2048, 4096) == 1              # 256 tiles: full grid


# ------------------------------------------------- tensor helpers (no launches)

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("call", [
    # CPU tensors: host pointers must never reach a kernel.
    lambda: dg.matmul_tn_f16(torch.zeros(16, 16, dtype=torch.float16),
                             torch.zeros(16, 16, dtype=torch.float16)),
    lambda: dg.matmul_tn_f8(torch.zeros(16, 16, dtype=torch.uint8),
                            torch.zeros(16, 16, dtype=torch.uint8), 1.0, 1.0),
    lambda: dg.qkt(torch.zeros(2, 8, 16, dtype=torch.float16),
                   torch.zeros(2, 8, 16, dtype=torch.float16)),
    lambda: dg.attention(torch.zeros(1, 8, 128, dtype=torch.float16),
                         torch.zeros(1, 8, 128, dtype=torch.float16),
                         torch.zeros(1, 128, 8, dtype=torch.float16)),
    lambda: dg.matmul_f16(torch.zeros(16, 16, dtype=torch.float16),
                          torch.zeros(16, 16, dtype=torch.float16)),
])
def test_helpers_reject_host_tensors(call):
    with pytest.raises(ValueError, match="GPU"):
        call()


def test_helpers_reject_strided_rows():
    a = torch.zeros(16, 32, dtype=torch.float16)[:, ::2]   # stride(1) == 2
    b = torch.zeros(16, 16, dtype=torch.float16)
    with pytest.raises(ValueError, match="contiguous"):
        dg.matmul_tn_f16(a, b)
    with pytest.raises(ValueError, match="contiguous"):
        dg.matmul_tn_f8(torch.zeros(16, 32, dtype=torch.uint8)[:, ::2],
                        torch.zeros(16, 16, dtype=torch.uint8), 1.0, 1.0)
    q = torch.zeros(2, 8, 32, dtype=torch.float16)[:, :, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        dg.qkt(q, torch.zeros(2, 8, 16, dtype=torch.float16))


@pytest.mark.parametrize("out,match", [
    (torch.zeros(8, 16, dtype=torch.float16), "shape"),          # fewer than N rows
    (torch.zeros(16, 8, dtype=torch.float16), "shape"),          # fewer than M columns
    (torch.zeros(16, 16, dtype=torch.float32), "dtype"),
    (torch.zeros(16, 32, dtype=torch.float16)[:, ::2], "contiguous"),
    (torch.zeros(16, 16, dtype=torch.float16).as_strided((16, 16), (4, 1)), "overlap"),
])
def test_helpers_reject_bad_out(out, match):
    a = torch.zeros(16, 16, dtype=torch.float16)
    with pytest.raises(ValueError, match=match):
        dg.matmul_tn_f16(a, a, out=out)
    if out.dtype == torch.float16 and match != "dtype":
        with pytest.raises(ValueError, match=match):
            dg.matmul_f16(a, a, out=out)


def test_qkt_and_attention_reject_bad_out():
    q = torch.zeros(2, 8, 16, dtype=torch.float16)
    with pytest.raises(ValueError, match="shape"):
        dg.qkt(q, q, out=torch.zeros(2, 8, 4, dtype=torch.float16))
    with pytest.raises(ValueError, match="dtype"):
        dg.qkt(q, q, out=torch.zeros(2, 8, 8, dtype=torch.bfloat16))
    q = torch.zeros(1, 8, 128, dtype=torch.float16)
    vt = torch.zeros(1, 128, 8, dtype=torch.float16)
    with pytest.raises(ValueError, match="shape"):
        dg.attention(q, q, vt, out=torch.zeros(1, 4, 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="dtype"):
        dg.matmul_tn_f8(torch.zeros(16, 16, dtype=torch.uint8), torch.zeros(16, 16, dtype=torch.uint8),
                        1.0, 1.0, out=torch.zeros(16, 16, dtype=torch.float16))


def test_clock_record_validation():
    L = dg.lib()
    assert L.gemm_clock_record(None, 0) == dg.DG_OK
    assert L.gemm_clock_records_used() == 0
    assert L.gemm_clock_record(None, 5) == dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_clock_record(A_ADDR, 0) == dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_clock_record(A_ADDR, -1) == dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_clock_record(A_ADDR + 4, 8) == dg.DG_ERR_UNSUPPORTED
    assert L.gemm_clock_record(None, 0) == dg.DG_OK


def test_noalloc_splitk_host_rules():
    L = dg.lib()
    f = L.gemm_f16_tn_splitk_noalloc
    # Beyond the 32 MiB array: rejected on the host, before any device call.
    assert f(A_ADDR, B_ADDR, C_ADDR, 1024, 1024, 16384, 16384, 16384, 1024, 9, None) == \
        dg.DG_ERR_UNSUPPORTED
    assert f(A_ADDR, B_ADDR, C_ADDR, 4096, 4096, 8192, 8192, 8192, 4096, 64, None) == \
        dg.DG_ERR_UNSUPPORTED
    assert f(A_ADDR, B_ADDR, C_ADDR, 128, 128, 8192, 8192, 8192, 128, 0, None) == \
        dg.DG_ERR_INVALID_ARGUMENT
    assert f(A_ADDR, B_ADDR, C_ADDR, 128, 128, 8192, 8192, 8192, 128, 65, None) == \
        dg.DG_ERR_INVALID_ARGUMENT
    # The gemm_f16_tn rules still apply (K % 8, null A), and M = 0 is a no-op.
    assert f(A_ADDR, B_ADDR, C_ADDR, 128, 128, 8188, 8192, 8192, 128, 4, None) == \
        dg.DG_ERR_UNSUPPORTED
    assert f(None, B_ADDR, C_ADDR, 128, 128, 8192, 8192, 8192, 128, 4, None) == \
        dg.DG_ERR_INVALID_ARGUMENT
    assert f(None, None, None, 0, 128, 8192, 8192, 8192, 128, 4, None) == dg.DG_OK


def test_library_source_allocates_nothing():
    """No entry point allocates device memory: the library's sources name no
    allocation call (comments aside)."""
    for name in ("gemm_tn.hip", "attention.hip"):
        text = open(os.path.join(ROOT, "dense_gemm_tn_amd", "csrc", name)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        code = "\n".join(re.sub(r"//.*$", "", ln) for ln in text.splitlines())
        for call in ("hipMalloc", "hipFree", "hipHostMalloc", "hipMallocAsync", "hipExtMalloc"):
            assert call not in code, (name, call)


# ------------------------------------------------- plans (host logic, no launches)

def _no_device():
    if torch_device_count() > 0:
        pytest.skip("plan expectations assume the 256-CU default of a device-less host")


@pytest.mark.parametrize("M,N,K,batch,fp8", [
    (4096, 4096, 4096, 1, False),    # one full round
    (8192, 8192, 8192, 1, True),     # four full rounds
    (1920, 13900, 4096, 1, False),   # 224-wide tiles: 504 of 512 slots
    (256, 256, 256, 1, False),
    (255, 257, 256, 1, False),
    (4096, 4096, 128, 64, False),    # skinny-K heads
    (8192, 8192, 8192, 1, False),
    (6144, 6144, 4096, 1, False),
    (8192, 8448, 4096, 1, False),
])
def test_plan_keeps_single_launch(M, N, K, batch, fp8, monkeypatch):
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    _no_device()
    for ws in (0, 1 << 40):
        p = dg.tn_plan(M, N, K, batch=batch, workspace_bytes=ws, fp8=fp8)
        assert p == {"config": dg.tn_config(M, N, K, batch, fp8), "dp_cols": 0, "dp_config": -1,
                     "splits": 1, "workspace_bytes": 0}


@pytest.mark.parametrize("M,N,K,batch,fp8", [
    (4096, 4608, 4096, 1, False),    # 288 tiles of 256 x 256: a second round of 32
    (4096, 4608, 4096, 1, True),
    (4096, 4352, 4096, 1, False),
    (4000, 4352, 4096, 1, True),
    (2048, 9216, 8192, 1, False),
    (4096, 4352, 256, 2, False),     # two heads, 256-deep contraction
])
def test_plan_splits_ragged_last_round(M, N, K, batch, fp8, monkeypatch):
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    _no_device()
    p = dg.tn_plan(M, N, K, batch=batch, fp8=fp8)
    assert p["config"] == dg.tn_config(M, N, K, batch, fp8)
    assert p["dp_config"] in (0, 1) and p["splits"] == 1 and p["workspace_bytes"] == 0
    w = 256 if p["dp_config"] == 0 else 224
    assert 0 < p["dp_cols"] < N and p["dp_cols"] % w == 0
    # The first columns fill whole rounds of one block per CU (at most one
    # round fewer than the single launch of that tile width would take).
    col_tiles = -(-M // 256) * batch
    rounds = -(-col_tiles * -(-N // w) // 256)
    assert col_tiles * (p["dp_cols"] // w) <= 256 * (rounds - 1)
    assert col_tiles * (p["dp_cols"] // w + 1) > 256 * (rounds - 1)
    # DG_GEMM_TILE forces one launch.
    monkeypatch.setenv("DG_GEMM_TILE", "256")
    assert dg.tn_plan(M, N, K, batch=batch, fp8=fp8)["dp_cols"] == 0


def test_plan_workspace_rules(monkeypatch):
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    _no_device()
    M, N, K = 4096, 4352, 4096
    need = dg.tn_workspace_bytes(M, N, K)
    p = dg.tn_plan(M, N, K, workspace_bytes=need)
    assert need > 0 and p["workspace_bytes"] == need and p["splits"] > 1 and p["dp_cols"] > 0
    # The tail's split-K partials: splits x tail columns of padded M.
    assert need == dg.splitk_workspace_bytes(M, N - p["dp_cols"], p["splits"])
    q = dg.tn_plan(M, N, K, workspace_bytes=need - 1)
    assert q["workspace_bytes"] <= need - 1
    # Few tiles and a long K: split-K of the whole product, the chooser's count.
    r = dg.tn_plan(512, 512, 32768, workspace_bytes=1 << 30)
    assert r["dp_cols"] == 0 and r["splits"] == dg.splitk_choose(512, 512, 32768) > 1
    assert r["workspace_bytes"] == dg.splitk_workspace_bytes(512, 512, r["splits"])
    assert dg.tn_workspace_bytes(4096, 4096, 4096) == 0
    assert dg.tn_workspace_bytes(-1, 4, 4) == -1
    L = dg.lib()
    assert L.gemm_tn_plan(0, 4, 4, 4, 1, 0, None) == dg.DG_ERR_INVALID_ARGUMENT
    out = (ctypes.c_int64 * 5)()
    assert L.gemm_tn_plan(0, 4, 4, 4, 1, -1, ctypes.addressof(out)) == dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_tn_plan(0, 4, -4, 4, 1, 0, ctypes.addressof(out)) == dg.DG_ERR_INVALID_ARGUMENT


# 4096 x 4352 x 4096 at the fake addresses (A 32 MiB, B and C 34 MiB each).
# With a large workspace its plan uses 16 MiB of it (checked first: every
# case below must fail before a launch).
WS = (A_ADDR, B_ADDR, C_ADDR, 4096, 4352, 4096, 4096, 4096, 4096)
ARENA = 1 << 30


@pytest.mark.parametrize("tail,status", [
    ((None, 16), dg.DG_ERR_INVALID_ARGUMENT),                  # no workspace, nonzero bytes
    ((0x20000000, -1), dg.DG_ERR_INVALID_ARGUMENT),            # negative size
    ((A_ADDR + 4096, ARENA), dg.DG_ERR_INVALID_ARGUMENT),      # used bytes overlap A
    ((B_ADDR - 4096, ARENA), dg.DG_ERR_INVALID_ARGUMENT),      # used bytes overlap B
    ((C_ADDR + (1 << 20), ARENA), dg.DG_ERR_INVALID_ARGUMENT),  # used bytes overlap C
    ((0x20000008, ARENA), dg.DG_ERR_UNSUPPORTED),              # misaligned
])
def test_ws_call_validation(tail, status):
    used = dg.tn_plan(4096, 4352, 4096, workspace_bytes=ARENA)["workspace_bytes"]
    used8 = dg.tn_plan(4096, 4352, 4096, workspace_bytes=ARENA, fp8=True)["workspace_bytes"]
    if tail[1] == ARENA and used == 0:
        pytest.skip("on this device the plan needs no workspace; the call would launch")
    L = dg.lib()
    assert L.gemm_f16_tn_ws(*WS, *tail, None) == status
    if tail[1] != ARENA or used8 > 0:
        assert L.gemm_f8_tn_ws(*WS, 1.0, 1.0, *tail, None) == status


def test_ws_call_keeps_tn_rules():
    L = dg.lib()
    # K % 8 and a null A fail as for gemm_f16_tn; M = 0 is a no-op.
    assert L.gemm_f16_tn_ws(A_ADDR, B_ADDR, C_ADDR, 128, 128, 8188, 8192, 8192, 128, None, 0,
                            None) == dg.DG_ERR_UNSUPPORTED
    assert L.gemm_f16_tn_ws(None, B_ADDR, C_ADDR, 128, 128, 8192, 8192, 8192, 128, None, 0,
                            None) == dg.DG_ERR_INVALID_ARGUMENT
    assert L.gemm_f16_tn_ws(None, None, None, 0, 128, 8192, 8192, 8192, 128, None, 0,
                            None) == dg.DG_OK
