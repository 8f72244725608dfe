"""Host-side checks of the C ABI (no kernel launches: runs without a GPU).

  * the library loads and exports every function declared in include/dense_gemm_tn.h;
  * argument validation returns the documented status before any HIP call;
  * the block -> tile order is a bijection onto all (head, tile_m, tile_n) for
    every workload's grid and for ragged grids, and each XCD receives a
    contiguous run of logical tiles.
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
