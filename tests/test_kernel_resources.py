"""Compile-time resources of every kernel (no GPU needed).

The device code of both sources is compiled with the build's flags and the
compiler's resource-usage remarks (the resource report the RDNA page reads in
"Measuring resources": registers, scratch, LDS).  Every kernel must run
without scratch (no register spills: a spill in the 256-register kernels
turns into memory traffic inside the block), the 256 x 256 kernels must hold
their 256 accumulator registers as AGPRs at one wave per SIMD, and the report
is written to profiles/kernel_resources.md.
"""
import pytest

from dense_gemm_tn_amd import build


@pytest.fixture(scope="module")
def rows():
    r = build.resources()
    build.write_resource_report(r)
    return r


def test_every_kernel_reported(rows):
    names = {r["kernel"] for r in rows}
    for want in ("gemm_tn_ring_kernel<0, 8, true>", "gemm_tn_ring_kernel<1, 8, true>",
                 "gemm_tn_ring_kernel<0, 7, false>", "gemm_tn_ring_kernel<1, 7, false>",
                 "gemm_tn_kernel<0, 8, false, false, true>",
                 "gemm_tn_kernel<1, 8, true, false, false>",
                 "gemm_tn_skinny_kernel<0>", "gemm_tn_mid_kernel<0, false, false, false, 2, false>",
                 "gemm_tn_mid_kernel<0, false, false, false, 4, true>",
                 "gemm_tn_mid_kernel<1, false, false, true, 4, true>",
                 "gemm_tn_mid_kernel<1, false, false, true, 2, true>",
                 "gemm_splitk_reduce_kernel<0>", "attention_fwd_kernel"):
        assert any(want in n for n in names), want
    assert len(rows) >= 31


def test_no_scratch_anywhere(rows):
    bad = [(r["kernel"], r.get("ScratchSize [bytes/lane]"), r.get("VGPRs Spill"))
           for r in rows
           if r.get("ScratchSize [bytes/lane]") != "0" or r.get("VGPRs Spill", "0") != "0"]
    assert not bad, bad


def test_big_tiles_hold_accumulators_in_agprs(rows):
    """256-row tiles: accumulators in AGPRs at one wave per SIMD; two [A | B]
    stages (128 KiB), or the TN kernel's three A and two B strips (160 KiB)."""
    for r in rows:
        if "gemm_tn_kernel<" in r["kernel"] or "gemm_tn_ring_kernel<" in r["kernel"]:
            assert int(r["AGPRs"]) >= 224 and r["Occupancy [waves/SIMD]"] == "1", r
            lds = 163840 if "ring" in r["kernel"] else 131072
            assert int(r["LDS Size [bytes/block]"]) == lds, r


def test_mid_kernel_rings_fit_their_occupancy(rows):
    """The 128 x 128 kernel: two-stage ring (64 KiB) at two blocks per CU, the
    four-stage ring (128 KiB) for grids of one block per CU; both in the
    general form and in the fixed-offset form for whole K-steps."""
    seen = set()
    for r in rows:
        if "gemm_tn_mid_kernel<" in r["kernel"]:
            stages = r["kernel"].split("<")[1].split(",")[4].strip()
            lds = int(r["LDS Size [bytes/block]"])
            assert (stages, lds) in (("2", 65536), ("4", 131072)), r
            if stages == "2":
                assert int(r["Occupancy [waves/SIMD]"]) >= 2, r
            seen.add(stages)
    assert seen == {"2", "4"}
