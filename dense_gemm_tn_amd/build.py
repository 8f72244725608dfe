"""Build step for the gfx950 library: hipcc, in-tree output.

    python -m dense_gemm_tn_amd.build            # build libdense_gemm_tn.so
    python -m dense_gemm_tn_amd.build --resources  # also write the kernel resource report

compiles ``csrc/gemm_tn.hip`` (GEMM kernels) and ``csrc/attention.hip`` (fused
attention forward) into objects in parallel and links them into
``libdense_gemm_tn.so`` next to this file.  ``resources()`` compiles the
device code once more with the compiler's resource-usage remarks and returns,
per kernel, its VGPR / AGPR / SGPR counts, scratch bytes per lane, LDS bytes per
block and occupancy (waves per SIMD).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("gemm_tn.hip", "attention.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdense_gemm_tn.so")
RESOURCE_REPORT = os.path.join(ROOT, "profiles", "kernel_resources.md")

HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=gfx950",
    "-fPIC",
    # Keep the compiler from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _run_all(cmds, verbose=False):
    """Run the commands concurrently; raise if any fails.  Returns their stderr."""
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
    errs = [p.communicate()[1] for p in procs]
    for cmd, p, err in zip(cmds, procs, errs):
        if p.returncode != 0:
            sys.stderr.write(err)
            raise subprocess.CalledProcessError(p.returncode, cmd)
    return errs


def build(verbose: bool = False) -> str:
    tag = "%d" % os.getpid()
    objs = [os.path.join(HERE, "%s.%s.o" % (os.path.basename(s), tag)) for s in SRCS]
    tmp = LIB + ".tmp" + tag
    try:
        _run_all([[hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-c", "-o", o, s]
                  for s, o in zip(SRCS, objs)], verbose)
        _run_all([[hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]],
                 verbose)
        os.replace(tmp, LIB)
    finally:
        for f in objs + [tmp]:
            if os.path.exists(f):
                os.remove(f)
    return LIB


_REMARK = re.compile(r"remark:\s+([\w \[\]/]+?): (.*?) \[-Rpass-analysis=kernel-resource-usage\]")


def resources() -> list[dict]:
    """Per-kernel resource usage from the compiler's remarks (device code of
    both sources, the build's flags), in source order."""
    cmds = [[hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "--cuda-device-only", "-c", "-o", os.devnull,
             "-Rpass-analysis=kernel-resource-usage", s] for s in SRCS]
    rows = []
    for src, err in zip(SRCS, _run_all(cmds)):
        cur = None
        for line in err.splitlines():
            m = _REMARK.search(line)
            if not m:
                continue
            key, val = m.group(1).strip(), m.group(2).strip()
            if key == "Function Name":
                cur = {"symbol": val, "source": os.path.basename(src)}
                rows.append(cur)
            elif cur is not None:
                cur[key] = val
    names = subprocess.run(["c++filt"], input="\n".join(r["symbol"] for r in rows),
                           capture_output=True, text=True).stdout.splitlines()
    for r, n in zip(rows, names):
        r["kernel"] = n.strip()
    return rows


def write_resource_report(rows: list[dict], path: str = RESOURCE_REPORT) -> str:
    cols = [("VGPRs", "VGPRs"), ("AGPRs", "AGPRs"), ("TotalSGPRs", "SGPRs"),
            ("ScratchSize [bytes/lane]", "scratch B/lane"), ("VGPRs Spill", "VGPR spills"),
            ("LDS Size [bytes/block]", "LDS B/block"), ("Occupancy [waves/SIMD]", "waves/SIMD")]
    lines = ["# Kernel resources (compiler report)", "",
             "Command: `python -m dense_gemm_tn_amd.build --resources` (hipcc %s"
             " --cuda-device-only -Rpass-analysis=kernel-resource-usage on each source)."
             % " ".join(HIPCC_FLAGS), "",
             "| kernel | source | " + " | ".join(c[1] for c in cols) + " |",
             "|---|---|" + "---|" * len(cols)]
    for r in rows:
        lines.append("| `%s` | %s | " % (r["kernel"], r["source"]) +
                     " | ".join(r.get(c[0], "?") for c in cols) + " |")
    text = "\n".join(lines) + "\n"
    old = open(path).read() if os.path.exists(path) else None
    if old != text:
        with open(path, "w") as f:
            f.write(text)
    return path


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    if "--resources" in sys.argv:
        print(write_resource_report(resources()))
