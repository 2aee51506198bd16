"""Build libslq.so (the HIP kernels and the C ABI of include/slice.h) for gfx950.

Run as ``python -m layer_sliced_quantized_amd.build`` or through
``__graft_entry__.build()``.  Sources compile in parallel, then link in-tree.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "slq")
LIB = os.path.join(HERE, "libslq.so")
SOURCES = ["gemv.hip", "chain.hip", "gemm.hip", "gemm_q4.hip", "gemm_q8.hip", "deltanet.hip", "attn.hip", "misc.hip", "slice.cpp"] + [
    f"gemv_{q}_{e}.hip" for q in ("q4", "q8") for e in ("store", "swiglu", "resid")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # every multiply-add in the kernels is written out explicitly; the compiler
    # may not fuse others, so results do not depend on code shape
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Kernels whose hand-placed memory waits count only their own loads: the
# batched MFMA products (k_gemm_*) wait for a fixed number of outstanding
# vector loads per block, which holds only if the compiler adds none (a
# scratch spill would).  Their sources are compiled with the resource-usage
# remarks and the build fails if any of them uses scratch.
NO_SCRATCH = {"gemm_q4.hip": "k_gemm_", "gemm_q8.hip": "k_gemm_", "gemm.hip": "k_gemm_"}


def scratch_users(remarks: str, prefix: str) -> list:
    """(kernel, bytes per lane) of every kernel whose mangled name holds
    `prefix` and whose resource-usage remark reports scratch."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and prefix in name and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    if src in NO_SCRATCH:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"compile of {src} failed:\n{r.stderr[-8000:]}")
    if src in NO_SCRATCH:
        bad = scratch_users(r.stderr, NO_SCRATCH[src])
        if bad:
            raise RuntimeError(f"{src}: kernels with hand-counted memory waits use scratch: {bad}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4, 16)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
