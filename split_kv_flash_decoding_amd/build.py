"""Compile the HIP library (libfd.so) for gfx950, in-tree.

Run as ``python -m split_kv_flash_decoding_amd.build``. The library is placed
next to this file; the binding loads it from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfd.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["fd_host.cpp", "fd_api.hip", "fd_partial_valu.hip", "fd_partial_mfma.hip", "fd_combine.hip",
           "fd_append.hip", "fd_prefill.hip", "fd_probe.hip"]

# Packed fp32 instructions stay off (the compiler would otherwise form
# v_pk_* fp32 ops from float code). MFMA accumulators live in ordinary VGPRs:
# with the default AGPR form the allocator copied the 32 accumulator registers
# out and back around every tile of the GQA kernel (68 extra moves per tile).
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(x for x in (res.stdout + res.stderr).splitlines() if noise not in x)
    if warn.strip() and verbose:
        sys.stderr.write(warn + "\n")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source to an object (in parallel), link libfd.so, and
    replace the library atomically."""
    cc = hipcc()
    objdir = tempfile.mkdtemp(prefix="fd_build_")
    try:
        objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
        cmds = [[cc, *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s),
                 "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max(1, min(len(cmds), os.cpu_count() or 1))) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB_PATH + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
