"""Build libnvfp4.so (the HIP library behind include/nvfp4.h) in-tree for gfx950.

Usage: ``python -m bit_block_scaled_nvfp4_amd.build`` or ``build()`` from Python.  Every call
compiles; the objects go to ``bit_block_scaled_nvfp4_amd/_build`` and the library next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4.so")
# reference kernels the benchmark times beside the decode product (not part of the product's ABI)
CEILING_SRC = "ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libnvfp4_ceiling.so")

SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "gemm_skinny.hip", "gemm_stream.hip", "kv_cache.hip",
           "fake_quant.hip"]

ARCH = "gfx950"

# -ffp-contract=off and correctly rounded division: the encoder's binary32 operations must be
# exactly the ones its contract states (no fused multiply-add, IEEE division).
# -packed-fp32-ops off: packed FP32 arithmetic is not used on this target.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the packed-fp32 feature; that warning is expected
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source for gfx950, link libnvfp4.so (and the benchmark's reference kernels,
    libnvfp4_ceiling.so); return the path of libnvfp4.so."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    ceil_obj = os.path.join(BUILD, os.path.splitext(CEILING_SRC)[0] + ".o")
    cmds.append([hipcc, *flags, "-c", os.path.join(CSRC, CEILING_SRC), "-o", ceil_obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for lib, lib_objs in ((LIB, objs), (CEILING_LIB, [ceil_obj])):
        tmp = lib + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
