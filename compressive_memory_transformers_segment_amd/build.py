"""Build the gfx950 HIP library ``libinfini_attn.so`` in-tree with hipcc.

Usage: ``python -m compressive_memory_transformers_segment_amd.build``.
Every source is compiled for gfx950 only, with packed-fp32 instructions off.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libinfini_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["infini_attn.hip", "segment_scan.hip", "segment_scan_mfma.hip", "fused_bf16.hip",
           "fused_f32.hip", "decode.hip", "block.hip", "backward.hip"]
ARCH = "gfx950"

# Extra flags per source. The fused attention kernel runs with the IEEE mode
# bit off, so that max/min on MFMA results need no NaN-quieting instructions
# (NaN inputs are not supported on that path).
FILE_FLAGS = {"fused_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # CDNA packed fp32 (v_pk_*_f32) stays off in every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link the shared library. Returns its path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="infini_attn_build_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC,
                         "-c", os.path.join(CSRC, src), "-o", obj])
        with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib,
              "-lrocblas"])
        dst_tmp = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, dst_tmp)
        os.replace(dst_tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
