"""The C ABI's host code (argument validation, workspace sizing, handle
creation and error paths) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer, and driven by tests/sanitizer/abi_driver.cpp on
this machine (no GPU needed: creation reports the missing device). The
sanitizers instrument the host code only (the gfx950 kernels are built as
usual and never run here); any memory error, signed overflow or other
undefined behaviour in the host paths aborts the driver."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressive_memory_transformers_segment_amd", "csrc")
SOURCES = ["infini_attn.hip", "segment_scan.hip", "segment_scan_mfma.hip", "fused_bf16.hip",
           "fused_f32.hip", "decode.hip", "block.hip", "backward.hip"]
ROCM = "/opt/rocm"


def _tool(name):
    for cand in (os.path.join(ROCM, "bin", name), os.path.join(ROCM, "llvm", "bin", name)):
        if os.path.exists(cand):
            return cand
    return shutil.which(name)


def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    hipcc, clang = _tool("hipcc"), _tool("clang++")
    if not hipcc or not clang:
        pytest.skip("ROCm toolchain not found")
    # The sanitizers apply to the host code only (each flag after -Xarch_host).
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory(prefix="ia_asan_") as tmp:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            procs.append(subprocess.Popen(
                [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 *(["-fno-honor-nans", "-mno-amdgpu-ieee"] if src == "fused_bf16.hip" else []),
                 "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src),
                 "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        for pr in procs:
            out, _ = pr.communicate()
            assert pr.returncode == 0, out
        drv = os.path.join(tmp, "abi_driver")
        link = subprocess.run(
            [clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-I", os.path.join(ROOT, "include"),
             os.path.join(ROOT, "tests", "sanitizer", "abi_driver.cpp"), *objs,
             "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
             "-lamdhip64", "-lrocblas", "-o", drv],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert link.returncode == 0, link.stdout
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
                   HIP_VISIBLE_DEVICES="")
        run = subprocess.run([drv], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                             env=env, timeout=120)
        print(run.stdout)
        assert run.returncode == 0, run.stdout
        assert "runtime error" not in run.stdout and "AddressSanitizer" not in run.stdout
