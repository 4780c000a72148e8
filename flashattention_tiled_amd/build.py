"""Build the HIP library (libfa2.so) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# the parts of the library, compiled as the one translation unit fa2_lib.hip
PARTS = [os.path.join(CSRC, f) for f in
         ("fa2_lib.hip", "fa2_runtime.hip", "fa2_fwd.hip", "fa2_splitkv.hip", "fa2_tile.h",
          "fa2_host.h", "fa2_combine.h", "fa2_plan.h", "fa2_fwd_fp8.hip")]
SOURCES = [os.path.join(CSRC, "fa2_lib.hip")]
# the files that hold the prefill kernel's (fa2_fwd_kernel's) code
PREFILL_KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("fa2_plan.h", "fa2_tile.h", "fa2_fwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa2.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are disabled for all device code. Matrix-core
# results are kept in VGPRs (not AGPRs): the online softmax rescales the
# output accumulator in place, and in the AGPR form the compiler copies the
# whole accumulator out and back on every loop iteration.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build_library(force: bool = True, extra_flags=None) -> str:
    """Compile csrc/fa2_lib.hip (which includes the other parts) into libfa2.so
    next to this file."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = [HIPCC, *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-o", tmp, *SOURCES]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


PROBE_SOURCE = os.path.join(CSRC, "fa2_probe.hip")
PROBE_LIB_PATH = os.path.join(PKG, "libfa2probe.so")


def build_probe(force: bool = True) -> str:
    """Compile the matrix-core ceiling probe (csrc/fa2_probe.hip), a
    measurement aid kept out of the attention library, into libfa2probe.so."""
    if force or not os.path.exists(PROBE_LIB_PATH):
        tmp = PROBE_LIB_PATH + ".tmp"
        cmd = [HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-o", tmp, PROBE_SOURCE]
        subprocess.run(cmd, check=True)
        os.replace(tmp, PROBE_LIB_PATH)
    return PROBE_LIB_PATH


TIMELINE_LIB_PATH = os.path.join(PKG, "libfa2_timeline.so")


def build_timeline(force: bool = True) -> str:
    """Compile the library's sources with -DFA2_TIMELINE, in which every
    prefill workgroup records clock stamps (include/fa2_timeline.h; a
    measurement aid, read by timeline.py), into libfa2_timeline.so."""
    if force or not os.path.exists(TIMELINE_LIB_PATH):
        tmp = TIMELINE_LIB_PATH + ".tmp"
        cmd = [HIPCC, *HIP_FLAGS, "-DFA2_TIMELINE", "-I", INCLUDE, "-o", tmp, *SOURCES]
        subprocess.run(cmd, check=True)
        os.replace(tmp, TIMELINE_LIB_PATH)
    return TIMELINE_LIB_PATH


# the files that hold the split-KV kernels' code (partial and combine)
SPLITKV_KERNEL_SOURCES = [os.path.join(CSRC, f) for f in
                          ("fa2_plan.h", "fa2_tile.h", "fa2_combine.h", "fa2_splitkv.hip")]
# the files that hold the FP8 prefill kernel's code
FP8_KERNEL_SOURCES = [os.path.join(CSRC, f) for f in
                      ("fa2_plan.h", "fa2_tile.h", "fa2_fwd.hip", "fa2_fwd_fp8.hip")]


def sources_sha(paths) -> str:
    """SHA-256 over source files (name and bytes of each), which keys
    measurements taken of a kernel to the code they measured."""
    h = hashlib.sha256()
    for path in paths:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def prefill_kernel_sha() -> str:
    """SHA-256 over the prefill kernel's source files (sources_sha)."""
    return sources_sha(PREFILL_KERNEL_SOURCES)


if __name__ == "__main__":
    print(build_library())
    print(build_probe())
