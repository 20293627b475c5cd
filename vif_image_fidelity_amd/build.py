"""Builds libvif_amd.so (the C-ABI library of include/vif.h and
include/fssim.h) in-tree.

  python -m vif_image_fidelity_amd.build

hipcc cross-compiles for gfx950 without a GPU.  The flags fix every rounding
of the arithmetic: no contraction into fused multiply-adds, correctly
rounded fp32 division, IEEE denormals, no fast-math (ADR-1444 "float_vif_hip
runs the arithmetic of the CUDA twin ...", Context), and packed-fp32
instructions disabled.  Sources are rebuilt every call.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvif_amd.so")

SOURCES = ["vif_kernels.hip", "vif_selftest.hip", "vif_api.cpp",
           "vif_taps.cpp", "vif_options.cpp", "vif_rows.cpp", "vif_noalloc.hip",
           "fssim_kernels.hip",
           "fssim_api.cpp", "fssim_taps.cpp"]

ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-builtin-exp",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


EXAMPLE_SRC = os.path.join(CSRC, "score_raw.c")
EXAMPLE = os.path.join(HERE, "score_raw")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_example(verbose=False):
    """Compile score_raw.c, a plain C caller of the library's C ABI (gcc,
    C11), against the freshly built library."""
    tmp = EXAMPLE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), "-o", tmp, EXAMPLE_SRC,
           "-L", HERE, "-lvif_amd", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("gcc failed building %s" % EXAMPLE)
    os.replace(tmp, EXAMPLE)
    return EXAMPLE


def build(verbose=False):
    """Compile every source into vif_image_fidelity_amd/libvif_amd.so, then
    the C example that calls it."""
    tmp = LIB + ".tmp%d" % os.getpid()
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = (["hipcc"] + FLAGS + ["-shared", "-o", tmp] + srcs +
           ["-I", os.path.join(ROOT, "include")])
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB)
    os.replace(tmp, LIB)
    build_example(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
