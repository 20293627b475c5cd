"""The library's host-only code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): the library's own sources and flags,
with the host side of every translation unit instrumented (the GPU code is
unchanged), and a plain C driver (sanitize_host_driver.c) calling the entry
points that need no device: the strip geometry over every strip boundary of
small frames, the host sums and scores from row sums under every option path,
the tap generators, the constructors' refusals of bad geometry and options,
and the error strings.  A memory error or undefined behaviour makes the
driver exit non-zero."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")

SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG),
                    reason="needs hipcc and ROCm's clang")
def test_host_code_clean_under_asan_ubsan(tmp_path):
    from vif_image_fidelity_amd import build
    lib = str(tmp_path / "libvif_amd.so")
    srcs = [os.path.join(build.CSRC, s) for s in build.SOURCES]
    r = subprocess.run(["hipcc"] + build.FLAGS + SANITIZE_HOST +
                       ["-shared", "-o", lib] + srcs +
                       ["-I", os.path.join(ROOT, "include")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "sanitize_host_driver")
    r = subprocess.run([CLANG, "-std=c11", "-O1", "-g",
                        "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROCM, "include"), "-o", exe,
                        os.path.join(HERE, "sanitize_host_driver.c"),
                        "-L", str(tmp_path), "-lvif_amd",
                        "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        "-Wl,-rpath," + str(tmp_path),
                        "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # leak checking is off: the HIP runtime keeps its own allocations
    # until exit
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ok" in r.stdout
