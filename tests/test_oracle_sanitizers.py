"""Both CPU oracles built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and run on edge geometries: 16x16 and odd frames at
every bit depth, tiny planes where the mirror reaches furthest, the IEEE
special cases of a zero noise variance, the option paths, and float SSIM
frames from 1x1 (the 11-tap window wraps the border many times) to factors 2
and 3 with odd sizes.  A memory error or undefined behaviour makes the
program exit non-zero.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracles_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off",
           "-fno-fast-math", "-fno-builtin", "-msse2", "-mfpmath=sse",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", ORACLE, "-o", exe,
           os.path.join(HERE, "sanitize_driver.c"),
           os.path.join(ORACLE, "vif_oracle.c"),
           os.path.join(ORACLE, "fssim_oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ok" in r.stdout
