"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

oracle/sanitize_driver.c calls every oracle entry point on small ragged shapes with buffers of
exactly the documented sizes: fp32 and bf16, every activation, pooled and full outputs, every
general geometry (K in {1, 3, 5}, stride 1 or 2, each padding below K), sampled forms against
full ones, the GEMM chain and the epilogue-only functions. This test builds it together with
oracle.c using gcc's host sanitizers (nothing here is GPU code) and requires a clean run. A
read one element past a buffer, a signed index overflow or a misaligned access aborts the run.
Two such slips planted by hand were caught: a weight buffer one element short, and an
off-by-one tap loop in the 3x3 pre-activation sum.
"""
import os
import shutil
import subprocess

import pytest

ORACLE = os.path.join(os.path.dirname(__file__), "..", "oracle")


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    build = subprocess.run(
        [gcc, "-O1", "-g", "-std=c11", "-Wall", "-Wno-unknown-pragmas", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(ORACLE, "oracle.c"),
         os.path.join(ORACLE, "sanitize_driver.c"), "-lm", "-o", exe],
        stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if build.returncode != 0 and "sanitize" in build.stdout and "cannot find" in build.stdout:
        pytest.skip("sanitizer runtime not available: " + build.stdout[-300:])
    assert build.returncode == 0, build.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300, env=env)
    assert run.returncode == 0 and "clean" in run.stdout, run.stdout[-4000:]
