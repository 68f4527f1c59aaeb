"""The float64 oracle and the input generator under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

oracle/selfcheck.c drives every oracle and generator function on small inputs
and checks facts that hold by construction (hand-built unpacking, s*q + b per
element, threaded decodes equal to the serial one, K = E, grouping counts, the
RMS closed form); the sanitizers report any out-of-bounds access, use after
free, leak or undefined behaviour on the way.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "selfcheck")
    cmd = ["gcc", "-g", "-O1", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-fopenmp",
           os.path.join(ROOT, "oracle", "selfcheck.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="3", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "selfcheck ok" in run.stdout
