"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, no recovery) and driven through every function on small and edge-case
shapes (empty M, N or K, one element, a ragged K) by oracle_sanitize_main.c.
An out-of-bounds access, a leak or undefined behaviour in the oracle makes
the test program exit non-zero.  CPU only; the sanitizers are host-code tools."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-Werror",
           "-I" + os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "oracle_sanitize_main.c"),
           os.path.join(ROOT, "oracle", "sq_oracle.c"), "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("gcc has no sanitizer runtime here")
    assert build.returncode == 0, build.stderr
    # a library preloaded into every process would come before the ASan
    # runtime; the link-order check is off so that it does not refuse to run
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle sanitizer run ok" in run.stdout
