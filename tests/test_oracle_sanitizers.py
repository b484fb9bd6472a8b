"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, CPU only) and run over every entry point on small, ragged and edge
shapes (tests/oracle_sanitize_driver.c): no out-of-bounds access, no use of
freed memory, no undefined behaviour (the build aborts on the first report)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # (verify_asan_link_order=0: the sanitizer runtime need not be the first
    # library of the process when the environment preloads one of its own)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
