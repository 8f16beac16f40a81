"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: tests/sanitize/
oracle_driver.c calls every oracle function over the parameters' edge cases (no tokens, one
token, a window covering everything, no and full eviction, 4-bit budgets, many heads) and
random shapes and rows (zeros, tiny, saturating, huge values); a sanitizer report aborts the
run. Skipped where the compiler has no sanitizer runtime. CPU only."""
import os
import shutil
import subprocess

import pytest

from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_clean_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
           os.path.join(HERE, "sanitize", "oracle_driver.c"), oracle_build.SRC, "-o", exe, "-lm"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0:
        if "asan" in b.stderr or "ubsan" in b.stderr or "sanitize" in b.stderr:
            pytest.skip("no sanitizer runtime: " + b.stderr[-200:])
        raise AssertionError(b.stderr)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "oracle driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
