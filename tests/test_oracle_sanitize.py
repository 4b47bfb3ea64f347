"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc) and run through every function on small inputs by
tests/sanitize/oracle_driver.c.  Any out-of-bounds access, use after free,
leak, signed overflow or other undefined behaviour aborts the driver."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'oracle')}", "-o", str(exe),
           os.path.join(HERE, "sanitize", "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "mita_oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "cannot find" in r.stderr and "asan" in r.stderr:
        pytest.skip("gcc sanitizer runtimes are not installed")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "ok" in r.stdout
