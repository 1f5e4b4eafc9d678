"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a build
of moe_oracle.c with both (host code only: the oracle is plain C on the
CPU), and the oracle's pin tests run against it in a child process (the ASan
runtime preloaded, since the interpreter itself is not instrumented).  Any
out-of-bounds access, use after free or undefined operation in the oracle
aborts the child and fails this test.  The pin that compares a second
compiler's build of the oracle is left out (it builds its own library)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime for gcc here")
    so = str(tmp_path / "liboracle_san.so")
    oracle.build(out=so, extra=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                "-fno-omit-frame-pointer", "-g"))
    env = dict(os.environ, BEF_ORACLE_LIB=so, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "not second_compiler",
                        os.path.join(ROOT, "tests", "test_oracle_codecs.py"),
                        os.path.join(ROOT, "tests", "test_oracle_layer.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    print(r.stdout.strip().splitlines()[-1])
