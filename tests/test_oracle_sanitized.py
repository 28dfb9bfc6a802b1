"""The oracle's pins again, against an AddressSanitizer + UndefinedBehaviorSanitizer build of
the same C source (CPU only): any out-of-bounds access, use after free, signed overflow or
other undefined behaviour in the oracle fails the run.  A planted out-of-bounds call (an
output array one row short) must be caught, which shows the sanitizers are live."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_build.py", "tests/test_oracle_greedy.py", "tests/test_oracle_sample.py",
        "tests/test_oracle_commit.py", "tests/test_oracle_lm_head.py", "tests/test_oracle_best_first.py",
        "tests/test_oracle_attention.py"]


def _runtime(name):
    try:
        path = subprocess.check_output(["gcc", "-print-file-name=" + name], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not shutil.which("gcc") or not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not available")
    lib = str(tmp_path_factory.mktemp("san") / "libtmv_oracle_san.so")
    subprocess.check_call(["gcc", "-std=gnu99", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
                           "-fPIC", "-shared", "-o", lib, os.path.join(ROOT, "oracle", "tmv_oracle.c"), "-lm"])
    env = dict(os.environ, TMV_ORACLE_LIB=lib, LD_PRELOAD=asan + " " + ubsan,
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env


def test_oracle_pins_under_sanitizers(sanitized):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS], cwd=ROOT,
                       env=sanitized, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def test_planted_overflow_is_caught(sanitized):
    code = """
import ctypes, numpy as np, oracle
lib = oracle._load()
B, M, D = 1, 6, 3
parents = np.array([[0, 0, 1, 1, 2, 2, 3]], np.int32)
n = np.array([6], np.int32)
anc = np.zeros((B, M, D + 1), np.int32)      # one row short: rows 0..M need M + 1
depth = np.zeros((B, M + 1), np.int32)
st = np.zeros(B, np.int32)
p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
lib.tmvref_build_ancestors(B, M, D, 0, p(parents), None, p(n), p(anc), p(depth), p(st))
print("not caught")
"""
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stdout, r.stderr[-2000:])
