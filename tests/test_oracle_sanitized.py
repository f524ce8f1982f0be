"""The oracle's pins rerun against an AddressSanitizer + UndefinedBehaviorSanitizer
build of the oracle (gcc, CPU only; oracle/build.py --sanitized).  A planted
heap overflow in a separate scratch program, built with the same flags, shows
that the sanitizers are live in this environment."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    if p.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("the AddressSanitizer runtime is not installed")
    return path


def test_sanitizers_catch_a_planted_heap_overflow(tmp_path):
    _asan_runtime()
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\nint main(void) {\n  volatile int* p = malloc(4 * sizeof(int));\n"
                   "  int s = p[4];  /* one past the end */\n  free((void*)p);\n  return s & 0;\n}\n")
    exe = tmp_path / "overflow"
    flags = [f for f in ob.SAN_FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run(["gcc", *flags, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    # UBSan's object-size check or ASan's redzone stops it, whichever runs first
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr or "insufficient space" in r.stderr


def test_oracle_pins_under_address_and_ub_sanitizers():
    asan = _asan_runtime()
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    ob.build(sanitized=True)
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    tests = [t for t in tests if not t.endswith("test_oracle_sanitized.py")]
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", ORACLE_SANITIZED="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
