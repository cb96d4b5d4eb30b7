"""The C oracle's own pins, run against a build of the oracle instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; gcc).

Any out-of-bounds access, use after free, signed overflow, misaligned load
or other undefined behaviour in ngram_oracle.c aborts the run: UBSan is built
with -fno-sanitize-recover, and the sanitizer runtime is preloaded into the
child interpreter so that the instrumented library can load.  Leak checks are
off (the interpreter itself keeps memory until exit)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ngram_oracle.c")
PINS = ["tests/test_oracle_hash.py", "tests/test_oracle_forward.py", "tests/test_oracle_grad.py",
        "tests/test_oracle_step.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = str(tmp_path / "libngram_oracle_asan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared", "-fPIC",
                           SRC, "-o", lib, "-lm"])
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", NGRAM_ORACLE_LIB=lib)
    check = ("import oracle, sys; p = oracle.lib()._name; print(p); "
             f"sys.exit(0 if p == {lib!r} else 3)")
    r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr   # the instrumented build is the one loaded
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
