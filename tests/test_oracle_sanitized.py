"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle library is rebuilt with -fsanitize=address,undefined (host code,
any report fatal) and every oracle pin test runs against it in a child
process, with the sanitizer runtime preloaded into the interpreter.  A memory
error or an undefined operation anywhere in the oracle's arithmetic, decoders
or packers the pins exercise fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_clean_under_asan_and_ubsan(tmp_path):
    import oracle
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    lib = oracle.build(str(tmp_path / "libqref_san.so"), sanitize=True)
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    pins = [p for p in pins if not p.endswith("test_oracle_sanitized.py")]
    env = dict(os.environ, QREF_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the mutant builds inside the pins stay unsanitized (they only need to fail pins)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
