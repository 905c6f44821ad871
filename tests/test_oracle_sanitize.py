"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The pin suite (tests/test_oracle_pins.py) runs in a subprocess against a
build of oracle/kvq_oracle.c with -fsanitize=address,undefined and no
recovery, so an out-of-bounds access, a use after free, a signed overflow
or an invalid shift in the oracle ends the run with a report.  CPU only:
the sanitized library is host code built with gcc.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
SAN_FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_pins_pass_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libkvq_oracle_san.so")
    obuild.build(out=lib, extra_flags=SAN_FLAGS)
    env = dict(os.environ, KVQ_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=97",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in out, out
    assert "runtime error:" not in out, out
    assert r.returncode == 0, out   # 97 / 98: a sanitizer report ended the run
