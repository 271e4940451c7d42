"""The oracle's own C under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.c is built by gcc with both sanitizers (any report aborts) and the
oracle's pins (tests/test_oracle.py) are run on that build in a child process:
an out-of-bounds index, a signed overflow in an offset or a bad shift in the
oracle would fail here even where its values happen to agree with the pins.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", lib,
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = {**os.environ, "RATTN_ORACLE_LIB": lib, "LD_PRELOAD": asan,
           "ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"}
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle.py")], capture_output=True, text=True,
                       env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
