"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
oracle.c is compiled with gcc -fsanitize=address,undefined (host code only)
and the oracle pins run against that build in a child process, which fails
on any out-of-bounds access, use after free or undefined operation."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-fast-math",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fPIC", "-shared", "-pthread", os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"],
                   check=True)
    env = dict(os.environ)
    env["MOE_ORACLE_LIB"] = lib
    # the sanitizer runtime must come first; anything already preloaded stays
    env["LD_PRELOAD"] = " ".join(p for p in (asan, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized oracle pins failed (exit {r.returncode}):\n{tail}"
    assert "passed" in r.stdout and "liboracle_san" not in r.stderr, tail
