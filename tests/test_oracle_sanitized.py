"""The oracle's pin suites run against a build of oracle.c with AddressSanitizer
and UndefinedBehaviorSanitizer (gcc, host code only): any out-of-bounds access,
use of freed memory, signed overflow, invalid shift or misaligned access in
the oracle aborts the run."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_sampler_pins.py",
          "tests/test_oracle_parallel.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    env = dict(os.environ)
    env["ORACLE_LIB"] = lib
    # the sanitizer runtime has to come first; anything already preloaded stays
    env["LD_PRELOAD"] = ":".join(x for x in (asan, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"   # the interpreter's own allocations
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    probe = subprocess.run([sys.executable, "-c", "import oracle; oracle._load(); "
                            "print(open('/proc/self/maps').read().count('liboracle_asan.so') > 0)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip() == "True", probe.stdout + probe.stderr   # the sanitized build ran
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", *SUITES], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, tail
    assert "runtime error" not in res.stderr, tail
