"""The host half of libpaged_attn (argument checks, launch plan, C ABI) built
with AddressSanitizer and UndefinedBehaviorSanitizer (clang, -Xarch_host: the
device code is built as usual), and the ABI, binding and concurrent-calls
suites run against it in a child process with clang's runtime preloaded: an
out-of-bounds access, a use of freed memory, an invalid enum value, a signed
overflow or a bad shift on any host path those suites reach aborts the run.
A second build with ThreadSanitizer runs the concurrent-calls suite."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi.py", "tests/test_binding_checks.py", "tests/test_host_threads.py"]


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "paged_attn_build", os.path.join(ROOT, "paged_kv_gqa_02_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_suites_under_host_asan_and_ubsan(tmp_path):
    b = _build_module()
    runtime = b.host_sanitizer_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    lib = b.build(out=str(tmp_path / "libpaged_attn_hsan.so"), host_sanitize="address")
    env = dict(os.environ)
    env["PAGED_ATTN_LIB"] = lib
    env["LD_PRELOAD"] = ":".join(x for x in (runtime, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"     # the interpreter's own allocations
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    probe = subprocess.run([sys.executable, "-c", "import paged_kv_gqa_02_amd; "
                            "print(open('/proc/self/maps').read().count('libpaged_attn_hsan.so') > 0)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip().endswith("True"), probe.stdout + probe.stderr   # the sanitized build ran
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", *SUITES], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, tail
    assert "runtime error" not in res.stderr, tail


def test_threaded_host_calls_under_thread_sanitizer(tmp_path):
    """The same host half built with ThreadSanitizer; the concurrent-calls
    suite (eight threads in the C ABI at once) and the ABI suite run against
    it: a data race between the library's threads aborts the run."""
    b = _build_module()
    runtime = b.host_sanitizer_runtime("thread")
    if runtime is None:
        pytest.skip("clang's ThreadSanitizer runtime is not installed")
    lib = b.build(out=str(tmp_path / "libpaged_attn_tsan.so"), host_sanitize="thread")
    env = dict(os.environ)
    env["PAGED_ATTN_LIB"] = lib
    env["LD_PRELOAD"] = ":".join(x for x in (runtime, os.environ.get("LD_PRELOAD", "")) if x)
    env["TSAN_OPTIONS"] = "halt_on_error=1"
    probe = subprocess.run([sys.executable, "-c", "import paged_kv_gqa_02_amd; "
                            "print(open('/proc/self/maps').read().count('libpaged_attn_tsan.so') > 0)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip().endswith("True"), probe.stdout + probe.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", "tests/test_host_threads.py", "tests/test_abi.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "WARNING: ThreadSanitizer" not in res.stderr, tail
