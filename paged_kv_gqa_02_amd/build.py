"""Build libpaged_attn.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", name) for name in ("paged_attn.hip", "decode.hip", "append.hip", "staged.hip",
                                                      "spec_sample.hip")]
LIB = os.path.join(PKG, "libpaged_attn.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-Wall",
    # no packed fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# The LDS-staged kernel never feeds a NaN to a min / max (dead keys are masked
# by index before the row max, dead V rows zeroed), so its max reductions need
# no NaN quieting: relaxed NaN handling and the non-IEEE mode drop those moves.
FILE_FLAGS = {"staged.hip": ["-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee"]}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in res.stderr.splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    return err


# Host code only (the argument checks, the launch plan, the C ABI): sanitizer
# builds for the CPU tests, every finding fatal.  The device code is built as
# usual.  The sanitizer runtime is not linked in; the process that loads such a
# build preloads clang's (host_sanitizer_runtime).  "address":
# AddressSanitizer and UndefinedBehaviorSanitizer; "thread": ThreadSanitizer.
HOST_SANITIZE_FLAGS = {
    "address": ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer"],
    "thread": ["-Xarch_host", "-fsanitize=thread", "-Xarch_host", "-fno-omit-frame-pointer"],
}
_RUNTIME = {"address": "asan", "thread": "tsan"}


def host_sanitizer_runtime(kind: str = "address"):
    """clang's shared runtime of this ROCm for the sanitizer `kind`, or None."""
    import glob
    name = f"libclang_rt.{_RUNTIME[kind]}-x86_64.so"
    hits = sorted(glob.glob(f"/opt/rocm/llvm/lib/clang/*/lib/linux/{name}"))
    return hits[-1] if hits else None


def build(verbose: bool = False, out: str = LIB, host_sanitize: str | None = None) -> str:
    """Compile every source to an object (each with its own flags), then link.
    host_sanitize: None, "address" or "thread" (a host-code sanitizer build)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmpdir = tempfile.mkdtemp(prefix="paged_attn_build_")
    san = HOST_SANITIZE_FLAGS[host_sanitize] if host_sanitize else []
    try:
        objs, notes = [], []
        for src in SRCS:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            extra = FILE_FLAGS.get(os.path.basename(src), [])
            notes.append(_run([hipcc, *HIPCC_FLAGS, *extra, *san, "-I", INCLUDE, "-c", src, "-o",
                               obj]))
            objs.append(obj)
        tmp = out + ".tmp"
        notes.append(_run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    if verbose:
        for n in notes:
            if n.strip():
                print(n, file=sys.stderr)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
