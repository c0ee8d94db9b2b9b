"""Host-sanitized build of libchipmunk.so for the CPU tests of the C ABI.

Compiles the same sources as dynamic_column_sparse_amd/build.py into
_build/sanitized/libchipmunk.so with AddressSanitizer and UndefinedBehavior-
Sanitizer on the HOST code only (the validation, launch and timer code of the
ABI; every -fsanitize flag is applied with -Xarch_host, device code is built
as usual), then runs tests/test_abi_cpu.py against it in a child process with
the sanitizer runtime preloaded.  Any sanitizer report fails the run.

    python tests/sanitized_build.py
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from dynamic_column_sparse_amd import build as B  # noqa: E402

OUT = os.path.join(ROOT, "_build", "sanitized")
LIB = os.path.join(OUT, "libchipmunk.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("the clang AddressSanitizer runtime was not found under /opt/rocm/llvm")
    return cands[-1]


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    digest = B._digest()

    def one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [B.hipcc(), *B.common_flags(), *SAN, f'-DCHIPMUNK_SOURCE_DIGEST="{digest}"', "-c",
               os.path.join(B.CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
        return obj

    with ThreadPoolExecutor(min(len(B.SOURCES), 8)) as ex:
        objs = list(ex.map(one, B.SOURCES))
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    return LIB


def run_abi_tests() -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["CHIPMUNK_LIBRARY"] = LIB
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_cpu.py")]
    return subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT)


if __name__ == "__main__":
    build()
    r = run_abi_tests()
    print(r.stdout[-3000:], r.stderr[-3000:])
    sys.exit(r.returncode)
