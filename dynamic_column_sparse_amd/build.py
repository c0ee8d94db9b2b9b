"""Build the HIP library ``libchipmunk.so`` in-tree for gfx950 with hipcc.

Each source compiles to an object under ``_build/`` (in parallel), then one
shared-library link.  Every call rebuilds everything, so the result always
matches the sources; the sources' digest is compiled in
(``chipmunk_source_digest()``) and checked when the library is loaded.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libchipmunk.so")

SOURCES = ["abi.cpp", "mlp.hip", "topk.hip", "attn.hip", "writeback.hip", "step.hip", "quant.hip", "noalloc.hip", "check.hip"]
ARCH = "gfx950"


def _digest() -> str:
    # Loaded by path so that `python build.py` works without the package import
    # (which would load the library being rebuilt).
    import importlib.util
    spec = importlib.util.spec_from_file_location("_chipmunk_digest", os.path.join(HERE, "digest.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.source_digest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libchipmunk.so)")


def common_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
        # packed fp32 vector ops stay off in all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), f'-DCHIPMUNK_SOURCE_DIGEST="{digest}"', "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    digest = _digest()
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} (sources {digest})")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
