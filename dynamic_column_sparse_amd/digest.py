"""Digest of the library's sources (every file under ``csrc/`` and ``include/``).

``build.py`` compiles it into ``libchipmunk.so`` (``chipmunk_source_digest()``);
``lib.py`` refuses a library whose digest differs from the sources beside it,
so the code that runs is the code in the tree.
"""
from __future__ import annotations

import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DIRS = (os.path.join(HERE, "csrc"), os.path.join(ROOT, "include"))
SUFFIXES = (".hip", ".h", ".cpp", ".hpp")


def source_files() -> list:
    out = []
    for d in DIRS:
        for f in sorted(os.listdir(d)):
            if f.endswith(SUFFIXES):
                out.append(os.path.join(d, f))
    return out


def source_digest() -> str:
    """First 16 hex digits of SHA-256 over (relative path, contents) of every source."""
    h = hashlib.sha256()
    for p in source_files():
        h.update(os.path.relpath(p, ROOT).encode() + b"\0")
        with open(p, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]
