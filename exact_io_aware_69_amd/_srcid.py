"""Identity of the sources libfa.so is built from.

The SHA-256 (first 16 hex digits) of every HIP source and header under
``csrc/``, of ``include/``, and of the build script, each prefixed with its
relative path. ``build.py`` bakes it into the library (``fa_build_id()``);
``_lib.lib()`` recomputes it from the sources beside the library and refuses
a library built from other sources.
"""
from __future__ import annotations

import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def source_files() -> list:
    files = []
    csrc = os.path.join(PKG, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            files.append(os.path.join(csrc, name))
    inc = os.path.join(ROOT, "include")
    for name in sorted(os.listdir(inc)):
        if name.endswith(".h"):
            files.append(os.path.join(inc, name))
    files.append(os.path.join(PKG, "build.py"))
    return files


def source_id() -> str:
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode())
        h.update(b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]
