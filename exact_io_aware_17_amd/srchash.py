"""Hash of the library's sources (csrc/ and include/), stamped into libfa.so
at build time so that a library built from other sources is never loaded."""
from __future__ import annotations

import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE_DIRS = [os.path.join(HERE, "csrc"), os.path.join(os.path.dirname(HERE), "include")]


def source_hash() -> str:
    """First 16 hex digits of SHA-256 over every source file's name and bytes."""
    h = hashlib.sha256()
    for d in SOURCE_DIRS:
        for name in sorted(os.listdir(d)):
            if not name.endswith((".hip", ".h", ".cpp")):
                continue
            h.update(name.encode())
            h.update(b"\0")
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
            h.update(b"\0")
    return h.hexdigest()[:16]
