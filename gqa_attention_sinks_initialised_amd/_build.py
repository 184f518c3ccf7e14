"""Build the gfx950 HIP library in-tree with hipcc (no JIT, no torch extension).

Every HIP object is compiled with packed-fp32 instructions disabled, so the
compiler never emits the packed fp32 add/mul/fma forms.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn_sink.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattnsink.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile csrc/attn_sink.hip into the package directory; returns the path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
