"""Build the gfx950 HIP library in-tree with hipcc (no JIT, no torch extension).

Every HIP object is compiled with packed-fp32 instructions disabled, so the
compiler never emits the packed fp32 add/mul/fma forms.

The build also asks the compiler for its per-kernel resource report
(registers, scratch, spills) and refuses a library in which any kernel uses
scratch memory.  The bf16 prefill kernel's direct-to-LDS ring waits for its
own loads with hand-counted vector-memory counters; those counts are right
only while no other vector-memory instruction -- a scratch spill is one --
is in flight in the loop, so a spilling build would race silently instead of
failing.
"""
from __future__ import annotations

import os
import re
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
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"

_REMARK = re.compile(r"remark:\s+(Function Name|[A-Za-z][A-Za-z ]*?)(?: \[[^\]]*\])?:\s*(\S+)\s*"
                     r"\[-Rpass-analysis=kernel-resource-usage\]")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def parse_resource_report(text: str) -> dict:
    """{mangled kernel name: {field: int}} from the compiler's
    kernel-resource-usage remarks (fields such as 'VGPRs', 'AGPRs',
    'ScratchSize', 'VGPRs Spill', 'SGPRs Spill', 'Occupancy')."""
    kernels, cur = {}, None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = kernels.setdefault(val, {})
        elif cur is not None:
            try:
                cur[key] = int(val)
            except ValueError:
                cur[key] = val
    return kernels


def scratch_users(kernels: dict) -> list:
    """Kernels that use scratch memory or spill registers."""
    bad = []
    for name, f in kernels.items():
        if (f.get("ScratchSize", 0) or f.get("VGPRs Spill", 0) or f.get("SGPRs Spill", 0)
                or f.get("Dynamic Stack") == "True"):
            bad.append(name)
    return bad


def compile_library(out_path: str, src: str = SRC, extra_flags=()) -> dict:
    """Compile `src` into the shared library `out_path`; return the resource
    report.  Raises RuntimeError if hipcc fails or if any kernel uses
    scratch memory or spills."""
    cmd = [hipcc(), *HIPCC_FLAGS, RESOURCE_FLAG, *extra_flags, "-I", INCLUDE, src, "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    kernels = parse_resource_report(res.stderr)
    if not kernels:
        raise RuntimeError("hipcc printed no kernel resource report:\n%s" % res.stderr[-2000:])
    bad = scratch_users(kernels)
    if bad:
        raise RuntimeError("kernels use scratch memory or spill registers (the hand-counted "
                           "memory waits would race): %s" % ", ".join(
                               "%s %s" % (n, kernels[n]) for n in bad))
    return kernels


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile csrc/attn_sink.hip into the package directory; returns the path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    try:
        kernels = compile_library(tmp, extra_flags=extra_flags)
    except RuntimeError:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise
    if verbose:
        for name, f in sorted(kernels.items()):
            print(name, f)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
