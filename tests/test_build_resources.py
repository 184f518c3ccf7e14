"""The library's kernels use no scratch memory (CPU only: hipcc cross-compiles).

The bf16 prefill kernel waits for its direct-to-LDS loads with hand-counted
vector-memory counters; those counts hold only while no other
vector-memory instruction (such as a register spill to scratch) is in flight
in its loop.  The build therefore reads the compiler's per-kernel resource
report and refuses any kernel with scratch or spills; these tests check
that the report is read, that the product library passes, and that a kernel
which does use scratch is refused.
"""
import pytest

from gqa_attention_sinks_initialised_amd import _build

SPILLING_KERNEL = r"""
#include <hip/hip_runtime.h>
extern "C" __global__ void uses_scratch(float* out, int n) {
  float a[256];
  for (int i = 0; i < 256; ++i) a[i] = out[i * n + threadIdx.x];
  out[threadIdx.x] = a[(threadIdx.x * 7 + n) & 255];
}
"""


@pytest.fixture(scope="module")
def report(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("lib") / "libattnsink.so")
    return _build.compile_library(out)


def test_every_kernel_instance_is_reported(report):
    names = list(report)
    for kind, n in (("prefill_kernel", 12), ("decode_kernel", 4), ("merge_kernel", 10)):
        assert sum(kind in x for x in names) == n, (kind, names)


def test_no_kernel_uses_scratch_or_spills(report):
    assert _build.scratch_users(report) == []
    for name, f in report.items():
        assert f["ScratchSize"] == 0 and f["VGPRs Spill"] == 0 and f["SGPRs Spill"] == 0, name


def test_bf16_prefill_keeps_two_waves_per_simd(report):
    """The direct-to-LDS ragged bf16 instances (the kernel behind the prefill
    figures) must fit two waves per SIMD."""
    for name, f in report.items():
        if "prefill_kernelILi1ELi2ELi4ELb0E" in name:
            assert f["Occupancy"] >= 2 and f["VGPRs"] + f["AGPRs"] <= 256, (name, f)


def test_a_kernel_that_uses_scratch_is_refused(tmp_path):
    src = tmp_path / "spill.hip"
    src.write_text(SPILLING_KERNEL)
    with pytest.raises(RuntimeError, match="scratch"):
        _build.compile_library(str(tmp_path / "spill.so"), src=str(src))
