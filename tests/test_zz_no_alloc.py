"""The entry point that allocates nothing: attn_sink_decode_paged_static.

For callers that cannot allocate device memory (code under HIP graph
capture, tight serving loops, harnesses that forbid hipMalloc), split paged
decode + merge runs with its partial states in the library's static device
array.  Called through the C ABI, its output must equal, bit for bit, that of
attn_sink_decode_paged (split) + attn_sink_merge on the same inputs, and
match the fp64 oracle, on two calls in a row with the second smaller than
the first; work too large for the array is refused before anything runs.
"""
import pytest
import torch

import oracle
import workloads
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")


def _dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _reference(lib, d, splits):
    pm, pd, po = lib.attn_sink_decode_paged(d["q"], d["k_cache"], d["v_cache"],
                                            d["page_table"], d["kv_lens"], d["sinks"],
                                            d["group"], d["sm_scale"], splits)
    out = torch.full_like(d["q"], NAN)
    lib.attn_sink_merge(pm, pd, po, out=out, out_dtype=d["q"].dtype)
    return out


def _static(lib, d, splits):
    out = torch.full_like(d["q"], NAN)
    lib.attn_sink_decode_paged_static(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                      d["kv_lens"], d["sinks"], d["group"], d["sm_scale"],
                                      splits, out=out)
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_static_decode_matches_allocating_path_twice(lib, dtype):
    big = workloads.decode_inputs([3000, 1, 700, 0, 4097, 64], hq=16, hkv=2, dtype=dtype,
                                  seed=5, sink_std=1.5)
    small = workloads.decode_inputs([33, 250], hq=8, hkv=1, dtype=dtype, seed=6,
                                    sink_std=1.5)
    for d, splits in ((big, 9), (small, 3)):
        dd = _dev(d)
        got = _static(lib, dd, splits)
        ref = _reference(lib, dd, splits)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), ref.cpu()), "static != decode + merge (S=%d)" % splits
        assert_close(got.cpu(), oracle.decode_paged(d["q"], d["k_cache"], d["v_cache"],
                                                    d["page_table"], d["kv_lens"],
                                                    d["sinks"], d["group"], d["sm_scale"]),
                     dtype, "static decode S=%d" % splits)


def test_static_decode_unsplit_and_split_decode_workload(lib):
    """The split-KV decode workload (B=4, kv_len 131072, 64 splits: 4.3 MB of
    partial states) fits the array; unsplit calls never touch it."""
    d = workloads.workload(4, device="cpu", cache_device=DEV)
    dd = _dev(d)
    got = _static(lib, dd, 64)
    ref = _reference(lib, dd, 64)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    one = _static(lib, dd, 1)
    plain = lib.attn_sink_decode_paged(dd["q"], dd["k_cache"], dd["v_cache"], dd["page_table"],
                                       dd["kv_lens"], dd["sinks"], 8, dd["sm_scale"], 1)
    torch.cuda.synchronize()
    assert torch.equal(one, plain)


def test_static_decode_refuses_work_beyond_the_array(lib):
    d = _dev(workloads.decode_inputs([40] * 64, hq=64, hkv=8, dtype=torch.bfloat16, seed=7))
    out = torch.full_like(d["q"], NAN)
    with pytest.raises(lib.AttnSinkError, match="static scratch"):
        lib.attn_sink_decode_paged_static(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                          d["kv_lens"], d["sinks"], 8, 0.125, 128, out=out)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(out.float()))
