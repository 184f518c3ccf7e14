"""Host-side checks of the C ABI (no GPU needed, no compute call).

The library must load, export every entry point that include/attn_sink.h
declares, and reject bad arguments with the documented status before it
touches the GPU.
"""
import ctypes
import os
import re

import pytest

import gqa_attention_sinks_initialised_amd as m

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "attn_sink.h")

OK, INVALID, UNSUPPORTED, LAUNCH = 0, 1, 2, 3


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_sink_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(m.LIB_PATH):
        m.build()
    return m.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("attn_sink_prefill", "attn_sink_prefill_partials", "attn_sink_prefill_paged",
              "attn_sink_decode_paged", "attn_sink_merge", "attn_sink_decode_paged_static",
              "attn_sink_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert set(_declared_functions()) == set(m.SYMBOLS)


def test_status_strings(L):
    assert m.status_string(OK) == "ok"
    assert m.status_string(INVALID) == "invalid argument"
    assert m.status_string(UNSUPPORTED) == "unsupported configuration"
    assert m.status_string(LAUNCH) == "kernel launch failed"
    assert "static scratch" in m.status_string(4)
    assert m.status_string(99) == "unknown status"


# Fake, 16-byte aligned, never-dereferenced device addresses: every call below
# must fail validation before anything is launched.
A = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10008)  # 8-byte aligned only


def _prefill(L, **kw):
    args = dict(q=A, k=A, v=A, sinks=A, cq=A, ck=A, batch=1, tq=4, tkv=4, maxq=4, hkv=1,
                group=1, dim=64, scale=0.125, causal=1, dtype=1, out=A, stream=None)
    args.update(kw)
    return L.attn_sink_prefill(*args.values())


def _decode(L, **kw):
    args = dict(q=A, kc=A, vc=A, pt=A, lens=A, sinks=A, batch=1, maxp=4, npages=4, hkv=1,
                group=1, dim=64, page=16, scale=0.125, dtype=1, splits=1, pm=None, pd=None,
                po=None, out=A, stream=None)
    args.update(kw)
    return L.attn_sink_decode_paged(*args.values())


def _prefill_partials(L, **kw):
    args = dict(q=A, k=A, v=A, sinks=A, cq=A, ck=A, batch=1, tq=4, tkv=4, maxq=4, hkv=1,
                group=1, dim=64, scale=0.125, causal=1, dtype=1, splits=3, pm=A, pd=A, po=A,
                stream=None)
    args.update(kw)
    return L.attn_sink_prefill_partials(*args.values())


def _prefill_paged(L, **kw):
    args = dict(q=A, kc=A, vc=A, pt=A, cq=A, lens=A, sinks=A, batch=1, tq=4, maxq=4, maxp=4,
                npages=4, hkv=1, group=1, dim=64, page=16, scale=0.125, causal=1, dtype=1,
                splits=1, pm=None, pd=None, po=None, out=A, stream=None)
    args.update(kw)
    return L.attn_sink_prefill_paged(*args.values())


def _merge(L, **kw):
    args = dict(pm=A, pd=A, po=A, batch=1, hq=1, splits=2, dim=64, dtype=1, out=A, stream=None)
    args.update(kw)
    return L.attn_sink_merge(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(sinks=None), INVALID),
    (dict(k=None), INVALID), (dict(cq=None), INVALID),
    (dict(q=None, out=None, tq=0), OK), (dict(k=None, v=None, tkv=0, batch=0), OK),
    (dict(q=MIS), INVALID), (dict(batch=-1), INVALID), (dict(hkv=0), INVALID),
    (dict(group=0), INVALID), (dict(causal=2), INVALID), (dict(dtype=7), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=-1.0), INVALID),
    (dict(dim=128), UNSUPPORTED), (dict(group=65), UNSUPPORTED),
    (dict(tq=1 << 30, hkv=8, group=8), UNSUPPORTED),
    # nothing to do: accepted without a launch
    (dict(batch=0), OK), (dict(tq=0), OK), (dict(maxq=0), OK)])
def test_prefill_validation(L, kw, code):
    assert _prefill(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(pt=None), INVALID), (dict(splits=0), INVALID),
    (dict(kc=None), INVALID), (dict(kc=None, vc=None, npages=0, batch=0), OK),
    (dict(out=None), INVALID),                                  # splits == 1 needs out
    (dict(splits=4), INVALID),                                  # splits > 1 needs partials
    (dict(splits=4, pm=A, pd=A, po=MIS, out=None), INVALID),    # misaligned partial_o
    (dict(kc=MIS), INVALID), (dict(maxp=0), INVALID), (dict(npages=-1), INVALID),
    (dict(dtype=5), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(dim=32), UNSUPPORTED), (dict(page=32), UNSUPPORTED), (dict(group=17), UNSUPPORTED),
    (dict(maxp=1 << 28), UNSUPPORTED),
    (dict(batch=0), OK), (dict(batch=0, splits=3, pm=A, pd=A, po=A, out=None), OK)])
def test_decode_validation(L, kw, code):
    assert _decode(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(pm=None), INVALID), (dict(pd=None), INVALID), (dict(po=MIS), INVALID),
    (dict(splits=0), INVALID), (dict(splits=65537), INVALID), (dict(q=None), INVALID),
    (dict(k=None), INVALID), (dict(ck=None), INVALID), (dict(causal=3), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(dim=96), UNSUPPORTED),
    (dict(group=65), UNSUPPORTED), (dict(k=None, v=None, tkv=0, batch=0), OK),
    (dict(batch=0), OK), (dict(tq=0, q=None), OK), (dict(maxq=0), OK)])
def test_prefill_partials_validation(L, kw, code):
    assert _prefill_partials(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(pt=None), INVALID), (dict(lens=None), INVALID),
    (dict(cq=None), INVALID), (dict(kc=None), INVALID), (dict(out=None), INVALID),
    (dict(splits=0), INVALID), (dict(splits=4), INVALID),          # splits > 1 needs partials
    (dict(splits=4, pm=A, pd=A, po=MIS, out=None), INVALID), (dict(kc=MIS), INVALID),
    (dict(maxp=0), INVALID), (dict(npages=-1), INVALID), (dict(causal=-1), INVALID),
    (dict(dtype=2), INVALID), (dict(scale=0.0), INVALID),
    (dict(dim=32), UNSUPPORTED), (dict(page=8), UNSUPPORTED), (dict(group=80), UNSUPPORTED),
    (dict(maxp=1 << 27), UNSUPPORTED),
    (dict(npages=1 << 20, hkv=8, batch=0), OK),       # a 16 GiB cache is accepted
    (dict(kc=None, vc=None, npages=0, batch=0), OK), (dict(batch=0), OK),
    (dict(tq=0, q=None, out=None), OK),
    (dict(batch=0, splits=3, pm=A, pd=A, po=A, out=None), OK)])
def test_prefill_paged_validation(L, kw, code):
    assert _prefill_paged(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(pm=None), INVALID), (dict(out=None), INVALID), (dict(po=MIS), INVALID),
    (dict(splits=0), INVALID), (dict(hq=0), INVALID), (dict(dtype=3), INVALID),
    (dict(dim=16), UNSUPPORTED), (dict(batch=0), OK)])
def test_merge_validation(L, kw, code):
    assert _merge(L, **kw) == code


def test_binding_refuses_cpu_tensors(L):
    import torch
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(4, 1, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        m.attn_sink_prefill(q, k, k, torch.zeros(2), cu, cu, 4, 2)


TOO_LARGE = 4


def _decode_static(L, **kw):
    args = dict(q=A, kc=A, vc=A, pt=A, lens=A, sinks=A, batch=1, maxp=4, npages=4, hkv=1,
                group=1, dim=64, page=16, scale=0.125, dtype=1, splits=2, out=A, stream=None)
    args.update(kw)
    return L.attn_sink_decode_paged_static(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(out=MIS), INVALID),
    (dict(splits=0), INVALID), (dict(kc=MIS), INVALID), (dict(dtype=5), INVALID),
    (dict(dim=32), UNSUPPORTED), (dict(group=17), UNSUPPORTED),
    # 64 x 64 rows x 128 chunks of (64 + 2) floats: 138 MB > 16 MiB
    (dict(batch=64, hkv=8, group=8, splits=128), TOO_LARGE),
    (dict(batch=0, splits=3), OK), (dict(batch=0, splits=1), OK)])
def test_decode_static_validation(L, kw, code):
    """The no-alloc entry point rejects bad arguments, and work whose split
    states would not fit its static scratch array, before anything runs."""
    assert _decode_static(L, **kw) == code


class _FakeGpuTensor:
    """Stands in for a contiguous GPU tensor: _dev reads only these fields."""

    def __init__(self, device):
        self.device, self.is_cuda = device, True

    def is_contiguous(self):
        return True


def test_binding_requires_one_gpu_for_all_tensors():
    """The library launches on the stream's GPU with the tensors' addresses,
    so the binding refuses tensors spread over two GPUs before any call."""
    import torch
    a, b = torch.device("cuda:0"), torch.device("cuda:1")
    assert m._dev(_FakeGpuTensor(a), None, _FakeGpuTensor(a)) == a
    with pytest.raises(ValueError, match="same GPU"):
        m._dev(_FakeGpuTensor(a), _FakeGpuTensor(b))
    with pytest.raises(ValueError, match="on the GPU"):
        m._dev(torch.zeros(2))
