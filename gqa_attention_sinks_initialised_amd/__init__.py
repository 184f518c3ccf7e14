"""Grouped-query attention with per-head attention sinks on MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/attn_sink.h``.  The
functions carry the C names (``attn_sink_prefill``, ``attn_sink_decode_paged``,
``attn_sink_merge``); they only check and marshal arguments -- every step of
the computation runs in the HIP kernels of ``libattnsink.so``.  PyTorch is
used for device memory and the current stream only.  There is no fallback:
if the library is missing or a call fails, an exception is raised.

The operation (page "GPT-OSS on Day 0", perplexity.ai, sections "Attention:
GQA with Attention Sinks" and "Kernels for GPT-OSS / Sink Attention"): each
query head's softmax includes one learned sink logit that has no value row;
query head h reads key/value head h // G.  Ragged prefill and paged decode
follow page "Fast embeddings on GPUs", section "ROSE".
"""
from __future__ import annotations

import ctypes
import math
import os

from ._build import LIB_PATH, build  # noqa: F401

F32, BF16 = 0, 1
HEAD_DIM = 64
PAGE_SIZE = 16

_lib = None

SYMBOLS = ("attn_sink_prefill", "attn_sink_prefill_partials", "attn_sink_prefill_paged",
           "attn_sink_decode_paged", "attn_sink_merge", "attn_sink_decode_paged_static",
           "attn_sink_status_string")


class AttnSinkError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load the built HIP library (never builds; raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise AttnSinkError(
            "HIP library %s is not built; run __graft_entry__.build() first" % path)
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_sink_prefill.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, P]
    lib.attn_sink_decode_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I,
                                           P, P, P, P, P]
    lib.attn_sink_prefill_partials.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I,
                                               I, I, P, P, P, P]
    lib.attn_sink_prefill_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I,
                                            F, I, I, I, P, P, P, P, P]
    lib.attn_sink_merge.argtypes = [P, P, P, I, I, I, I, I, P, P]
    lib.attn_sink_decode_paged_static.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I,
                                                  I, P, P]
    for f in (lib.attn_sink_prefill, lib.attn_sink_prefill_partials,
              lib.attn_sink_prefill_paged, lib.attn_sink_decode_paged, lib.attn_sink_merge,
              lib.attn_sink_decode_paged_static):
        f.restype = ctypes.c_int
    lib.attn_sink_status_string.argtypes = [I]
    lib.attn_sink_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(rc: int) -> str:
    return load_library().attn_sink_status_string(int(rc)).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise AttnSinkError("%s: %s (status %d)" % (what, status_string(rc), rc))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    """Check that the tensors are contiguous and on one GPU; return it."""
    dev = None
    for t in ts:
        if t is None:
            continue
        _need(t.is_cuda, "all tensors must be on the GPU")
        _need(t.is_contiguous(), "all tensors must be contiguous")
        if dev is None:
            dev = t.device
        _need(t.device == dev, "all tensors must be on the same GPU")
    return dev


def _invoke(name, device, stream, *args):
    """Call library entry point `name` with `args` and the stream, with the
    tensors' GPU current (a null stream means that GPU's null stream).
    Without a stream, the tensors' GPU's current torch stream is used."""
    import torch
    lib = load_library()
    with torch.cuda.device(device):
        if stream is None:
            stream = torch.cuda.current_stream(device)
        _need(stream.device == device, "the stream is on another GPU than the tensors")
        rc = getattr(lib, name)(*args, ctypes.c_void_p(stream.cuda_stream))
    _check(rc, name)


def attn_sink_prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int,
                      group_size: int, sm_scale: float | None = None, causal: bool = True,
                      out=None, stream=None):
    """Ragged prefill.  q [total_q, Hkv*G, 64], k/v [total_kv, Hkv, 64] (bf16 or
    fp32), sinks [Hkv*G] fp32, cu_seqlens_* [B+1] int32.  Returns out."""
    import torch
    dev = _dev(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, out)
    dt = _dtype_code(q)
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v dtypes differ")
    _need(sinks.dtype == torch.float32, "sinks must be float32")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_kv.dtype == torch.int32,
          "cu_seqlens must be int32")
    _need(q.dim() == 3 and k.dim() == 3 and v.shape == k.shape, "bad q/k/v shapes")
    hkv = k.shape[1]
    _need(q.shape[1] == hkv * group_size, "q heads != kv heads * group_size")
    _need(q.shape[2] == k.shape[2], "head_dim mismatch")
    _need(sinks.numel() == q.shape[1], "sinks must have one value per query head")
    batch = cu_seqlens_q.numel() - 1
    _need(cu_seqlens_kv.numel() == batch + 1, "cu_seqlens length mismatch")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype, "bad out tensor")
    _invoke("attn_sink_prefill", dev, stream,
            _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv),
            batch, q.shape[0], k.shape[0], int(max_seqlen_q), hkv, int(group_size), q.shape[2],
            float(sm_scale), int(bool(causal)), dt, _ptr(out))
    return out


def _partials(q, S, partial_m, partial_d, partial_o):
    """Allocate missing split partial buffers [rows, Hq, S] / [rows, Hq, S, D]."""
    import torch
    rows, hq, dim = q.shape
    f32 = dict(device=q.device, dtype=torch.float32)
    if partial_m is None:
        partial_m = torch.empty((rows, hq, S), **f32)
    if partial_d is None:
        partial_d = torch.empty((rows, hq, S), **f32)
    if partial_o is None:
        partial_o = torch.empty((rows, hq, S, dim), **f32)
    _need(partial_m.shape == (rows, hq, S) and partial_d.shape == (rows, hq, S) and
          partial_o.shape == (rows, hq, S, dim), "bad partial shapes")
    _need(all(t.dtype == torch.float32 for t in (partial_m, partial_d, partial_o)),
          "partials must be float32")
    return partial_m, partial_d, partial_o


def attn_sink_prefill_partials(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv,
                               max_seqlen_q: int, group_size: int, num_splits: int,
                               sm_scale: float | None = None, causal: bool = True,
                               partial_m=None, partial_d=None, partial_o=None, stream=None):
    """Split-KV ragged prefill: returns (partial_m, partial_d, partial_o) of
    shapes [total_q, Hq, S], [total_q, Hq, S], [total_q, Hq, S, 64] for
    attn_sink_merge (batch = total_q)."""
    import torch
    dev = _dev(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, partial_m, partial_d, partial_o)
    dt = _dtype_code(q)
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v dtypes differ")
    _need(sinks.dtype == torch.float32, "sinks must be float32")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_kv.dtype == torch.int32,
          "cu_seqlens must be int32")
    _need(q.dim() == 3 and k.dim() == 3 and v.shape == k.shape, "bad q/k/v shapes")
    hkv = k.shape[1]
    _need(q.shape[1] == hkv * group_size, "q heads != kv heads * group_size")
    _need(sinks.numel() == q.shape[1], "sinks must have one value per query head")
    batch = cu_seqlens_q.numel() - 1
    _need(cu_seqlens_kv.numel() == batch + 1, "cu_seqlens length mismatch")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    S = int(num_splits)
    pm, pd, po = _partials(q, S, partial_m, partial_d, partial_o)
    _invoke("attn_sink_prefill_partials", dev, stream,
            _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv),
            batch, q.shape[0], k.shape[0], int(max_seqlen_q), hkv, int(group_size), q.shape[2],
            float(sm_scale), int(bool(causal)), dt, S, _ptr(pm), _ptr(pd), _ptr(po))
    return pm, pd, po


def attn_sink_prefill_paged(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, sinks,
                            max_seqlen_q: int, group_size: int, sm_scale: float | None = None,
                            causal: bool = True, num_splits: int = 1, partial_m=None,
                            partial_d=None, partial_o=None, out=None, stream=None):
    """Paged (chunked) prefill.  q [total_q, Hkv*G, 64] packed by cu_seqlens_q;
    k_cache [pages, Hkv, 16, 64]; v_cache [pages, Hkv, 64, 16]; page_table
    [B, max_pages] int32; kv_lens [B] int32 (keys in the cache, the new
    tokens' included).  num_splits == 1 returns out; num_splits > 1 returns
    (partial_m, partial_d, partial_o) for attn_sink_merge."""
    import torch
    dev = _dev(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, sinks, partial_m,
               partial_d, partial_o, out)
    dt = _dtype_code(q)
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "dtype mismatch")
    _need(page_table.dtype == torch.int32 and kv_lens.dtype == torch.int32 and
          cu_seqlens_q.dtype == torch.int32, "page_table / cu_seqlens_q / kv_lens must be int32")
    _need(k_cache.dim() == 4 and v_cache.dim() == 4, "caches must be 4-d")
    num_pages, hkv, page, dim = k_cache.shape
    _need(v_cache.shape == (num_pages, hkv, dim, page), "v_cache must be [pages, Hkv, D, P]")
    _need(q.dim() == 3 and q.shape[1] == hkv * group_size, "q heads != kv heads * group_size")
    batch = cu_seqlens_q.numel() - 1
    _need(page_table.dim() == 2 and page_table.shape[0] == batch, "bad page_table")
    _need(kv_lens.numel() == batch, "bad kv_lens")
    _need(sinks.dtype == torch.float32 and sinks.numel() == q.shape[1], "bad sinks")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(dim)
    S = int(num_splits)
    if S == 1:
        if out is None:
            out = torch.empty_like(q)
        _need(out.shape == q.shape and out.dtype == q.dtype, "bad out tensor")
        pm = pd = po = None
    else:
        pm, pd, po = _partials(q, S, partial_m, partial_d, partial_o)
    _invoke("attn_sink_prefill_paged", dev, stream,
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(cu_seqlens_q),
            _ptr(kv_lens), _ptr(sinks), batch, q.shape[0], int(max_seqlen_q),
            page_table.shape[1], num_pages, hkv, int(group_size), dim, page, float(sm_scale),
            int(bool(causal)), dt, S, _ptr(pm), _ptr(pd), _ptr(po), _ptr(out))
    return out if S == 1 else (pm, pd, po)


def attn_sink_decode_paged(q, k_cache, v_cache, page_table, kv_lens, sinks,
                           group_size: int, sm_scale: float | None = None,
                           num_splits: int = 1, partial_m=None, partial_d=None,
                           partial_o=None, out=None, stream=None):
    """Paged decode.  q [B, Hkv*G, 64]; k_cache [pages, Hkv, 16, 64];
    v_cache [pages, Hkv, 64, 16]; page_table [B, max_pages] int32;
    kv_lens [B] int32.  num_splits == 1 returns out; num_splits > 1 fills and
    returns (partial_m, partial_d, partial_o) for attn_sink_merge."""
    import torch
    dev = _dev(q, k_cache, v_cache, page_table, kv_lens, sinks, partial_m, partial_d,
               partial_o, out)
    dt = _dtype_code(q)
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "dtype mismatch")
    _need(page_table.dtype == torch.int32 and kv_lens.dtype == torch.int32,
          "page_table / kv_lens must be int32")
    _need(k_cache.dim() == 4 and v_cache.dim() == 4, "caches must be 4-d")
    num_pages, hkv, page, dim = k_cache.shape
    _need(v_cache.shape == (num_pages, hkv, dim, page), "v_cache must be [pages, Hkv, D, P]")
    _need(q.dim() == 3 and q.shape[2] == dim, "q must be [B, Hkv*G, D] with the caches' D")
    batch, hq = q.shape[0], q.shape[1]
    _need(hq == hkv * group_size, "q heads != kv heads * group_size")
    _need(page_table.dim() == 2 and page_table.shape[0] == batch, "bad page_table")
    _need(kv_lens.numel() == batch, "bad kv_lens")
    _need(sinks.dtype == torch.float32 and sinks.numel() == hq, "bad sinks")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(dim)
    S = int(num_splits)
    _need(S >= 1, "num_splits must be >= 1")
    if S == 1:
        if out is None:
            out = torch.empty_like(q)
        _need(out.shape == q.shape and out.dtype == q.dtype, "bad out tensor")
    else:
        partial_m, partial_d, partial_o = _partials(q, S, partial_m, partial_d, partial_o)
    _invoke("attn_sink_decode_paged", dev, stream,
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(kv_lens),
            _ptr(sinks), batch, page_table.shape[1], num_pages, hkv, int(group_size), dim,
            page, float(sm_scale), dt, S, _ptr(partial_m), _ptr(partial_d), _ptr(partial_o),
            _ptr(out))
    return out if S == 1 else (partial_m, partial_d, partial_o)


def attn_sink_merge(partial_m, partial_d, partial_o, out=None, out_dtype=None, stream=None):
    """Merge split states: m, d [B, Hq, S], o [B, Hq, S, 64] fp32 -> [B, Hq, 64]."""
    import torch
    dev = _dev(partial_m, partial_d, partial_o, out)
    _need(partial_m.dim() == 3 and partial_o.dim() == 4, "bad partial shapes")
    batch, hq, S = partial_m.shape
    dim = partial_o.shape[-1]
    _need(partial_d.shape == partial_m.shape and partial_o.shape == (batch, hq, S, dim),
          "bad partial shapes")
    _need(all(t.dtype == torch.float32 for t in (partial_m, partial_d, partial_o)),
          "partials must be float32")
    if out is None:
        out = torch.empty((batch, hq, dim), device=partial_m.device,
                          dtype=out_dtype or torch.bfloat16)
    _need(out.shape == (batch, hq, dim), "out must be [B, Hq, D]")
    _need(out_dtype is None or out.dtype == out_dtype, "out dtype differs from out_dtype")
    _invoke("attn_sink_merge", dev, stream,
            _ptr(partial_m), _ptr(partial_d), _ptr(partial_o), batch, hq, S, dim,
            _dtype_code(out), _ptr(out))
    return out


def attn_sink_decode_paged_static(q, k_cache, v_cache, page_table, kv_lens, sinks,
                                  group_size: int, sm_scale: float | None = None,
                                  num_splits: int = 1, out=None, stream=None):
    """Split paged decode + merge in one library call that allocates nothing:
    the partial states live in the library's 16 MiB static device array.
    Arguments as attn_sink_decode_paged; returns out [B, Hkv*G, 64].  Calls
    that overlap on one GPU share that array and race."""
    import torch
    dev = _dev(q, k_cache, v_cache, page_table, kv_lens, sinks, out)
    dt = _dtype_code(q)
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "dtype mismatch")
    _need(page_table.dtype == torch.int32 and kv_lens.dtype == torch.int32,
          "page_table / kv_lens must be int32")
    _need(k_cache.dim() == 4 and v_cache.dim() == 4, "caches must be 4-d")
    num_pages, hkv, page, dim = k_cache.shape
    _need(v_cache.shape == (num_pages, hkv, dim, page), "v_cache must be [pages, Hkv, D, P]")
    _need(q.dim() == 3 and q.shape[2] == dim, "q must be [B, Hkv*G, D] with the caches' D")
    batch, hq = q.shape[0], q.shape[1]
    _need(hq == hkv * group_size, "q heads != kv heads * group_size")
    _need(page_table.dim() == 2 and page_table.shape[0] == batch, "bad page_table")
    _need(kv_lens.numel() == batch, "bad kv_lens")
    _need(sinks.dtype == torch.float32 and sinks.numel() == hq, "bad sinks")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(dim)
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype, "bad out tensor")
    _invoke("attn_sink_decode_paged_static", dev, stream,
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(kv_lens),
            _ptr(sinks), batch, page_table.shape[1], num_pages, hkv, int(group_size), dim,
            page, float(sm_scale), dt, int(num_splits), _ptr(out))
    return out


def default_num_splits(kv_lens_host, num_kv_heads: int, cus: int = 256) -> int:
    """Split count for paged decode: enough (sequence, kv head, chunk) work
    items for about six workgroups per compute unit (three rounds of the two
    8-wave split-decode workgroups a CU holds), so that a chunk stays long."""
    b = len(kv_lens_host)
    if b == 0:
        return 1
    items = b * num_kv_heads
    target = 6 * cus
    s = max(1, -(-target // items))
    max_pages = max(1, max((int(L) + PAGE_SIZE - 1) // PAGE_SIZE for L in kv_lens_host))
    return int(min(s, max_pages, 256))


def default_prefill_splits(batch: int, num_kv_heads: int, group_size: int, max_seqlen_q: int,
                           max_seqlen_kv: int, cus: int = 256) -> int:
    """Split count for prefill (attn_sink_prefill_partials / _paged): enough
    workgroups for two per compute unit (the bf16 prefill kernel's
    occupancy), each chunk keeping at least 256 keys so that the partial
    states stay small next to the work.  Few query tiles over long key
    ranges (chunked prefill) split; full prefill batches do not."""
    tokens_per_wg = 4 * (64 // group_size)
    wgs = -(-max_seqlen_q // tokens_per_wg) * batch * num_kv_heads
    if wgs <= 0:
        return 1
    s = -(-2 * cus // wgs)
    return int(max(1, min(s, max_seqlen_kv // 256)))
