"""fp64 CPU oracle for GQA attention with per-head sinks -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product library never loads it,
and it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module only builds it with gcc and marshals arrays through ctypes.  What it
computes, and the readings taken where the pages are silent, are stated at the
top of ``oracle.c``: page "GPT-OSS on Day 0" (perplexity.ai), sections
"Attention: GQA with Attention Sinks" and "Kernels for GPT-OSS / Sink
Attention"; page "Fast embeddings on GPUs", section "ROSE" (ragged and paged
attention).

Inputs may be torch CPU tensors or numpy arrays in fp32, bf16 (torch) or
fp64; bf16 values are widened exactly.  Every output is a float64 numpy array.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIBRARY points the tests at another build of oracle.c (the mutation
# test builds copies with planted mistakes and checks that the pins fail).
_LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_prefill_rows.argtypes = [P, P, P, I, P, P, P, I, I, I, I, D, I, I,
                                            L, P, P, P, P]
        lib.oracle_decode_paged_rows.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I,
                                                 I, D, I, L, P, P, P, P]
        lib.oracle_decode_partials_rows.argtypes = [P, P, P, I, P, P, P, I, I, I, I,
                                                    I, I, D, I, I, L, P, P, P, P, P,
                                                    P]
        lib.oracle_prefill_partials_rows.argtypes = [P, P, P, I, P, P, P, I, I, I,
                                                     I, D, I, I, I, I, L, P, P, P,
                                                     P, P, P]
        lib.oracle_prefill_paged_rows.argtypes = [P, P, P, I, P, P, P, P, I, I, I,
                                                  I, I, I, D, I, I, I, L, P, P, P,
                                                  P, P, P, P]
        lib.oracle_merge.argtypes = [P, P, P, L, I, I, P]
        lib.oracle_max_threads.argtypes = []
        for f in (lib.oracle_prefill_rows, lib.oracle_decode_paged_rows,
                  lib.oracle_decode_partials_rows, lib.oracle_prefill_partials_rows,
                  lib.oracle_prefill_paged_rows, lib.oracle_merge,
                  lib.oracle_max_threads):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().oracle_max_threads()


def _elems(x):
    """(contiguous numpy array, element-type code) without changing values."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            raise TypeError("unsupported tensor dtype %s" % x.dtype)
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    raise TypeError("unsupported array dtype %s" % x.dtype)


def _i32(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k, v, sinks, cu_q, cu_kv, num_kv_heads: int, group: int,
            sm_scale: float, causal: bool, rows=None):
    """Ragged prefill.  q [total_q, Hkv*G, D], k/v [total_kv, Hkv, D].

    rows=None computes every (token, head) row and returns [total_q, Hq, D];
    otherwise rows is a pair (tokens, heads) of equal-length int sequences and
    the result is [len(tokens), D].
    """
    qa, dt = _elems(q)
    ka, dk = _elems(k)
    va, dv = _elems(v)
    if not (dt == dk == dv):
        raise TypeError("q, k, v must share one element type")
    cq, ck = _i32(cu_q), _i32(cu_kv)
    s = _f64(sinks)
    total_q, hq, dim = qa.shape
    if hq != num_kv_heads * group:
        raise ValueError("q heads != num_kv_heads * group")
    batch = len(cq) - 1
    if rows is None:
        toks = np.repeat(np.arange(total_q, dtype=np.int64), hq)
        heads = np.tile(np.arange(hq, dtype=np.int32), total_q)
    else:
        toks = np.ascontiguousarray(np.asarray(rows[0], dtype=np.int64))
        heads = np.ascontiguousarray(np.asarray(rows[1], dtype=np.int32))
    n = len(toks)
    max_kv = int(max(1, (ck[1:] - ck[:-1]).max() if batch > 0 else 1))
    out = np.zeros((n, dim), dtype=np.float64)
    scratch = np.zeros(max_threads() * max_kv, dtype=np.float64)
    rc = _load().oracle_prefill_rows(
        _ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(s), _ptr(cq), _ptr(ck), batch,
        num_kv_heads, group, dim, float(sm_scale), int(bool(causal)), max_kv, n,
        _ptr(toks), _ptr(heads), _ptr(out), _ptr(scratch))
    if rc != 0:
        raise ValueError("oracle_prefill_rows: a row lies outside every sequence")
    if rows is None:
        return out.reshape(total_q, hq, dim)
    return out


def _prefill_rows(total_q, hq, rows):
    if rows is None:
        toks = np.repeat(np.arange(total_q, dtype=np.int64), hq)
        heads = np.tile(np.arange(hq, dtype=np.int32), total_q)
    else:
        toks = np.ascontiguousarray(np.asarray(rows[0], dtype=np.int64))
        heads = np.ascontiguousarray(np.asarray(rows[1], dtype=np.int32))
    return toks, heads


def prefill_partials(q, k, v, sinks, cu_q, cu_kv, num_kv_heads: int, group: int,
                     sm_scale: float, causal: bool, splits: int, unit: int = 16,
                     rows=None):
    """Split-KV partial states of ragged prefill; each sequence's keys are cut
    into S chunks of ceil(ceil(Lkv/unit)/S) units and only chunk 0 carries
    the sink.  Returns m, d [..., S] and o [..., S, D] with ... = [total_q, Hq]
    for rows=None, else [n_rows]."""
    qa, dt = _elems(q)
    ka, dk = _elems(k)
    va, dv = _elems(v)
    if not (dt == dk == dv):
        raise TypeError("q, k, v must share one element type")
    cq, ck = _i32(cu_q), _i32(cu_kv)
    s = _f64(sinks)
    total_q, hq, dim = qa.shape
    if hq != num_kv_heads * group:
        raise ValueError("q heads != num_kv_heads * group")
    batch = len(cq) - 1
    toks, heads = _prefill_rows(total_q, hq, rows)
    n = len(toks)
    max_kv = int(max(1, (ck[1:] - ck[:-1]).max() if batch > 0 else 1))
    m = np.zeros((n, splits), dtype=np.float64)
    d = np.zeros((n, splits), dtype=np.float64)
    o = np.zeros((n, splits, dim), dtype=np.float64)
    scratch = np.zeros(max_threads() * max_kv, dtype=np.float64)
    rc = _load().oracle_prefill_partials_rows(
        _ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(s), _ptr(cq), _ptr(ck), batch,
        num_kv_heads, group, dim, float(sm_scale), int(bool(causal)), int(unit),
        int(splits), max_kv, n, _ptr(toks), _ptr(heads), _ptr(m), _ptr(d), _ptr(o),
        _ptr(scratch))
    if rc != 0:
        raise ValueError("oracle_prefill_partials_rows: bad row")
    if rows is None:
        return (m.reshape(total_q, hq, splits), d.reshape(total_q, hq, splits),
                o.reshape(total_q, hq, splits, dim))
    return m, d, o


def prefill_paged(q, k_cache, v_cache, page_table, cu_q, kv_lens, sinks, group: int,
                  sm_scale: float, causal: bool, splits: int = 0, rows=None):
    """Paged (chunked) prefill.  q [total_q, Hkv*G, D]; k_cache [pages, Hkv, P, D];
    v_cache [pages, Hkv, D, P]; page_table [B, max_pages]; cu_q [B+1];
    kv_lens [B] (all keys in the cache, the new tokens' included).

    splits=0 returns the attention output ([total_q, Hq, D] or [n_rows, D]);
    splits>=1 returns the partial states (m, d, o) of page-aligned chunks."""
    qa, dt = _elems(q)
    ka, dk = _elems(k_cache)
    va, dv = _elems(v_cache)
    if not (dt == dk == dv):
        raise TypeError("q, k_cache, v_cache must share one element type")
    pt, cq, lens, s = _i32(page_table), _i32(cu_q), _i32(kv_lens), _f64(sinks)
    total_q, hq, dim = qa.shape
    hkv, psz = ka.shape[1], ka.shape[2]
    if hq != hkv * group:
        raise ValueError("q heads != num_kv_heads * group")
    batch = len(cq) - 1
    toks, heads = _prefill_rows(total_q, hq, rows)
    n = len(toks)
    max_len = int(max(1, lens.max() if batch > 0 else 1))
    S = int(splits)
    out = np.zeros((n, dim), dtype=np.float64)
    m = np.zeros((n, max(S, 1)), dtype=np.float64)
    d = np.zeros((n, max(S, 1)), dtype=np.float64)
    o = np.zeros((n, max(S, 1), dim), dtype=np.float64)
    scratch = np.zeros(max_threads() * max_len, dtype=np.float64)
    rc = _load().oracle_prefill_paged_rows(
        _ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(pt), _ptr(cq), _ptr(lens), _ptr(s),
        batch, pt.shape[1], hkv, group, dim, psz, float(sm_scale),
        int(bool(causal)), S, max_len, n, _ptr(toks), _ptr(heads), _ptr(out),
        _ptr(m), _ptr(d), _ptr(o), _ptr(scratch))
    if rc != 0:
        raise ValueError("oracle_prefill_paged_rows: bad row")
    if S == 0:
        return out.reshape(total_q, hq, dim) if rows is None else out
    if rows is None:
        return (m.reshape(total_q, hq, S), d.reshape(total_q, hq, S),
                o.reshape(total_q, hq, S, dim))
    return m, d, o


def _decode_rows(q, rows):
    batch, hq = q.shape[0], q.shape[1]
    if rows is None:
        rb = np.repeat(np.arange(batch, dtype=np.int32), hq)
        rh = np.tile(np.arange(hq, dtype=np.int32), batch)
    else:
        rb = np.ascontiguousarray(np.asarray(rows[0], dtype=np.int32))
        rh = np.ascontiguousarray(np.asarray(rows[1], dtype=np.int32))
    return rb, rh


def decode_paged(q, k_cache, v_cache, page_table, kv_lens, sinks, group: int,
                 sm_scale: float, rows=None):
    """Paged decode.  q [B, Hkv*G, D]; k_cache [pages, Hkv, P, D];
    v_cache [pages, Hkv, D, P]; page_table [B, max_pages]; kv_lens [B].

    Returns [B, Hq, D] (rows=None) or [n_rows, D] for rows=(seqs, heads).
    """
    qa, dt = _elems(q)
    ka, dk = _elems(k_cache)
    va, dv = _elems(v_cache)
    if not (dt == dk == dv):
        raise TypeError("q, k_cache, v_cache must share one element type")
    pt, lens, s = _i32(page_table), _i32(kv_lens), _f64(sinks)
    batch, hq, dim = qa.shape
    hkv, psz = ka.shape[1], ka.shape[2]
    max_pages = pt.shape[1]
    rb, rh = _decode_rows(qa, rows)
    n = len(rb)
    max_len = int(max(1, lens.max() if batch > 0 else 1))
    out = np.zeros((n, dim), dtype=np.float64)
    scratch = np.zeros(max_threads() * max_len, dtype=np.float64)
    rc = _load().oracle_decode_paged_rows(
        _ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(pt), _ptr(lens), _ptr(s), batch,
        max_pages, hkv, group, dim, psz, float(sm_scale), max_len, n, _ptr(rb),
        _ptr(rh), _ptr(out), _ptr(scratch))
    if rc != 0:
        raise ValueError("oracle_decode_paged_rows: bad row")
    return out.reshape(batch, hq, dim) if rows is None else out


def decode_partials(q, k_cache, v_cache, page_table, kv_lens, sinks, group: int,
                    sm_scale: float, splits: int, rows=None):
    """Split-KV partial states (m, d, o) of paged decode; only chunk 0 carries
    the sink.  Shapes: m, d [..., S]; o [..., S, D] with ... = [B, Hq] for
    rows=None, else [n_rows]."""
    qa, dt = _elems(q)
    ka, _ = _elems(k_cache)
    va, _ = _elems(v_cache)
    pt, lens, s = _i32(page_table), _i32(kv_lens), _f64(sinks)
    batch, hq, dim = qa.shape
    hkv, psz = ka.shape[1], ka.shape[2]
    rb, rh = _decode_rows(qa, rows)
    n = len(rb)
    max_len = int(max(1, lens.max() if batch > 0 else 1))
    m = np.zeros((n, splits), dtype=np.float64)
    d = np.zeros((n, splits), dtype=np.float64)
    o = np.zeros((n, splits, dim), dtype=np.float64)
    scratch = np.zeros(max_threads() * max_len, dtype=np.float64)
    rc = _load().oracle_decode_partials_rows(
        _ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(pt), _ptr(lens), _ptr(s), batch,
        pt.shape[1], hkv, group, dim, psz, float(sm_scale), int(splits), max_len,
        n, _ptr(rb), _ptr(rh), _ptr(m), _ptr(d), _ptr(o), _ptr(scratch))
    if rc != 0:
        raise ValueError("oracle_decode_partials_rows: bad row")
    if rows is None:
        return (m.reshape(batch, hq, splits), d.reshape(batch, hq, splits),
                o.reshape(batch, hq, splits, dim))
    return m, d, o


def merge(m, d, o):
    """Merge split states: m, d [..., S], o [..., S, D] -> [..., D]."""
    m, d, o = _f64(m), _f64(d), _f64(o)
    lead = m.shape[:-1]
    splits, dim = o.shape[-2], o.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    out = np.zeros((rows, dim), dtype=np.float64)
    _load().oracle_merge(_ptr(m), _ptr(d), _ptr(o), rows, splits, dim, _ptr(out))
    return out.reshape(*lead, dim)
