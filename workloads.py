"""Seeded synthetic inputs for GQA attention with per-head sinks.

This module only draws random inputs and lays them out; it holds none of the
attention arithmetic.  The HIP library's tests and benchmark and the fp64
oracle both consume what it returns, so the two sides always see identical
values (bf16 inputs are rounded once, here, by round-to-nearest-even).

Layouts (shared by every caller):
  ragged prefill:  q [total_q, Hq, D], k / v [total_kv, Hkv, D],
                   cu_seqlens_q / cu_seqlens_kv [B+1] int32, sinks [Hq] fp32
  paged decode:    q [B, Hq, D], k_cache [num_pages, Hkv, P, D],
                   v_cache [num_pages, Hkv, D, P] (dim-major pages),
                   page_table [B, max_pages] int32 (-1 past a sequence's last
                   page), kv_lens [B] int32, sinks [Hq] fp32
  paged prefill:   q [total_q, Hq, D] with cu_seqlens_q, and the paged cache
                   of decode (pack_paged lays ragged k / v out that way)

The named workloads follow the benchmark configurations of the project:
  1  tiny causal prefill, fp32: B=1, L=128, Hq=8, Hkv=2, D=64
  2  causal prefill, bf16: B=4 x 2048, Hq=64, Hkv=8, D=64
  3  paged decode, bf16: B=64, kv_len ~ U{512..8192}, 16-token pages
  4  long split-KV decode, bf16: B=4, kv_len 131072, 64 splits
  5  ragged causal prefill with numeric edge cases, bf16: 16 sequences,
     len ~ U{128..4096}, sinks from {-inf, 0, N(0,1), +20}, Q multipliers
     {1, 2, 4, 7.5} so that logits reach about +-30
  6  chunked prefill against the paged cache, bf16: B=1, 512 new query
     tokens, kv_len 32768 (the new tokens' keys included), Hq=64, Hkv=8
Seeds are 1000 + workload number.
"""
from __future__ import annotations

import math

import torch

SEED_BASE = 1000
HEAD_DIM = 64
PAGE = 16


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device, dtype, mult=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(dtype)


def cu_from_lens(lens) -> torch.Tensor:
    lens = torch.as_tensor(lens, dtype=torch.int64)
    cu = torch.zeros(len(lens) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    return cu.to(torch.int32)


def prefill_inputs(lens_q, lens_kv=None, *, hq=8, hkv=2, dim=HEAD_DIM,
                   dtype=torch.bfloat16, seed=0, qkv_scale=1.0, q_head_mult=None,
                   sinks=None, sink_std=1.0, device="cpu"):
    """Ragged prefill inputs.  q_head_mult: optional [Hq] multipliers applied
    to q before the cast; sinks: optional explicit [Hq] values."""
    lens_kv = list(lens_q) if lens_kv is None else list(lens_kv)
    g = _gen(seed, device)
    cu_q, cu_kv = cu_from_lens(lens_q), cu_from_lens(lens_kv)
    tq, tkv = int(cu_q[-1]), int(cu_kv[-1])
    q = torch.randn((tq, hq, dim), generator=g, device=device) * qkv_scale
    if q_head_mult is not None:
        q = q * torch.as_tensor(q_head_mult, dtype=torch.float32,
                                device=device).view(1, hq, 1)
    k = _randn((tkv, hkv, dim), g, device, torch.float32, qkv_scale)
    v = _randn((tkv, hkv, dim), g, device, torch.float32, qkv_scale)
    if sinks is None:
        s = torch.randn((hq,), generator=g, device=device) * sink_std
    else:
        s = torch.as_tensor(sinks, dtype=torch.float32, device=device)
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), sinks=s.float(),
                cu_seqlens_q=cu_q.to(device), cu_seqlens_kv=cu_kv.to(device),
                lens_q=list(map(int, lens_q)), lens_kv=list(map(int, lens_kv)),
                num_kv_heads=hkv, group=hq // hkv, head_dim=dim,
                sm_scale=1.0 / math.sqrt(dim))


def page_table_for(kv_lens, page=PAGE, seed=0, max_pages=None, pad=-1,
                   extra_pages=0):
    """Random physical placement: ids = randperm(total pages), assigned in
    (sequence, page) order; entries past a sequence's last page hold `pad`.
    Returns (page_table [B, max_pages] int32, num_pages)."""
    g = _gen(seed + 7919, "cpu")
    npg = [(int(L) + page - 1) // page for L in kv_lens]
    total = sum(npg)
    if max_pages is None:
        max_pages = max(1, max(npg) if npg else 1)
    num_pages = total + extra_pages
    perm = torch.randperm(num_pages, generator=g)[:total].to(torch.int32)
    pt = torch.full((len(kv_lens), max_pages), pad, dtype=torch.int32)
    off = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt, num_pages


def pack_paged(k, v, lens_kv, page=PAGE, seed=0, max_pages=None, extra_pages=0,
               fill=0.0):
    """Scatter ragged k / v [total_kv, Hkv, D] into a paged cache: K pages
    [num_pages, Hkv, P, D], V pages [num_pages, Hkv, D, P] (dim-major), with
    the random placement of page_table_for.  Slots past a sequence's last key
    and pages no sequence uses hold `fill` (e.g. NaN, to show they are never
    read).  Returns dict(k_cache, v_cache, page_table, kv_lens, num_pages,
    max_pages) on k's device."""
    lens = [int(x) for x in lens_kv]
    pt, num_pages = page_table_for(lens, page, seed, max_pages, extra_pages=extra_pages)
    total, hkv, dim = k.shape
    dev = k.device
    kc = torch.full((num_pages, hkv, page, dim), fill, dtype=k.dtype, device=dev)
    vc = torch.full((num_pages, hkv, dim, page), fill, dtype=v.dtype, device=dev)
    if total > 0:
        lt = torch.as_tensor(lens, dtype=torch.int64)
        seq = torch.repeat_interleave(torch.arange(len(lens)), lt)
        pos = torch.arange(total) - cu_from_lens(lens).long()[seq]
        phys = pt.long()[seq, pos // page].to(dev)
        slot = (pos % page).to(dev)
        kc[phys, :, slot, :] = k            # token t -> page row t % P
        vc[phys, :, :, slot] = v            # token t -> page column t % P
    return dict(k_cache=kc, v_cache=vc, page_table=pt.to(dev),
                kv_lens=torch.as_tensor(lens, dtype=torch.int32).to(dev),
                num_pages=num_pages, max_pages=pt.shape[1])


def decode_inputs(kv_lens, *, hq=8, hkv=2, dim=HEAD_DIM, page=PAGE,
                  dtype=torch.bfloat16, seed=0, qkv_scale=1.0, sink_std=1.0,
                  sinks=None, max_pages=None, extra_pages=0, device="cpu",
                  cache_device=None):
    """Paged decode inputs (one query token per sequence).  The cache may be
    drawn on `cache_device` (e.g. the GPU, for the 1 GiB workloads)."""
    cache_device = device if cache_device is None else cache_device
    pt, num_pages = page_table_for(kv_lens, page, seed, max_pages,
                                   extra_pages=extra_pages)
    g = _gen(seed, "cpu")
    b = len(kv_lens)
    q = (torch.randn((b, hq, dim), generator=g) * qkv_scale).to(dtype)
    if sinks is None:
        s = torch.randn((hq,), generator=g) * sink_std
    else:
        s = torch.as_tensor(sinks, dtype=torch.float32)
    gc = _gen(seed + 1, cache_device)
    kc = _randn((num_pages, hkv, page, dim), gc, cache_device, dtype, qkv_scale)
    vc = _randn((num_pages, hkv, dim, page), gc, cache_device, dtype, qkv_scale)
    return dict(q=q.to(device), k_cache=kc, v_cache=vc,
                page_table=pt.to(device),
                kv_lens=torch.as_tensor(list(kv_lens), dtype=torch.int32).to(device),
                sinks=s.float().to(device), num_pages=num_pages,
                max_pages=pt.shape[1], num_kv_heads=hkv, group=hq // hkv,
                head_dim=dim, page_size=page, sm_scale=1.0 / math.sqrt(dim))


def c5_sinks_and_mults(hq, seed):
    """Per-head sink category h mod 4 -> {-inf, 0, N(0,1), +20}; Q multiplier
    {1, 2, 4, 7.5}[(h // 4) mod 4]."""
    g = _gen(seed + 17, "cpu")
    draws = torch.randn((hq,), generator=g)
    sinks = torch.empty(hq)
    for h in range(hq):
        cat = h % 4
        sinks[h] = (-math.inf, 0.0, float(draws[h]), 20.0)[cat]
    mults = [(1.0, 2.0, 4.0, 7.5)[(h // 4) % 4] for h in range(hq)]
    return sinks, mults


def workload(n: int, device="cpu", cache_device=None) -> dict:
    """The named workloads 1..6 (see module docstring)."""
    seed = SEED_BASE + n
    if n == 1:
        d = prefill_inputs([128], hq=8, hkv=2, dtype=torch.float32, seed=seed,
                           qkv_scale=1.0 / 8.0, sink_std=1.0, device=device)
        d.update(kind="prefill", causal=True,
                 name="tiny causal prefill fp32 B=1 L=128 Hq=8 Hkv=2 D=64")
        return d
    if n == 2:
        d = prefill_inputs([2048] * 4, hq=64, hkv=8, dtype=torch.bfloat16,
                           seed=seed, sink_std=math.sqrt(2.0), device=device)
        d.update(kind="prefill", causal=True,
                 name="causal prefill bf16 B=4 L=2048 Hq=64 Hkv=8 D=64")
        return d
    if n == 3:
        g = _gen(seed + 3, "cpu")
        lens = torch.randint(512, 8193, (64,), generator=g).tolist()
        d = decode_inputs(lens, hq=64, hkv=8, dtype=torch.bfloat16, seed=seed,
                          sink_std=math.sqrt(2.0), max_pages=512, device=device,
                          cache_device=cache_device)
        d.update(kind="decode", num_splits=None,
                 name="paged decode bf16 B=64 kv_len U[512,8192] Hq=64 Hkv=8 "
                      "D=64 page 16")
        return d
    if n == 4:
        d = decode_inputs([131072] * 4, hq=64, hkv=8, dtype=torch.bfloat16,
                          seed=seed, sink_std=math.sqrt(2.0), device=device,
                          cache_device=cache_device)
        d.update(kind="decode", num_splits=64,
                 name="split-KV decode bf16 B=4 kv_len 131072 Hq=64 Hkv=8 D=64 "
                      "page 16, 64 splits")
        return d
    if n == 5:
        g = _gen(seed + 3, "cpu")
        lens = torch.randint(128, 4097, (16,), generator=g).tolist()
        sinks, mults = c5_sinks_and_mults(64, seed)
        d = prefill_inputs(lens, hq=64, hkv=8, dtype=torch.bfloat16, seed=seed,
                           q_head_mult=mults, sinks=sinks, device=device)
        d.update(kind="prefill", causal=True,
                 name="ragged causal prefill bf16 16 seqs len U[128,4096] Hq=64 "
                      "Hkv=8 D=64, edge-case sinks and logits")
        return d
    if n == 6:
        d = prefill_inputs([512], [32768], hq=64, hkv=8, dtype=torch.bfloat16, seed=seed,
                           sink_std=math.sqrt(2.0), device=device)
        d.update(pack_paged(d["k"], d["v"], d["lens_kv"], seed=seed + 1))
        d.update(kind="prefill_paged", causal=True,
                 name="chunked prefill bf16 B=1, 512 new tokens on a paged cache of 32768 "
                      "keys, Hq=64 Hkv=8 D=64 page 16")
        return d
    raise ValueError("workload number must be 1..6")
