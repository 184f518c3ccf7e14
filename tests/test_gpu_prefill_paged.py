"""GPU parity of paged (chunked) prefill and split-KV prefill (MI355X).

Paged prefill runs several new query tokens per sequence against the paged
cache (page "Fast embeddings on GPUs", section "ROSE"); split-KV prefill cuts
each sequence's key range into chunks whose partial states attn_sink_merge
combines, the sink carried by chunk 0 only (page "GPT-OSS on Day 0", section
"Kernels for GPT-OSS / Sink Attention").

A chunk's state (m, d, o) is one of many equivalent ones (the kernel keeps a
reference max that may trail the true max by a bounded amount), so partial
states are compared through what is unique: m + ln d and o / d, with the
empty states (-inf, 0, 0) and chunk 0's sink-only state (s, 1, 0) exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_close, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")


def _dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def paged_case(lens_q, lens_kv, hq, hkv, dtype, seed, fill=NAN, **kw):
    """Ragged inputs plus the same keys scattered into a paged cache whose
    unused slots and pages hold `fill`."""
    kw.setdefault("sink_std", 1.5)
    d = workloads.prefill_inputs(lens_q, lens_kv, hq=hq, hkv=hkv, dtype=dtype, seed=seed, **kw)
    d.update(workloads.pack_paged(d["k"], d["v"], d["lens_kv"], seed=seed + 1,
                                  extra_pages=3, fill=fill))
    return d


def _nan_outputs(q, splits, partials=False):
    """Output (splits == 1), or split partial buffers, pre-filled with NaN so
    that any element the grid never writes fails the comparison."""
    nan = float("nan")
    if splits == 1 and not partials:
        return dict(out=torch.full_like(q, nan))
    rows, hq, dim = q.shape
    f32 = dict(device=q.device, dtype=torch.float32)
    return dict(partial_m=torch.full((rows, hq, splits), nan, **f32),
                partial_d=torch.full((rows, hq, splits), nan, **f32),
                partial_o=torch.full((rows, hq, splits, dim), nan, **f32))


def run_paged(lib, d, causal=True, splits=1):
    dd = _dev(d)
    r = lib.attn_sink_prefill_paged(dd["q"], dd["k_cache"], dd["v_cache"], dd["page_table"],
                                    dd["cu_seqlens_q"], dd["kv_lens"], dd["sinks"],
                                    max(d["lens_q"] + [0]), d["group"], d["sm_scale"], causal,
                                    num_splits=splits, **_nan_outputs(dd["q"], splits))
    torch.cuda.synchronize()
    return r.cpu() if splits == 1 else tuple(t.cpu() for t in r)


def run_ragged_partials(lib, d, causal, splits):
    dd = _dev(d)
    r = lib.attn_sink_prefill_partials(dd["q"], dd["k"], dd["v"], dd["sinks"],
                                       dd["cu_seqlens_q"], dd["cu_seqlens_kv"],
                                       max(d["lens_q"] + [0]), d["group"], splits,
                                       d["sm_scale"], causal,
                                       **_nan_outputs(dd["q"], splits, partials=True))
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in r)


def oracle_paged(d, causal=True, splits=0, rows=None):
    return oracle.prefill_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                d["cu_seqlens_q"], d["kv_lens"], d["sinks"], d["group"],
                                d["sm_scale"], causal, splits=splits, rows=rows)


def check_partials(got, ref, dtype, sinks, what):
    """Compare kernel partial states with the oracle's through their unique
    parts; empty and sink-only states must be exact.  sinks broadcasts
    against the state shape without its split axis."""
    gm, gd, go = (t.double().numpy() for t in got)
    rm, rd, ro = ref
    empty = rm == -math.inf
    np.testing.assert_array_equal(gm == -math.inf, empty, err_msg=what + ": empty pattern")
    np.testing.assert_array_equal(gd[empty], 0.0)
    np.testing.assert_array_equal(go[empty], 0.0)
    # chunk 0 with no visible key and a finite sink: exactly (s, 1, 0)
    sink_only = (rd == 1.0) & np.all(ro == 0.0, axis=-1) & ~empty
    sink_only[..., 1:] = False
    if sink_only.any():
        s = np.broadcast_to(sinks.double().numpy()[..., None], rm.shape)
        np.testing.assert_array_equal(gd[sink_only], 1.0)
        np.testing.assert_array_equal(go[sink_only], 0.0)
        np.testing.assert_allclose(gm[sink_only], s[sink_only], rtol=1e-6, atol=1e-6)
    live = ~empty
    lse_tol = 1e-2 if dtype == torch.bfloat16 else 2e-5
    np.testing.assert_allclose(gm[live] + np.log(gd[live]), rm[live] + np.log(rd[live]),
                               rtol=0, atol=lse_tol, err_msg=what + ": m + ln d")
    atol, rtol = tol_for(dtype)
    on = go[live] / gd[live][:, None]
    rn = ro[live] / rd[live][:, None]
    bad = np.abs(on - rn) > atol + rtol * np.abs(rn)
    assert not bad.any(), "%s: o/d out of tolerance at %d elements" % (what, int(bad.sum()))


CASES = [
    # lens_q, lens_kv, hq, hkv, causal
    ([1], [1], 8, 2, True),
    ([5, 20, 1], [37, 20, 64], 8, 2, True),          # new tokens at the end of a cache
    ([64, 65], [200, 65], 8, 1, True),               # page-unaligned starts of the queries
    ([130, 7], [1000, 300], 16, 2, True),            # short chunk against a long cache
    ([50, 1], [20, 80], 4, 2, True),                 # Lq > Lkv: leading rows see no key
    ([70, 129], [150, 3], 8, 4, False),              # non-causal
    ([0, 40, 0, 9], [0, 40, 5, 9], 4, 1, True),      # empty sequences / empty cache
    ([300], [300], 64, 1, True),                     # group 64
    ([97], [130], 6, 2, True),                       # group 3
    ([129], [257], 2, 2, True),                      # group 1
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_prefill_sweep_matches_oracle(lib, dtype, case):
    lens_q, lens_kv, hq, hkv, causal = CASES[case]
    d = paged_case(lens_q, lens_kv, hq, hkv, dtype, seed=40 + case)
    out = run_paged(lib, d, causal)
    assert_close(out, oracle_paged(d, causal), dtype, "paged case %d" % case)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_paged_equals_ragged_kernel_bitwise(lib, dtype):
    """The paged kernel reads the same K/V values into the same MFMA
    operands as the ragged kernel, so the outputs agree bit for bit."""
    d = paged_case([300, 77, 5], [300, 1000, 40], 16, 2, dtype, seed=3)
    dd = _dev(d)
    rag = lib.attn_sink_prefill(dd["q"], dd["k"], dd["v"], dd["sinks"], dd["cu_seqlens_q"],
                                dd["cu_seqlens_kv"], 300, d["group"], d["sm_scale"], True)
    torch.cuda.synchronize()
    assert torch.equal(run_paged(lib, d), rag.cpu())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_paged_prefill_sink_extremes(lib, dtype):
    """Sinks -inf, 0, moderate and +20 with logits up to about +-30."""
    sinks = torch.tensor([-math.inf, 0.0, 1.3, 20.0, -math.inf, -2.0, 20.0, 0.5])
    mults = [1.0, 2.0, 4.0, 7.5, 7.5, 4.0, 2.0, 1.0]
    d = paged_case([77, 200], [500, 200], 8, 2, dtype, seed=4, sinks=sinks, q_head_mult=mults)
    assert_close(run_paged(lib, d), oracle_paged(d), dtype, "paged sink extremes")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [1, 2, 5, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_split_partials_and_merge(lib, dtype, splits, causal):
    """Ragged split prefill: partial states against the oracle's, and the
    merged result against the unsplit oracle."""
    d = paged_case([3, 130, 1, 0, 64], [85, 130, 600, 5, 64], 8, 2, dtype, seed=splits)
    got = run_ragged_partials(lib, d, causal, splits)
    ref = oracle.prefill_partials(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                                  d["cu_seqlens_kv"], 2, 4, d["sm_scale"], causal, splits)
    check_partials(got, ref, dtype, d["sinks"], "ragged S=%d" % splits)
    merged = lib.attn_sink_merge(*(t.to(DEV) for t in got), out_dtype=dtype)
    torch.cuda.synchronize()
    full = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                          d["cu_seqlens_kv"], 2, 4, d["sm_scale"], causal)
    assert_close(merged.cpu(), full, dtype, "ragged split merged")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [2, 5])
def test_ragged_split_sequence_major_order(lib, dtype, splits):
    """Split prefill whose work order is sequence-major per XCD (kv heads a
    multiple of 8, unequal lengths): every (sequence, head, tile, chunk) is
    written exactly once."""
    d = paged_case([3, 130, 1, 0, 64, 257], [85, 130, 600, 5, 64, 257], 16, 8, dtype,
                   seed=20 + splits)
    got = run_ragged_partials(lib, d, True, splits)
    ref = oracle.prefill_partials(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                                  d["cu_seqlens_kv"], 8, 2, d["sm_scale"], True, splits)
    check_partials(got, ref, dtype, d["sinks"], "ragged seq-major S=%d" % splits)
    merged = lib.attn_sink_merge(*(t.to(DEV) for t in got), out_dtype=dtype)
    torch.cuda.synchronize()
    full = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                          d["cu_seqlens_kv"], 8, 2, d["sm_scale"], True)
    assert_close(merged.cpu(), full, dtype, "ragged seq-major merged")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [2, 7, 64])
def test_paged_split_partials_and_merge(lib, dtype, splits):
    d = paged_case([3, 130, 1, 0, 64], [85, 130, 600, 5, 64], 8, 2, dtype, seed=10 + splits)
    got = run_paged(lib, d, True, splits)
    ref = oracle_paged(d, True, splits)
    check_partials(got, ref, dtype, d["sinks"], "paged S=%d" % splits)
    merged = lib.attn_sink_merge(*(t.to(DEV) for t in got), out_dtype=dtype)
    torch.cuda.synchronize()
    assert_close(merged.cpu(), oracle_paged(d, True), dtype, "paged split merged")


def test_split_empty_rows_keep_sink_in_chunk_zero(lib):
    """More queries than keys: rows that see nothing hold (s, 1, 0) in chunk
    0 and (-inf, 0, 0) elsewhere, and merge to 0."""
    sinks = torch.tensor([1.25, -math.inf, 0.0, 20.0])
    d = paged_case([6], [2], 4, 1, torch.bfloat16, seed=2, sinks=sinks)
    pm, pd, po = run_ragged_partials(lib, d, True, 3)
    for i in range(4):
        for h in range(4):
            s = float(sinks[h])
            if s == -math.inf:
                assert pm[i, h, 0] == -math.inf and pd[i, h, 0] == 0
            else:
                assert pd[i, h, 0] == 1 and abs(float(pm[i, h, 0]) - s) <= 1e-5 * max(1, abs(s))
            assert torch.all(po[i, h, 0] == 0)
            assert torch.all(pm[i, h, 1:] == -math.inf) and torch.all(pd[i, h, 1:] == 0)
    merged = lib.attn_sink_merge(pm.to(DEV), pd.to(DEV), po.to(DEV))
    torch.cuda.synchronize()
    assert torch.all(merged.cpu()[:4] == 0)


def test_paged_page_placement_and_poison_invariance(lib):
    """Two physical placements with different junk in unused slots give the
    same bits (unread slots never leak in, the tail of the last page
    included)."""
    d1 = paged_case([33, 100], [77, 500], 8, 2, torch.bfloat16, seed=5, fill=NAN)
    d2 = dict(d1)
    d2.update(workloads.pack_paged(d1["k"], d1["v"], d1["lens_kv"], seed=99, extra_pages=7,
                                   fill=float("inf")))
    a, b = run_paged(lib, d1), run_paged(lib, d2)
    assert torch.all(torch.isfinite(a.float()))
    assert torch.equal(a, b)


def test_paged_prefill_deterministic(lib):
    d = paged_case([200, 31], [900, 31], 16, 2, torch.bfloat16, seed=8)
    assert torch.equal(run_paged(lib, d), run_paged(lib, d))
    a = run_paged(lib, d, True, 5)
    b = run_paged(lib, d, True, 5)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_chunked_prefill_workload_full(lib):
    """The benchmark's chunked prefill: one sequence, 512 new tokens on a
    paged cache of 32768 keys (the new tokens' included), Hq 64 / Hkv 8,
    bf16, random page placement; unsplit, and split as the benchmark splits
    it then merged.  Every output element, and every partial state through
    m + ln d and o / d, against the fp64 oracle (about 20 s of oracle time on
    16 host cores)."""
    from gqa_attention_sinks_initialised_amd import default_prefill_splits
    d = workloads.workload(6)
    S = default_prefill_splits(1, 8, 8, 512, 32768)
    ref = oracle_paged(d, True)
    assert_close(run_paged(lib, d), ref, torch.bfloat16, "chunked prefill unsplit")
    got = run_paged(lib, d, True, S)
    merged = torch.full_like(_dev(d)["q"], NAN)
    lib.attn_sink_merge(*(t.to(DEV) for t in got), out=merged, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(merged.cpu(), ref, torch.bfloat16, "chunked prefill split %d" % S)
    check_partials(got, oracle_paged(d, True, S), torch.bfloat16, d["sinks"][None, :],
                   "chunked prefill partials")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [1, 3])
def test_paged_prefill_pages_past_4gib(lib, dtype, splits):
    """Caches of 4 GiB or more (an engine-sized cache) are read through
    64-bit page bases: with the same logical pages moved past the 4 GiB mark
    of a 5 GiB cache, the result is bit for bit that of the compact cache,
    and matches the oracle."""
    d = paged_case([40, 130, 1], [300, 130, 77], 8, 2, dtype, seed=91)
    small = run_paged(lib, d, True, splits)
    dd = _dev(d)
    kc, vc, pt = dd["k_cache"], dd["v_cache"], dd["page_table"]
    block = kc[0].numel() * kc.element_size()
    nbig = -(-(5 << 30) // block)
    big = dict(dd)
    big["k_cache"] = torch.empty((nbig,) + tuple(kc.shape[1:]), dtype=kc.dtype, device=DEV)
    big["v_cache"] = torch.empty((nbig,) + tuple(vc.shape[1:]), dtype=vc.dtype, device=DEV)
    n = kc.shape[0]
    new_ids = nbig - 1 - torch.arange(n, device=DEV)
    big["k_cache"][new_ids] = kc
    big["v_cache"][new_ids] = vc
    valid = (pt >= 0) & (pt < n)
    big["page_table"] = torch.where(valid, nbig - 1 - pt, pt).to(torch.int32)
    assert int(big["page_table"][valid].min()) * block >= (4 << 30)
    got = run_paged(lib, big, True, splits)
    del big
    if splits == 1:
        assert torch.equal(got.view(torch.int16) if dtype == torch.bfloat16 else got.view(torch.int32),
                           small.view(torch.int16) if dtype == torch.bfloat16 else small.view(torch.int32))
        assert_close(got, oracle_paged(d), dtype, "paged prefill, 5 GiB cache")
    else:
        for a, b in zip(got, small):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        check_partials(got, oracle_paged(d, True, splits), dtype, d["sinks"], "5 GiB cache")
