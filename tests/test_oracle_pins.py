"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties one part of the oracle's definition to an independent source:
torch's own scaled-dot-product attention (a textbook routine), closed forms,
invariants, a 50-digit mpmath brute force, and hand-derived worked examples.
They are chosen so that a plausible slip in the oracle -- a dropped sink term,
the sink multiplied by sm_scale, a wrong GQA head map, top-left instead of
bottom-right causal alignment, a sink counted in every split, a wrong page
index -- fails at least one of them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _f(x):
    return -math.inf if x == "-inf" else (math.inf if x == "inf" else float(x))


def _sdpa_fp64(q, k, v, group, scale, causal, sinks=None):
    """torch SDPA in fp64 for one sequence.  q [Lq, Hq, D], k/v [Lkv, Hkv, D].
    With sinks: one extra all-zero key and value row whose additive mask entry
    is the head's sink, so its logit is exactly s_h and it adds no value."""
    q = q.double().permute(1, 0, 2).unsqueeze(0)                   # [1,Hq,Lq,D]
    k = k.double().repeat_interleave(group, dim=1).permute(1, 0, 2).unsqueeze(0)
    v = v.double().repeat_interleave(group, dim=1).permute(1, 0, 2).unsqueeze(0)
    hq, lq, lkv = q.shape[1], q.shape[2], k.shape[2]
    if causal:
        allowed = causal_lower_right(lq, lkv)._materialize(device=q.device)
    else:
        allowed = torch.ones(lq, lkv, dtype=torch.bool)
    bias = torch.zeros(hq, lq, lkv, dtype=torch.float64)
    bias.masked_fill_(~allowed.unsqueeze(0), -math.inf)
    if sinks is not None:
        zk = torch.zeros(1, hq, 1, k.shape[3], dtype=torch.float64)
        k = torch.cat([k, zk], dim=2)
        v = torch.cat([v, zk], dim=2)
        col = torch.as_tensor(sinks, dtype=torch.float64).view(hq, 1, 1).expand(hq, lq, 1)
        bias = torch.cat([bias, col], dim=2)
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=bias.unsqueeze(0),
                                         scale=scale)
    return out[0].permute(1, 0, 2).numpy()                          # [Lq,Hq,D]


# ----------------------------------------------------------------- O1 / O2
@pytest.mark.parametrize("lq,lkv,causal,hq,hkv", [
    (17, 17, True, 4, 1), (9, 23, True, 6, 2), (13, 13, False, 8, 8),
    (5, 40, False, 4, 2), (33, 33, True, 8, 2)])
def test_no_sink_equals_sdpa(lq, lkv, causal, hq, hkv):
    """sink = -inf reduces to standard softmax attention (SDPA, fp64)."""
    d = workloads.prefill_inputs([lq], [lkv], hq=hq, hkv=hkv, dim=16,
                                 dtype=torch.float32, seed=lq * 31 + lkv,
                                 sinks=[-math.inf] * hq)
    got = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], hkv, hq // hkv, 0.37, causal)
    ref = _sdpa_fp64(d["q"], d["k"], d["v"], hq // hkv, 0.37, causal)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("lq,lkv,causal,hq,hkv", [
    (17, 17, True, 4, 1), (9, 23, True, 6, 2), (13, 13, False, 8, 8),
    (3, 3, True, 4, 4)])
def test_finite_sink_equals_sdpa_with_zero_key(lq, lkv, causal, hq, hkv):
    """A finite sink is a zero key whose additive bias is s_h and whose value
    row is zero: SDPA over [K; 0], [V; 0] with that bias column."""
    d = workloads.prefill_inputs([lq], [lkv], hq=hq, hkv=hkv, dim=16,
                                 dtype=torch.float32, seed=7 + lq, sink_std=2.0)
    got = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], hkv, hq // hkv, 0.25, causal)
    ref = _sdpa_fp64(d["q"], d["k"], d["v"], hq // hkv, 0.25, causal,
                     sinks=d["sinks"].double())
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_ragged_batch_equals_per_sequence():
    """Packed ragged batches give each sequence's own result."""
    lens_q, lens_kv = [5, 1, 12, 7], [5, 9, 12, 30]
    d = workloads.prefill_inputs(lens_q, lens_kv, hq=4, hkv=2, dim=8,
                                 dtype=torch.float32, seed=3, sink_std=1.5)
    got = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], 2, 2, 0.5, True)
    cq, ck = d["cu_seqlens_q"].tolist(), d["cu_seqlens_kv"].tolist()
    for b in range(4):
        ref = _sdpa_fp64(d["q"][cq[b]:cq[b + 1]], d["k"][ck[b]:ck[b + 1]],
                         d["v"][ck[b]:ck[b + 1]], 2, 0.5, True,
                         sinks=d["sinks"].double())
        np.testing.assert_allclose(got[cq[b]:cq[b + 1]], ref, rtol=1e-12,
                                   atol=1e-13)


def test_bf16_inputs_widened_exactly():
    """bf16 inputs are read as the exact values they encode."""
    d = workloads.prefill_inputs([11], hq=4, hkv=2, dim=16, dtype=torch.bfloat16,
                                 seed=5)
    got = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], 2, 2, 0.125, True)
    ref = oracle.prefill(d["q"].double(), d["k"].double(), d["v"].double(),
                         d["sinks"], d["cu_seqlens_q"], d["cu_seqlens_kv"], 2, 2,
                         0.125, True)
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------- O3
@pytest.mark.parametrize("sink", [-3.0, 0.0, 1.7, 20.0, -math.inf])
def test_all_keys_equal_closed_form(sink):
    """All keys equal to one vector kk: every visible key has logit
    x = scale * q.kk, so each weight is 1/(L_i + e^(s - x)) and
    out_i = (sum of the L_i visible v rows) / (L_i + e^(s - x))."""
    L, hq, dim, scale = 24, 2, 8, 0.3
    g = torch.Generator().manual_seed(11)
    q = torch.randn(L, hq, dim, generator=g, dtype=torch.float64)
    kk = torch.randn(dim, generator=g, dtype=torch.float64)
    k = kk.expand(L, 1, dim).clone()
    v = torch.randn(L, 1, dim, generator=g, dtype=torch.float64)
    sinks = torch.tensor([sink, sink / 2 if math.isfinite(sink) else sink])
    cu = torch.tensor([0, L], dtype=torch.int32)
    got = oracle.prefill(q, k, v, sinks, cu, cu, 1, hq, scale, True)
    qn, vn, kn = q.numpy(), v.numpy()[:, 0, :], kk.numpy()
    for i in range(L):
        for h in range(hq):
            x = scale * float(qn[i, h] @ kn)
            n = i + 1
            den = n + math.exp(float(sinks[h]) - x)
            np.testing.assert_allclose(got[i, h], vn[:n].sum(0) / den,
                                       rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------- O4
def test_unit_values_give_one_minus_sink_probability():
    """With every value row = 1 the output is sum_j w_j = 1 - p_sink,
    p_sink = e^s / (e^s + sum_j e^x_j), evaluated here with mpmath."""
    mpmath.mp.dps = 30
    lq, hq, hkv, dim, scale = 6, 4, 2, 8, 0.5
    d = workloads.prefill_inputs([lq], hq=hq, hkv=hkv, dim=dim,
                                 dtype=torch.float32, seed=21, sink_std=2.0)
    v = torch.ones_like(d["v"])
    got = oracle.prefill(d["q"], d["k"], v, d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], hkv, hq // hkv, scale, True)
    qn, kn, sn = d["q"].double().numpy(), d["k"].double().numpy(), d["sinks"].double().numpy()
    for i in range(lq):
        for h in range(hq):
            g = h // (hq // hkv)
            xs = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                                 for a, b in zip(qn[i, h], kn[j, g]))
                  for j in range(i + 1)]
            es = mpmath.exp(mpmath.mpf(float(sn[h])))
            p_sink = es / (es + mpmath.fsum(mpmath.exp(x) for x in xs))
            assert got[i, h] == pytest.approx(float(1 - p_sink), rel=1e-13, abs=1e-15)


# ---------------------------------------------------------------------- O5
def _brute_mp(q, k, v, sinks, group, scale, causal):
    """50-digit brute force: w_j = e^x_j / (sum_k e^x_k + e^s), no max shift."""
    mpmath.mp.dps = 50
    lq, hq, dim = q.shape
    lkv = k.shape[0]
    out = np.zeros((lq, hq, dim))
    for i in range(lq):
        for h in range(hq):
            g = h // group
            n = min(lkv, i + (lkv - lq) + 1) if causal else lkv
            n = max(n, 0)
            xs = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[i, h, e])) *
                                                  mpmath.mpf(float(k[j, g, e]))
                                                  for e in range(dim))
                  for j in range(n)]
            den = mpmath.fsum(mpmath.exp(x) for x in xs) + mpmath.exp(mpmath.mpf(float(sinks[h])))
            for e in range(dim):
                out[i, h, e] = float(mpmath.fsum(mpmath.exp(xs[j]) * mpmath.mpf(float(v[j, g, e]))
                                                 for j in range(n)) / den)
    return out


@pytest.mark.parametrize("lq,lkv,hq,hkv,dim,causal", [
    (4, 4, 2, 1, 4, True), (3, 8, 4, 2, 3, True), (5, 2, 2, 2, 4, False),
    (1, 7, 4, 1, 2, True)])
def test_mpmath_brute_force(lq, lkv, hq, hkv, dim, causal):
    d = workloads.prefill_inputs([lq], [lkv], hq=hq, hkv=hkv, dim=dim,
                                 dtype=torch.float32, seed=lq + 10 * lkv,
                                 sink_std=3.0, qkv_scale=2.0)
    got = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], hkv, hq // hkv, 0.7, causal)
    ref = _brute_mp(d["q"].double().numpy(), d["k"].double().numpy(),
                    d["v"].double().numpy(), d["sinks"].double().numpy(),
                    hq // hkv, 0.7, causal)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------- worked cases
def test_golden_worked_examples():
    with open(GOLDEN) as f:
        gold = json.load(f)
    for case in gold["prefill"]:
        q = torch.tensor(case["q"], dtype=torch.float64)
        k = torch.tensor(case["k"], dtype=torch.float64)
        v = torch.tensor(case["v"], dtype=torch.float64)
        sinks = [_f(s) for s in case["sinks"]]
        hkv = k.shape[1]
        cq = torch.tensor([0, q.shape[0]], dtype=torch.int32)
        ck = torch.tensor([0, k.shape[0]], dtype=torch.int32)
        got = oracle.prefill(q, k, v, torch.tensor(sinks, dtype=torch.float64), cq,
                             ck, hkv, case["group"], case["sm_scale"], case["causal"])
        np.testing.assert_allclose(got, np.array(case["expected"]), rtol=1e-14,
                                   atol=1e-15, err_msg=case["name"])
    for case in gold["merge"]:
        m = np.array([[_f(x) for x in case["m"]]])
        d = np.array([case["d"]])
        o = np.array([case["o"]])
        got = oracle.merge(m, d, o)
        np.testing.assert_allclose(got[0], case["expected"], rtol=1e-14,
                                   err_msg=case["name"])


def test_empty_key_set_gives_zero():
    """No visible key: finite sink takes all the mass (no value row) -> 0;
    sink = -inf -> empty softmax -> 0 by convention."""
    q = torch.randn(2, 2, 4, dtype=torch.float64)
    k = torch.zeros(0, 1, 4, dtype=torch.float64)
    cq = torch.tensor([0, 2], dtype=torch.int32)
    ck = torch.tensor([0, 0], dtype=torch.int32)
    got = oracle.prefill(q, k, k, torch.tensor([1.5, -math.inf]), cq, ck, 1, 2,
                         0.5, False)
    assert np.all(got == 0.0)


# ---------------------------------------------------------------------- O6
def _decode_case(lens, hq=8, hkv=2, dim=16, seed=0, sink_std=1.5):
    return workloads.decode_inputs(lens, hq=hq, hkv=hkv, dim=dim,
                                   dtype=torch.float32, seed=seed,
                                   sink_std=sink_std)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_split_merge_equals_unsplit(splits):
    d = _decode_case([0, 1, 15, 16, 17, 100, 257], seed=splits)
    full = oracle.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                               d["kv_lens"], d["sinks"], d["group"], 0.25)
    m, dd, o = oracle.decode_partials(d["q"], d["k_cache"], d["v_cache"],
                                      d["page_table"], d["kv_lens"], d["sinks"],
                                      d["group"], 0.25, splits)
    merged = oracle.merge(m, dd, o)
    np.testing.assert_allclose(merged, full, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("L,S,expect_tokens", [
    (85, 4, [32, 32, 21, 0]),          # 6 pages -> 2 per chunk, last chunk empty
    (128, 4, [32, 32, 32, 32]),        # 8 pages -> exactly 2 per chunk
    (20, 3, [16, 4, 0]),               # 2 pages -> 1 per chunk
    (0, 2, [0, 0]),                    # no keys at all
    (300, 7, [48, 48, 48, 48, 48, 48, 12])])
def test_split_bookkeeping_chunk_ranges_and_sink_once(L, S, expect_tokens):
    """Chunk c covers tokens [c*ppc*P, min((c+1)*ppc*P, L)) with
    ppc = ceil(ceil(L/P)/S); empty chunks are (-inf, 0, 0); the sink sits in
    chunk 0 only.  Checked with unit values and a zero query, so every logit
    is 0 and a chunk's d and o count its tokens."""
    d = _decode_case([L], hq=2, hkv=1, dim=4, seed=9)
    q0 = torch.zeros_like(d["q"])                          # all logits 0
    vc1 = torch.ones_like(d["v_cache"])
    sinks = torch.tensor([-math.inf, 0.5])
    m, dd, o = oracle.decode_partials(q0, d["k_cache"], vc1, d["page_table"],
                                      d["kv_lens"], sinks, 2, 0.25, S)
    for c in range(S):
        n = expect_tokens[c]
        if n == 0:
            assert m[0, 0, c] == -math.inf and dd[0, 0, c] == 0.0
            assert np.all(o[0, 0, c] == 0.0)
            if c == 0:      # chunk 0 keeps the sink even with no keys
                assert m[0, 1, 0] == 0.5 and dd[0, 1, 0] == 1.0
                assert np.all(o[0, 1, 0] == 0.0)
            else:
                assert m[0, 1, c] == -math.inf and dd[0, 1, c] == 0.0
            continue
        assert m[0, 0, c] == 0.0 and dd[0, 0, c] == n
        np.testing.assert_array_equal(o[0, 0, c], np.full(4, float(n)))
        # head 1: sink 0.5 > 0 sets m in chunk 0 only
        if c == 0:
            assert m[0, 1, c] == 0.5
            assert dd[0, 1, c] == pytest.approx(1.0 + n * math.exp(-0.5), rel=1e-15)
        else:
            assert m[0, 1, c] == 0.0 and dd[0, 1, c] == n


def test_sink_in_every_chunk_is_caught_by_closed_form():
    """Planted mistake (CPU only): counting the sink in every chunk of the
    split must break the all-keys-equal closed form that the correct merge
    satisfies."""
    lens, hq, dim, scale, S = [200], 2, 8, 0.3, 5
    d = _decode_case(lens, hq=hq, hkv=1, dim=dim, seed=4)
    kk = torch.randn(dim, generator=torch.Generator().manual_seed(2))
    kc = kk.view(1, 1, 1, dim).expand_as(d["k_cache"]).contiguous()
    sinks = torch.tensor([0.8, -1.1])
    m, dd, o = oracle.decode_partials(d["q"], kc, d["v_cache"], d["page_table"],
                                      d["kv_lens"], sinks, hq, scale, S)
    good = oracle.merge(m, dd, o)
    bad_d = dd.copy()
    for h in range(hq):
        for c in range(1, S):
            if m[0, h, c] != -math.inf:
                bad_d[0, h, c] += math.exp(float(sinks[h]) - m[0, h, c])
    bad = oracle.merge(m, bad_d, o)
    # closed form: all keys equal -> out = sum_j v_j / (L + e^(s - x))
    vsum = np.zeros((hq, dim))
    pt = d["page_table"][0].tolist()
    for t in range(lens[0]):
        vsum += d["v_cache"][pt[t // 16], 0, :, t % 16].double().numpy()
    for h in range(hq):
        x = scale * float(d["q"][0, h].double() @ kk.double())
        closed = vsum[h] / (lens[0] + math.exp(float(sinks[h]) - x))
        np.testing.assert_allclose(good[0, h], closed, rtol=1e-12, atol=1e-13)
        assert not np.allclose(bad[0, h], closed, rtol=1e-3, atol=1e-6)


# ---------------------------------------------------------------- O7 / O8
def _pack_paged(k, v, page, seed):
    """Scatter contiguous k/v [L, Hkv, D] into randomly placed pages
    (K page [Hkv][P][D], V page [Hkv][D][P])."""
    L, hkv, dim = k.shape
    npg = (L + page - 1) // page
    perm = torch.randperm(npg + 3, generator=torch.Generator().manual_seed(seed))[:npg]
    kc = torch.full((npg + 3, hkv, page, dim), float("nan"), dtype=k.dtype)
    vc = torch.full((npg + 3, hkv, dim, page), float("nan"), dtype=v.dtype)
    for t in range(L):
        kc[perm[t // page], :, t % page, :] = k[t]
        vc[perm[t // page], :, :, t % page] = v[t]
    return kc, vc, perm.to(torch.int32).view(1, npg)


@pytest.mark.parametrize("L", [1, 16, 37, 130])
def test_decode_equals_last_row_of_causal_prefill(L):
    hq, hkv, dim = 8, 2, 16
    d = workloads.prefill_inputs([L], hq=hq, hkv=hkv, dim=dim, dtype=torch.float32,
                                 seed=L, sink_std=1.5)
    pre = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], hkv, hq // hkv, 0.25, True)
    kc, vc, pt = _pack_paged(d["k"], d["v"], 16, seed=L + 1)
    dec = oracle.decode_paged(d["q"][L - 1:L], kc, vc, pt, torch.tensor([L]),
                              d["sinks"], hq // hkv, 0.25)
    np.testing.assert_allclose(dec[0], pre[L - 1], rtol=1e-13, atol=1e-14)


def test_page_permutation_invariance_is_exact():
    """Two physical placements of the same logical cache give bitwise equal
    fp64 results (the page walk reads the same values in the same order);
    unread NaN slots and pages never leak in."""
    L, hq, hkv, dim = 53, 4, 2, 8
    d = workloads.prefill_inputs([L], hq=hq, hkv=hkv, dim=dim, dtype=torch.float32,
                                 seed=77)
    outs = []
    for seed in (1, 2):
        kc, vc, pt = _pack_paged(d["k"], d["v"], 16, seed)
        outs.append(oracle.decode_paged(d["q"][:1], kc, vc, pt, torch.tensor([L]),
                                        d["sinks"], hq // hkv, 0.3))
    assert np.all(np.isfinite(outs[0]))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_sampled_rows_match_full():
    d = _decode_case([40, 90, 3], seed=5)
    full = oracle.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                               d["kv_lens"], d["sinks"], d["group"], 0.25)
    rows = ([2, 0, 1], [7, 3, 0])
    part = oracle.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                               d["kv_lens"], d["sinks"], d["group"], 0.25, rows=rows)
    for r, (b, h) in enumerate(zip(*rows)):
        np.testing.assert_array_equal(part[r], full[b, h])
    p = workloads.prefill_inputs([7, 9], hq=4, hkv=2, dim=8, dtype=torch.float32, seed=1)
    pf = oracle.prefill(p["q"], p["k"], p["v"], p["sinks"], p["cu_seqlens_q"],
                        p["cu_seqlens_kv"], 2, 2, 0.5, True)
    pr = oracle.prefill(p["q"], p["k"], p["v"], p["sinks"], p["cu_seqlens_q"],
                        p["cu_seqlens_kv"], 2, 2, 0.5, True, rows=([0, 15, 8], [3, 0, 2]))
    for r, (t, h) in enumerate(zip([0, 15, 8], [3, 0, 2])):
        np.testing.assert_array_equal(pr[r], pf[t, h])


# ------------------------------------------------- O9: paged (chunked) prefill
def _paged_prefill_case(lens_q, lens_kv, hq=8, hkv=2, dim=16, seed=0, fill=float("nan")):
    d = workloads.prefill_inputs(lens_q, lens_kv, hq=hq, hkv=hkv, dim=dim,
                                 dtype=torch.float32, seed=seed, sink_std=1.5)
    d.update(workloads.pack_paged(d["k"], d["v"], d["lens_kv"], seed=seed + 1,
                                  extra_pages=3, fill=fill))
    return d


@pytest.mark.parametrize("lens_q,lens_kv,causal", [
    ([5, 20, 1], [37, 20, 64], True),      # new tokens at the end of a longer cache
    ([5, 20, 1], [37, 20, 64], False),
    ([9, 3], [4, 0], True),                # more queries than keys; an empty cache
    ([16, 17], [16, 33], True)])           # page-boundary lengths
def test_paged_prefill_equals_ragged_prefill_bitwise(lens_q, lens_kv, causal):
    """The paged oracle on a cache scattered by pack_paged (random placement,
    NaN in every slot no key owns) reads the same values in the same order as
    the ragged oracle on the contiguous k / v, so the fp64 results are equal
    bit for bit; a wrong page index, slot, or V-page orientation breaks it."""
    d = _paged_prefill_case(lens_q, lens_kv, seed=len(lens_q) + int(causal))
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], 2, 4, 0.3, causal)
    got = oracle.prefill_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                               d["cu_seqlens_q"], d["kv_lens"], d["sinks"], 4, 0.3, causal)
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got, ref)


def test_paged_prefill_single_query_equals_decode():
    """One query token per sequence with the causal rule is exactly decode."""
    d = _paged_prefill_case([1, 1, 1, 1], [1, 16, 40, 129], seed=11)
    pre = oracle.prefill_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                               d["cu_seqlens_q"], d["kv_lens"], d["sinks"], 4, 0.25, True)
    dec = oracle.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                              d["kv_lens"], d["sinks"], 4, 0.25)
    np.testing.assert_array_equal(pre, dec)


@pytest.mark.parametrize("lq,lkv", [(6, 40), (40, 40), (50, 40), (1, 64)])
def test_paged_prefill_bottom_right_causal_closed_form(lq, lkv):
    """q = 0 makes every logit 0; one-hot values v_j = e_j then give
    out[i, d] = 1 / (n_i + e^s) for d < n_i and 0 beyond, where n_i =
    clip(i + lkv - lq + 1, 0, lkv) counts the keys row i sees (the queries
    are the last lq positions)."""
    dim = 64
    d = _paged_prefill_case([lq], [lkv], hq=2, hkv=1, dim=dim, seed=lq)
    q0 = torch.zeros_like(d["q"])
    v1 = torch.zeros((lkv, 1, dim))
    v1[torch.arange(lkv), 0, torch.arange(lkv)] = 1.0
    pk = workloads.pack_paged(d["k"], v1, [lkv], seed=5, fill=float("nan"))
    sinks = torch.tensor([0.7, -math.inf])
    got = oracle.prefill_paged(q0, pk["k_cache"], pk["v_cache"], pk["page_table"],
                               d["cu_seqlens_q"], pk["kv_lens"], sinks, 2, 0.125, True)
    for i in range(lq):
        n = min(max(i + lkv - lq + 1, 0), lkv)
        for h in range(2):
            s = float(sinks[h])                 # the fp32 value the oracle reads
            want = np.zeros(dim)
            if n > 0:
                want[:n] = 1.0 / (n + math.exp(s))
            np.testing.assert_allclose(got[i, h], want, rtol=1e-15, atol=0)


# ------------------------------------------------------ O10: split-KV prefill
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_split_merge_equals_unsplit(splits, causal):
    """Merging the split prefill states gives the unsplit result, for the
    ragged and the paged layout alike."""
    d = _paged_prefill_case([3, 30, 1, 0], [85, 30, 17, 5], seed=splits)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                         d["cu_seqlens_kv"], 2, 4, 0.3, causal)
    parts = oracle.prefill_partials(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"],
                                    d["cu_seqlens_kv"], 2, 4, 0.3, causal, splits)
    np.testing.assert_allclose(oracle.merge(*parts), ref, rtol=1e-12, atol=1e-13)
    pp = oracle.prefill_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                              d["cu_seqlens_q"], d["kv_lens"], d["sinks"], 4, 0.3, causal,
                              splits=splits)
    for a, b in zip(pp, parts):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_split_bookkeeping_causal_rows(paged):
    """Chunks follow the sequence's key range (85 keys, 6 units of 16, S = 4
    -> 32 keys per chunk) and are clipped to each row's causal limit: rows
    0..2 of 3 new tokens see 83, 84, 85 keys, so chunk 2 holds 19, 20, 21
    keys and chunk 3 none.  q = 0 and unit values make d and o count keys;
    the sink (0.5) sits in chunk 0 only."""
    d = _paged_prefill_case([3], [85], hq=2, hkv=1, dim=4, seed=3)
    q0 = torch.zeros_like(d["q"])
    v1 = torch.ones_like(d["v"])
    sinks = torch.tensor([-math.inf, 0.5])
    if paged:
        pk = workloads.pack_paged(d["k"], v1, [85], seed=8, fill=float("nan"))
        m, dd, o = oracle.prefill_paged(q0, pk["k_cache"], pk["v_cache"], pk["page_table"],
                                        d["cu_seqlens_q"], pk["kv_lens"], sinks, 2, 0.3,
                                        True, splits=4)
    else:
        m, dd, o = oracle.prefill_partials(q0, d["k"], v1, sinks, d["cu_seqlens_q"],
                                           d["cu_seqlens_kv"], 1, 2, 0.3, True, 4)
    expect = {0: [32, 32, 19, 0], 1: [32, 32, 20, 0], 2: [32, 32, 21, 0]}
    for i, counts in expect.items():
        for c, n in enumerate(counts):
            if n == 0:
                assert m[i, 0, c] == -math.inf and dd[i, 0, c] == 0.0
                assert m[i, 1, c] == -math.inf and dd[i, 1, c] == 0.0
                assert np.all(o[i, :, c] == 0.0)
                continue
            assert m[i, 0, c] == 0.0 and dd[i, 0, c] == n
            np.testing.assert_array_equal(o[i, 0, c], np.full(4, float(n)))
            if c == 0:
                assert m[i, 1, 0] == 0.5
                assert dd[i, 1, 0] == pytest.approx(1.0 + n * math.exp(-0.5), rel=1e-15)
                np.testing.assert_allclose(o[i, 1, 0], n * math.exp(-0.5), rtol=1e-15)
            else:
                assert m[i, 1, c] == 0.0 and dd[i, 1, c] == n


def test_prefill_split_empty_rows_keep_sink_in_chunk_zero():
    """A row that sees no key (more queries than keys) has (s, 1, 0) in
    chunk 0 and (-inf, 0, 0) elsewhere."""
    d = _paged_prefill_case([6], [2], hq=2, hkv=1, dim=4, seed=2)
    sinks = torch.tensor([1.25, -math.inf])
    m, dd, o = oracle.prefill_partials(d["q"], d["k"], d["v"], sinks, d["cu_seqlens_q"],
                                       d["cu_seqlens_kv"], 1, 2, 0.3, True, 3)
    for i in range(4):                       # rows 0..3 see 0 keys
        assert m[i, 0, 0] == 1.25 and dd[i, 0, 0] == 1.0 and np.all(o[i, 0, 0] == 0)
        assert m[i, 1, 0] == -math.inf and dd[i, 1, 0] == 0.0
        for c in (1, 2):
            assert m[i, :, c].tolist() == [-math.inf, -math.inf]
            assert np.all(dd[i, :, c] == 0) and np.all(o[i, :, c] == 0)
