"""GPU parity of paged decode, split-KV partials and the merge (MI355X).

Every comparison is against the fp64 oracle on the same (rounded) inputs, or
is a bit-exact construction whose answer is known without arithmetic.
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


def _to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run_decode(lib, d, splits):
    """Decode through the C ABI; splits > 1 goes through attn_sink_merge.
    Outputs and partial states start as NaN, so that any element the grid
    never writes fails the comparison."""
    q = d["q"]
    nan = float("nan")
    if splits == 1:
        out = torch.full_like(q, nan)
        lib.attn_sink_decode_paged(q, d["k_cache"], d["v_cache"], d["page_table"],
                                   d["kv_lens"], d["sinks"], d["group"], d["sm_scale"], 1,
                                   out=out)
        return out, None
    b, hq, dim = q.shape
    f32 = dict(device=q.device, dtype=torch.float32)
    pm = torch.full((b, hq, splits), nan, **f32)
    pd = torch.full((b, hq, splits), nan, **f32)
    po = torch.full((b, hq, splits, dim), nan, **f32)
    lib.attn_sink_decode_paged(q, d["k_cache"], d["v_cache"], d["page_table"], d["kv_lens"],
                               d["sinks"], d["group"], d["sm_scale"], splits, partial_m=pm,
                               partial_d=pd, partial_o=po)
    out = torch.full_like(q, nan)
    lib.attn_sink_merge(pm, pd, po, out=out, out_dtype=q.dtype)
    return out, (pm, pd, po)


def oracle_decode(d, rows=None):
    return oracle.decode_paged(d["q"].cpu(), d["k_cache"].cpu(), d["v_cache"].cpu(),
                               d["page_table"].cpu(), d["kv_lens"].cpu(), d["sinks"].cpu(),
                               d["group"], d["sm_scale"], rows=rows)


LENS = [0, 1, 15, 16, 17, 31, 100, 4097]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("group", [1, 4, 8, 16])
@pytest.mark.parametrize("splits", [1, 2, 7, 64, 300])
def test_decode_sweep_matches_oracle(lib, dtype, group, splits):
    d = workloads.decode_inputs(LENS, hq=2 * group, hkv=2, dtype=dtype, seed=group * 100 + splits,
                                sink_std=1.5, extra_pages=3)
    dd = _to_dev(d)
    out, _ = run_decode(lib, dd, splits)
    torch.cuda.synchronize()
    ref = oracle_decode(d)
    assert_close(out, ref, dtype, "decode G=%d S=%d %s" % (group, splits, dtype))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [1, 3])
def test_decode_more_than_64_sequences(lib, dtype, splits):
    """Past 64 sequences the grid's sequence index is used as is (no ranking
    by length)."""
    g = torch.Generator().manual_seed(70 + splits)
    lens = torch.randint(0, 300, (70,), generator=g).tolist()
    d = workloads.decode_inputs(lens, hq=8, hkv=2, dtype=dtype, seed=71 + splits, sink_std=1.5)
    out, _ = run_decode(lib, _to_dev(d), splits)
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(d), dtype, "decode B=70 S=%d" % splits)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_partials_match_oracle_and_bookkeeping(lib, dtype):
    """Chunk states: the empty/non-empty pattern and chunk 0's sink-only state
    are exact; finite m, d and o/d match the oracle's partials."""
    lens, S = [0, 5, 16, 40, 200, 1000], 6
    d = workloads.decode_inputs(lens, hq=8, hkv=2, dtype=dtype, seed=31, sink_std=1.5)
    dd = _to_dev(d)
    _, (pm, pd, po) = run_decode(lib, dd, S)
    torch.cuda.synchronize()
    rm, rd, ro = oracle.decode_partials(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                        d["kv_lens"], d["sinks"], d["group"], d["sm_scale"], S)
    gm, gd, go = pm.cpu().double().numpy(), pd.cpu().double().numpy(), po.cpu().double().numpy()
    empty = rm == -math.inf
    np.testing.assert_array_equal(gm == -math.inf, empty)
    np.testing.assert_array_equal(gd[empty], 0.0)
    np.testing.assert_array_equal(go[empty], 0.0)
    # zero-length sequence: chunk 0 is exactly the sink state (s, 1, 0)
    np.testing.assert_array_equal(gd[0, :, 0], 1.0)
    np.testing.assert_array_equal(go[0, :, 0], 0.0)
    np.testing.assert_allclose(gm[0, :, 0], d["sinks"].double().numpy(), rtol=1e-6)
    live = ~empty
    np.testing.assert_allclose(gm[live], rm[live], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(gd[live], rd[live], rtol=1e-3 if dtype == torch.bfloat16 else 1e-5)
    atol, rtol = tol_for(dtype)
    on = go[live] / gd[live][:, None]
    rn = ro[live] / rd[live][:, None]
    assert np.all(np.abs(on - rn) <= atol + rtol * np.abs(rn))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_one_hot_is_bit_exact(lib, out_dtype):
    """Exactly one chunk per row has a finite m (others (-inf, 0, 0)) and
    d = 2^k: the merged output must be o / 2^k exactly (then RNE to bf16)."""
    B, H, S, D = 3, 8, 11, 64
    g = torch.Generator().manual_seed(5)
    m = torch.full((B, H, S), -math.inf)
    dd = torch.zeros(B, H, S)
    o = torch.zeros(B, H, S, D)
    pick = torch.randint(0, S, (B, H), generator=g)
    kexp = torch.randint(-3, 6, (B, H), generator=g)
    ohot = torch.randn(B, H, D, generator=g)
    for b in range(B):
        for h in range(H):
            c = int(pick[b, h])
            m[b, h, c] = float(torch.randn(1, generator=g)) * 5
            dd[b, h, c] = 2.0 ** int(kexp[b, h])
            o[b, h, c] = ohot[b, h]
    out = lib.attn_sink_merge(m.to(DEV), dd.to(DEV), o.to(DEV), out_dtype=out_dtype)
    expect = ohot / (2.0 ** kexp.float()).unsqueeze(-1)
    torch.testing.assert_close(out.cpu(), expect.to(out_dtype), rtol=0, atol=0)


def test_merge_all_empty_rows_give_zero(lib):
    m = torch.full((2, 4, 3), -math.inf, device=DEV)
    z = torch.zeros((2, 4, 3), device=DEV)
    o = torch.zeros((2, 4, 3, 64), device=DEV)
    out = lib.attn_sink_merge(m, z, o, out_dtype=torch.float32)
    assert torch.all(out == 0)


def _logical_to_paged(k, v, page, perm_seed, extra=5, fill=float("nan")):
    """Scatter contiguous per-sequence k/v [L, Hkv, D] lists into one paged
    cache with a random physical placement."""
    lens = [x.shape[0] for x in k]
    hkv, dim = k[0].shape[1], k[0].shape[2]
    npg = [(L + page - 1) // page for L in lens]
    total = sum(npg) + extra
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(perm_seed))
    kc = torch.full((total, hkv, page, dim), fill, dtype=k[0].dtype)
    vc = torch.full((total, hkv, dim, page), fill, dtype=v[0].dtype)
    pt = torch.full((len(lens), max(1, max(npg))), -1, dtype=torch.int32)
    off = 0
    for b, L in enumerate(lens):
        for p in range(npg[b]):
            phys = int(perm[off + p])
            pt[b, p] = phys
            t0, t1 = p * page, min(L, (p + 1) * page)
            kc[phys, :, :t1 - t0, :] = k[b][t0:t1].permute(1, 0, 2)
            vc[phys, :, :, :t1 - t0] = v[b][t0:t1].permute(1, 2, 0)
        off += npg[b]
    return kc, vc, pt


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [1, 4])
def test_page_permutation_invariance_and_tail_poison(lib, dtype, splits):
    """Two physical placements of the same logical cache give bitwise equal
    outputs; NaN in unused page slots and unused pages never leaks in."""
    lens, hq, hkv = [1, 17, 64, 333], 8, 2
    g = torch.Generator().manual_seed(8)
    ks = [torch.randn(L, hkv, 64, generator=g).to(dtype) for L in lens]
    vs = [torch.randn(L, hkv, 64, generator=g).to(dtype) for L in lens]
    q = torch.randn(len(lens), hq, 64, generator=g).to(dtype)
    sinks = torch.randn(hq, generator=g)
    outs = []
    for seed, fill in ((1, float("nan")), (2, 0.0)):
        kc, vc, pt = _logical_to_paged(ks, vs, 16, seed, fill=fill)
        d = dict(q=q, k_cache=kc, v_cache=vc, page_table=pt,
                 kv_lens=torch.tensor(lens, dtype=torch.int32), sinks=sinks, group=hq // hkv,
                 sm_scale=0.125)
        out, _ = run_decode(lib, _to_dev(d), splits)
        outs.append(out.cpu())
    assert torch.all(torch.isfinite(outs[0].float()))
    assert torch.equal(outs[0], outs[1])
    ref = oracle_decode(dict(q=q, k_cache=kc, v_cache=vc, page_table=pt,
                             kv_lens=torch.tensor(lens, dtype=torch.int32), sinks=sinks,
                             group=hq // hkv, sm_scale=0.125))
    assert_close(outs[1], ref, dtype, "permuted pages")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [1, 3, 64])
def test_one_hot_retrieval_is_bit_exact(lib, dtype, splits):
    """sink = -inf and one key per sequence whose logit is > 1000 above every
    other: all other weights underflow to exactly 0, d = 1 and the output is
    that key's value row bit for bit, whichever page and chunk holds it."""
    lens, hq, hkv = [5, 16, 17, 700, 1601], 8, 2
    g = torch.Generator().manual_seed(12)
    targets = [int(torch.randint(0, L, (1,), generator=g)) for L in lens]
    ks, vs = [], []
    for L, t in zip(lens, targets):
        k = torch.rand(L, hkv, 64, generator=g) * 2 - 1
        k[:, :, 0] = torch.rand(L, hkv, generator=g) * 2 - 1
        k[t, :, 0] = 128.0
        ks.append(k.to(dtype))
        vs.append(torch.randn(L, hkv, 64, generator=g).to(dtype))
    q = torch.zeros(len(lens), hq, 64)
    q[:, :, 0] = 64.0
    q = q.to(dtype)
    kc, vc, pt = _logical_to_paged(ks, vs, 16, 3)
    d = dict(q=q, k_cache=kc, v_cache=vc, page_table=pt,
             kv_lens=torch.tensor(lens, dtype=torch.int32),
             sinks=torch.full((hq,), -math.inf), group=hq // hkv, sm_scale=0.125)
    out, _ = run_decode(lib, _to_dev(d), splits)
    out = out.cpu()
    for b, t in enumerate(targets):
        for h in range(hq):
            assert torch.equal(out[b, h], vs[b][t, h // (hq // hkv)]), (b, h)


@pytest.mark.parametrize("splits", [1, 5])
def test_decode_deterministic(lib, splits):
    """Split decode + merge and the single launch (whose waves merge in LDS)
    both reduce in a fixed order."""
    d = _to_dev(workloads.decode_inputs([900, 33, 4000], hq=16, hkv=2, seed=3))
    a, _ = run_decode(lib, d, splits)
    b, _ = run_decode(lib, d, splits)
    assert torch.equal(a, b)


def test_decode_c3_full_matches_oracle(lib):
    """Paged decode workload: B=64, kv_len U[512,8192], 64/8 heads, bf16."""
    d = workloads.workload(3, device="cpu", cache_device=DEV)
    dd = _to_dev(d)
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ref = oracle_decode(host)
    from gqa_attention_sinks_initialised_amd import default_num_splits
    for splits in (1, default_num_splits(d["kv_lens"].tolist(), 8)):
        out, _ = run_decode(lib, dd, splits)
        torch.cuda.synchronize()
        assert_close(out, ref, torch.bfloat16, "C3 splits=%d" % splits)


def test_decode_c4_full_matches_oracle(lib):
    """Long split-KV decode workload: B=4, kv_len 131072, 64 splits.  Every
    output element, and every one of the 256 x 64 partial states through its
    unique parts (m + ln d and o / d), against the fp64 oracle (a few seconds
    of oracle time on 16 host cores)."""
    d = workloads.workload(4, device="cpu", cache_device=DEV)
    dd = _to_dev(d)
    out, (pm, pd, po) = run_decode(lib, dd, 64)
    torch.cuda.synchronize()
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    assert_close(out, oracle_decode(host), torch.bfloat16, "C4 full")
    rm, rd, ro = oracle.decode_partials(host["q"], host["k_cache"], host["v_cache"],
                                        host["page_table"], host["kv_lens"], host["sinks"],
                                        8, host["sm_scale"], 64)
    gm, gd, go = (t.cpu().double().numpy() for t in (pm, pd, po))
    assert np.all(np.isfinite(gm)) and np.all(gd > 0), "every C4 chunk holds keys"
    np.testing.assert_allclose(gm + np.log(gd), rm + np.log(rd), rtol=0, atol=1e-4)
    atol, rtol = tol_for(torch.bfloat16)
    on, rn = go / gd[..., None], ro / rd[..., None]
    assert np.all(np.abs(on - rn) <= atol + rtol * np.abs(rn)), float(np.abs(on - rn).max())


@pytest.mark.parametrize("splits", [1, 3])
def test_decode_pages_past_4gib(lib, splits):
    """Pages may sit anywhere in caches larger than 4 GiB: the result is bit
    for bit that of the compact cache holding the same logical pages."""
    d = _to_dev(workloads.decode_inputs([37, 300, 1], hq=8, hkv=2, dtype=torch.bfloat16,
                                        seed=91, sink_std=1.5))
    small, _ = run_decode(lib, d, splits)
    kc, vc, pt = d["k_cache"], d["v_cache"], d["page_table"]
    block = kc[0].numel() * kc.element_size()
    nbig = -(-(5 << 30) // block)
    big = dict(d)
    big["k_cache"] = torch.empty((nbig,) + tuple(kc.shape[1:]), dtype=kc.dtype, device=DEV)
    big["v_cache"] = torch.empty((nbig,) + tuple(vc.shape[1:]), dtype=vc.dtype, device=DEV)
    n = kc.shape[0]
    new_ids = nbig - 1 - torch.arange(n, device=DEV)
    big["k_cache"][new_ids] = kc
    big["v_cache"][new_ids] = vc
    valid = (pt >= 0) & (pt < n)
    big["page_table"] = torch.where(valid, nbig - 1 - pt, pt).to(torch.int32)
    assert int(big["page_table"][valid].min()) * block >= (4 << 30)
    out, _ = run_decode(lib, big, splits)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), small.cpu().view(torch.int16))


def test_binding_rejects_misshaped_buffers(lib):
    """The C ABI cannot see buffer sizes, so the binding checks every
    caller-supplied output and partial buffer before anything is launched."""
    d = _to_dev(workloads.decode_inputs([40, 7], hq=8, hkv=2, dtype=torch.bfloat16, seed=1))
    args = (d["q"], d["k_cache"], d["v_cache"], d["page_table"], d["kv_lens"], d["sinks"],
            d["group"], d["sm_scale"])
    f32 = dict(device=DEV, dtype=torch.float32)
    with pytest.raises(ValueError):
        lib.attn_sink_decode_paged(*args, 1, out=torch.empty((2, 8, 32), device=DEV,
                                                             dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        lib.attn_sink_decode_paged(*args, 1, out=torch.empty((2, 8, 64), device=DEV,
                                                             dtype=torch.float32))
    with pytest.raises(ValueError):
        lib.attn_sink_decode_paged(*args, 3, partial_m=torch.empty((2, 8, 2), **f32))
    with pytest.raises(ValueError):
        lib.attn_sink_decode_paged(*args, 3, partial_o=torch.empty((2, 8, 3, 64), device=DEV,
                                                                   dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        lib.attn_sink_decode_paged(d["q"][:, :, :32].contiguous(), *args[1:], 1)
    pm, pd, po = (torch.zeros((2, 8, 3), **f32), torch.zeros((2, 8, 3), **f32),
                  torch.zeros((2, 8, 3, 64), **f32))
    with pytest.raises(ValueError):
        lib.attn_sink_merge(pm, pd, po, out=torch.empty((2, 8, 63), **f32))
    with pytest.raises(ValueError):
        lib.attn_sink_merge(pm, pd.double(), po)
    with pytest.raises(ValueError):
        lib.attn_sink_merge(pm, pd, po[:, :, :2].contiguous())
    with pytest.raises(ValueError):
        lib.attn_sink_merge(pm, pd, po, out=torch.empty((2, 8, 64), **f32),
                            out_dtype=torch.bfloat16)


def test_explicit_side_stream_gives_the_default_stream_result(lib):
    """Calls take an explicit stream; the result on a side stream is the
    default stream's, bit for bit (the decode kernels are deterministic)."""
    d = _to_dev(workloads.decode_inputs([300, 17, 1000], hq=16, hkv=2, dtype=torch.bfloat16,
                                        seed=3))
    args = (d["q"], d["k_cache"], d["v_cache"], d["page_table"], d["kv_lens"], d["sinks"],
            d["group"], d["sm_scale"])
    ref = lib.attn_sink_merge(*lib.attn_sink_decode_paged(*args, 3), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        parts = lib.attn_sink_decode_paged(*args, 3, stream=side)
        got = lib.attn_sink_merge(*parts, out_dtype=torch.bfloat16, stream=side)
    side.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
