"""The whole path can be captured into a HIP graph and replayed.

The library only enqueues kernels on the caller's stream: no host
synchronisation, no device-to-host copy, no memset and no allocation.  Page
"Fast embeddings on GPUs", section "CUDA Graph Management": the serving
engine captures one graph per (sequence count, token-count bucket), pads
token counts to multiples of 64 or 256, and replays the graph with new
contents in the same buffers.  So a graph captured once per bucket must
give the right answer, against the fp64 oracle, for every set of lengths,
offsets, page tables and values that fits the bucket, replay after replay,
with the program's own eager work and synchronisations between the replays.
"""
import math

import pytest
import torch

import oracle
import workloads
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")
BF16 = torch.bfloat16


def _dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def test_capture_and_replay_matches_eager_and_oracle(lib):
    """Prefill + split decode + merge + single-launch (unsplit) decode + split
    chunked (paged) prefill + merge, captured once: every replay gives the
    eager bits, and those match the oracle."""
    p = _dev(workloads.prefill_inputs([300, 77], hq=16, hkv=2, dtype=BF16, seed=3,
                                      sink_std=1.5))
    dh = workloads.decode_inputs([900, 33, 4000], hq=16, hkv=2, dtype=BF16, seed=4,
                                 sink_std=1.5)
    d = _dev(dh)
    S = 7
    out_p = torch.empty_like(p["q"])
    out_d = torch.empty_like(d["q"])
    out_d1 = torch.empty_like(d["q"])
    f32 = dict(device=DEV, dtype=torch.float32)
    pm = torch.empty((3, 16, S), **f32)
    pd = torch.empty((3, 16, S), **f32)
    po = torch.empty((3, 16, S, 64), **f32)

    # chunked prefill against a paged cache, split 3 ways, then merged
    ch = workloads.prefill_inputs([40, 9], [700, 130], hq=16, hkv=2, dtype=BF16, seed=5,
                                  sink_std=1.5)
    ch.update(workloads.pack_paged(ch["k"], ch["v"], ch["lens_kv"], seed=6))
    c = _dev(ch)
    SC = 3
    cm = torch.empty((49, 16, SC), **f32)
    cd = torch.empty((49, 16, SC), **f32)
    co = torch.empty((49, 16, SC, 64), **f32)
    out_c = torch.empty_like(c["q"])

    def path():
        lib.attn_sink_prefill(p["q"], p["k"], p["v"], p["sinks"], p["cu_seqlens_q"],
                              p["cu_seqlens_kv"], 300, p["group"], p["sm_scale"], True, out=out_p)
        lib.attn_sink_decode_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                   d["kv_lens"], d["sinks"], d["group"], d["sm_scale"], S,
                                   partial_m=pm, partial_d=pd, partial_o=po)
        lib.attn_sink_merge(pm, pd, po, out=out_d)
        lib.attn_sink_decode_paged(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                   d["kv_lens"], d["sinks"], d["group"], d["sm_scale"], 1,
                                   out=out_d1)
        lib.attn_sink_prefill_paged(c["q"], c["k_cache"], c["v_cache"], c["page_table"],
                                    c["cu_seqlens_q"], c["kv_lens"], c["sinks"], 40, c["group"],
                                    c["sm_scale"], True, num_splits=SC, partial_m=cm,
                                    partial_d=cd, partial_o=co)
        lib.attn_sink_merge(cm, cd, co, out=out_c)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_p, ref_d, ref_c = out_p.clone(), out_d.clone(), out_c.clone()
    ref_d1 = out_d1.clone()
    ph = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    assert_close(ref_p.cpu(), oracle.prefill(ph["q"], ph["k"], ph["v"], ph["sinks"],
                                             ph["cu_seqlens_q"], ph["cu_seqlens_kv"], 2, 8,
                                             ph["sm_scale"], True), BF16, "eager prefill")
    ref_dec = oracle.decode_paged(dh["q"], dh["k_cache"], dh["v_cache"], dh["page_table"],
                                  dh["kv_lens"], dh["sinks"], 8, dh["sm_scale"])
    assert_close(ref_d.cpu(), ref_dec, BF16, "eager decode")
    assert_close(ref_d1.cpu(), ref_dec, BF16, "eager single-launch decode")
    assert_close(ref_c.cpu(), oracle.prefill_paged(ch["q"], ch["k_cache"], ch["v_cache"],
                                                   ch["page_table"], ch["cu_seqlens_q"],
                                                   ch["kv_lens"], ch["sinks"], 8,
                                                   ch["sm_scale"], True), BF16, "eager chunked")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    for i in range(4):
        out_p.fill_(NAN)
        out_d.fill_(NAN)
        out_d1.fill_(NAN)
        out_c.fill_(NAN)
        pm.fill_(NAN)
        cm.fill_(NAN)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_p, ref_p), "prefill replay %d" % i
        assert torch.equal(out_d, ref_d), "decode+merge replay %d" % i
        assert torch.equal(out_d1, ref_d1), "single-launch decode replay %d" % i
        assert torch.equal(out_c, ref_c), "chunked prefill+merge replay %d" % i
        path()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out_p, ref_p) and torch.equal(out_d, ref_d)
        assert torch.equal(out_c, ref_c) and torch.equal(out_d1, ref_d1)


@pytest.mark.parametrize("bucket", [128, 256])
def test_bucketed_graph_replays_new_contents_match_oracle(lib, bucket):
    """One graph per token-count bucket (a multiple of 64): ragged prefill of
    up to `bucket` tokens in 3 sequences, and split paged decode + merge of 3
    sequences over a cache of fixed capacity.  The graph is captured once;
    each replay follows a fresh draw of lengths, offsets, page placement and
    values copied into the captured buffers, and every output row is
    compared with the oracle on that draw."""
    B, HQ, HKV, S = 3, 16, 2, 5
    MAXP, NPAGES = 64, 3 * 64
    f32 = dict(device=DEV, dtype=torch.float32)
    i32 = dict(device=DEV, dtype=torch.int32)
    # captured (static) buffers
    q = torch.zeros((bucket, HQ, 64), device=DEV, dtype=BF16)
    k = torch.zeros((bucket, HKV, 64), device=DEV, dtype=BF16)
    v = torch.zeros((bucket, HKV, 64), device=DEV, dtype=BF16)
    sinks = torch.zeros((HQ,), **f32)
    cu = torch.zeros((B + 1,), **i32)
    out_p = torch.zeros_like(q)
    qd = torch.zeros((B, HQ, 64), device=DEV, dtype=BF16)
    kc = torch.zeros((NPAGES, HKV, 16, 64), device=DEV, dtype=BF16)
    vc = torch.zeros((NPAGES, HKV, 64, 16), device=DEV, dtype=BF16)
    pt = torch.zeros((B, MAXP), **i32)
    kv_lens = torch.zeros((B,), **i32)
    dsinks = torch.zeros((HQ,), **f32)
    pm = torch.zeros((B, HQ, S), **f32)
    pd = torch.zeros((B, HQ, S), **f32)
    po = torch.zeros((B, HQ, S, 64), **f32)
    out_d = torch.zeros_like(qd)

    def path():
        lib.attn_sink_prefill(q, k, v, sinks, cu, cu, bucket, HQ // HKV, 0.125, True, out=out_p)
        lib.attn_sink_decode_paged(qd, kc, vc, pt, kv_lens, dsinks, HQ // HKV, 0.125, S,
                                   partial_m=pm, partial_d=pd, partial_o=po)
        lib.attn_sink_merge(pm, pd, po, out=out_d)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()

    gen = torch.Generator().manual_seed(bucket)
    for draw in range(3):
        # prefill lengths: 3 sequences, total within the bucket, one may be empty
        cuts = sorted(torch.randint(0, bucket + 1, (2,), generator=gen).tolist())
        total = int(torch.randint(bucket // 2, bucket + 1, (1,), generator=gen))
        lens = [min(cuts[0], total), min(cuts[1], total) - min(cuts[0], total),
                total - min(cuts[1], total)]
        pin = workloads.prefill_inputs(lens, hq=HQ, hkv=HKV, dtype=BF16, seed=10 * bucket + draw,
                                       sink_std=1.5)
        q.fill_(NAN)
        k.fill_(NAN)
        v.fill_(NAN)
        q[:total] = pin["q"].to(DEV)
        k[:total] = pin["k"].to(DEV)
        v[:total] = pin["v"].to(DEV)
        sinks.copy_(pin["sinks"])
        cu.copy_(pin["cu_seqlens_q"])
        # decode: lengths up to the capacity of each sequence's page-table row
        dl = torch.randint(0, MAXP * 16 + 1, (B,), generator=gen).tolist()
        npg = sum((L + 15) // 16 for L in dl)
        din = workloads.decode_inputs(dl, hq=HQ, hkv=HKV, dtype=BF16, seed=20 * bucket + draw,
                                      sink_std=1.5, max_pages=MAXP, extra_pages=NPAGES - npg)
        qd.copy_(din["q"])
        kc.copy_(din["k_cache"])
        vc.copy_(din["v_cache"])
        pt.copy_(din["page_table"])
        kv_lens.copy_(din["kv_lens"])
        dsinks.copy_(din["sinks"])
        out_p.fill_(NAN)
        out_d.fill_(NAN)
        pm.fill_(NAN)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_p = oracle.prefill(pin["q"], pin["k"], pin["v"], pin["sinks"], pin["cu_seqlens_q"],
                               pin["cu_seqlens_kv"], HKV, HQ // HKV, 0.125, True)
        assert_close(out_p[:total].cpu(), ref_p, BF16,
                     "bucket %d draw %d prefill lens %s" % (bucket, draw, lens))
        ref_d = oracle.decode_paged(din["q"], din["k_cache"], din["v_cache"], din["page_table"],
                                    din["kv_lens"], din["sinks"], HQ // HKV, 0.125)
        assert_close(out_d.cpu(), ref_d, BF16,
                     "bucket %d draw %d decode lens %s" % (bucket, draw, dl))
        # eager work of the program's own between replays
        x = torch.randn(1 << 20, device=DEV)
        assert math.isfinite(float(x.sum()))
