"""The whole path can be captured into a HIP graph and replayed.

The library only enqueues kernels on the caller's stream: no host
synchronisation, no device-to-host copy, no memset and no allocation.  A
captured prefill + split decode + merge + split chunked (paged) prefill +
merge sequence must therefore replay to
the same bits as the eager calls, replay after replay, with other eager work
and synchronisations between the replays (page "Fast embeddings on GPUs",
section "CUDA graph management": the serving engine captures whole forward
passes once per shape and replays them, so the kernels must not depend on
host-side dynamic state).
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def test_capture_and_replay_matches_eager(lib):
    p = _dev(workloads.prefill_inputs([300, 77], hq=16, hkv=2, dtype=torch.bfloat16, seed=3,
                                      sink_std=1.5))
    d = _dev(workloads.decode_inputs([900, 33, 4000], hq=16, hkv=2, dtype=torch.bfloat16,
                                     seed=4, sink_std=1.5))
    S = 7
    out_p = torch.empty_like(p["q"])
    out_d = torch.empty_like(d["q"])
    f32 = dict(device=DEV, dtype=torch.float32)
    pm = torch.empty((3, 16, S), **f32)
    pd = torch.empty((3, 16, S), **f32)
    po = torch.empty((3, 16, S, 64), **f32)

    # chunked prefill against a paged cache, split 3 ways, then merged
    c = workloads.prefill_inputs([40, 9], [700, 130], hq=16, hkv=2, dtype=torch.bfloat16,
                                 seed=5, sink_std=1.5)
    c.update(workloads.pack_paged(c["k"], c["v"], c["lens_kv"], seed=6))
    c = _dev(c)
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

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    for i in range(4):
        out_p.zero_()
        out_d.zero_()
        out_c.zero_()
        pm.fill_(float("nan"))
        cm.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_p, ref_p), "prefill replay %d" % i
        assert torch.equal(out_d, ref_d), "decode+merge replay %d" % i
        assert torch.equal(out_c, ref_c), "chunked prefill+merge replay %d" % i
        path()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out_p, ref_p) and torch.equal(out_d, ref_d)
        assert torch.equal(out_c, ref_c)
