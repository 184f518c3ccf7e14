"""Benchmark of the sink-attention hot path on one MI355X.

One step = one pass over every stage of the path on its synthetic workload:
  prefill  causal prefill, bf16, B=4 x 2048, Hq=64, Hkv=8, D=64      (MFMA-bound)
  decode   paged decode, bf16, B=64, kv_len U[512,8192], + merge     (HBM-bound)
  single   the same decode in one launch: unsplit, 16 waves per workgroup split
           each sequence's pages and merge in LDS (no partial states, no merge)
  split    split-KV decode, bf16, B=4, kv_len 131072, 64 splits, + merge (HBM-bound)
  paged    the prefill workload with keys and values in a paged cache
  chunked  chunked prefill: B=1, 512 new tokens on a 32768-key paged cache,
           unsplit, then split (default_prefill_splits: 4) + merge
  ragged   ragged causal prefill, 16 sequences U[128,4096], sinks -inf / 0 /
           N(0,1) / +20, logits up to about +-30 (reported, not in value)
`value` is the prefill throughput in TFLOP/s (algorithmic flops: 4*D per
causal-visible (query, key) pair) from HIP events around the prefill launch
on the stream it runs on; the decode stages report achieved HBM GB/s.  The
256 MB memory-side cache is flushed (a 1 GiB read) before each decode stage,
outside the kernel events.  The fp64 CPU oracle is timed on a bounded sample
of the prefill workload as a reported baseline (rank 0, N=1 only).

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def prefill_flops(lens_q, lens_kv, hq, dim, causal=True):
    pairs = 0
    for lq, lkv in zip(lens_q, lens_kv):
        if causal:
            shift = lkv - lq
            # row i sees min(lkv, max(0, i + shift + 1)) keys
            for i in range(lq):
                pairs += min(lkv, max(0, i + shift + 1))
        else:
            pairs += lq * lkv
    return 4.0 * dim * pairs * hq


def decode_bytes(kv_lens, hq, hkv, dim, splits, es=2):
    """Algorithmic HBM bytes of paged decode (+ merge when splits > 1)."""
    tokens = sum(int(L) for L in kv_lens)
    kv = tokens * hkv * dim * 2 * es                      # K and V of valid tokens
    b = len(kv_lens)
    q_o = 2 * b * hq * dim * es                           # q read, output written
    pages = sum((int(L) + 15) // 16 for L in kv_lens) * 4  # page-table entries
    partials = b * hq * splits * (dim + 2) * 4 if splits > 1 else 0
    decode = kv + b * hq * dim * es + pages + partials    # decode kernel
    merge = partials + b * hq * dim * es if splits > 1 else 0
    return dict(total=kv + q_o + pages + 2 * partials, decode=decode, merge=merge, kv=kv)


def counted_traffic():
    """Per-launch HBM bytes measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (scaled
    by a plain copy of known size), kept in profiles/hbm_traffic.json together
    with the hash of the kernel source they were taken on.  Returns None when
    the kernels have changed since (the figures no longer describe them)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    src = os.path.join(ROOT, "gqa_attention_sinks_initialised_amd", "csrc", "attn_sink.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return {k: v.get("fetch_bytes", 0.0) + v.get("write_bytes", 0.0)
            for k, v in rec.get("per_launch_bytes", {}).items()}


def profiled_clock():
    """Average shader clock (GHz) per kernel under its own load, from a
    rocprofv3 counter pass: GRBM_GUI_ACTIVE summed over the 8 XCDs, divided
    by 8 and by the dispatch's traced duration.  Kept in profiles/clock.json
    with the hash of the kernel source it was taken on; None once the kernels
    have changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "clock.json")
    src = os.path.join(ROOT, "gqa_attention_sinks_initialised_amd", "csrc", "attn_sink.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("clock_ghz")


def profiled_power():
    """Socket power per kernel and the vendor bf16 GEMM reference under the same power cap,
    from `bench.py --power` (profiles/power.json), while the kernel source hash matches."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "power.json")
    src = os.path.join(ROOT, "gqa_attention_sinks_initialised_amd", "csrc", "attn_sink.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for the "
                         "HBM byte counters)")
    ap.add_argument("--power", action="store_true",
                    help="only measure socket power and shader clocks (amd-smi) while each "
                         "main kernel runs back to back for a few seconds")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only; run with --gpus 1 "
              "(the multi-GPU split of this path is described, not built)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 28, device="cuda:0", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 1 << 30, "bytes_written": 1 << 30}))
        return

    import torch
    import gqa_attention_sinks_initialised_amd as attn
    import workloads

    attn.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.power:
        power_profile(attn, workloads, torch, dev)
        return

    # ---- inputs (seeded, synthetic), resident in HBM before timing
    c2 = workloads.workload(2, device=dev)
    c3 = workloads.workload(3, device=dev, cache_device=dev)
    c4 = workloads.workload(4, device=dev, cache_device=dev)
    s3 = attn.default_num_splits(c3["kv_lens"].tolist(), 8)
    s4 = 64
    out2 = torch.empty_like(c2["q"])
    hq = 64

    def mk_partials(b, s):
        f = dict(device=dev, dtype=torch.float32)
        return (torch.empty((b, hq, s), **f), torch.empty((b, hq, s), **f),
                torch.empty((b, hq, s, 64), **f))

    p3, p4 = mk_partials(64, s3), mk_partials(4, s4)
    o3 = torch.empty((64, hq, 64), device=dev, dtype=torch.bfloat16)
    o3s = torch.empty((64, hq, 64), device=dev, dtype=torch.bfloat16)
    o4 = torch.empty((4, hq, 64), device=dev, dtype=torch.bfloat16)
    # Reading (not writing) 1 GiB evicts the 256 MB memory-side cache without
    # leaving dirty lines whose write-back would land inside the next kernel.
    flush = torch.ones(1 << 28, device=dev, dtype=torch.float32)

    def run_prefill():
        attn.attn_sink_prefill(c2["q"], c2["k"], c2["v"], c2["sinks"], c2["cu_seqlens_q"],
                               c2["cu_seqlens_kv"], 2048, 8, c2["sm_scale"], True, out=out2)

    def run_decode(c, s, parts):
        attn.attn_sink_decode_paged(c["q"], c["k_cache"], c["v_cache"], c["page_table"],
                                    c["kv_lens"], c["sinks"], 8, c["sm_scale"], s,
                                    partial_m=parts[0], partial_d=parts[1],
                                    partial_o=parts[2])

    def run_decode_single():
        attn.attn_sink_decode_paged(c3["q"], c3["k_cache"], c3["v_cache"], c3["page_table"],
                                    c3["kv_lens"], c3["sinks"], 8, c3["sm_scale"], 1, out=o3s)

    # Further workloads: the prefill workload with its keys in a paged cache,
    # and chunked prefill (few query tiles, long paged cache) unsplit and split.
    pk2 = workloads.pack_paged(c2["k"], c2["v"], c2["lens_kv"], seed=2002)
    out2p = torch.empty_like(c2["q"])
    c6 = workloads.workload(6, device=dev)
    s6 = attn.default_prefill_splits(1, 8, 8, 512, 32768)
    out6 = torch.empty_like(c6["q"])
    p6 = mk_partials(c6["q"].shape[0], s6)
    o6 = torch.empty_like(c6["q"])

    # The ragged edge-case prefill workload (16 sequences, lengths U[128,4096],
    # sinks -inf / 0 / N(0,1) / +20, logits up to about +-30): reported beside
    # the main prefill figure, not part of value.
    c5 = workloads.workload(5, device=dev)
    out5 = torch.empty_like(c5["q"])
    mq5 = max(c5["lens_q"])

    def run_ragged_prefill():
        attn.attn_sink_prefill(c5["q"], c5["k"], c5["v"], c5["sinks"], c5["cu_seqlens_q"],
                               c5["cu_seqlens_kv"], mq5, 8, c5["sm_scale"], True, out=out5)

    def run_paged_prefill():
        attn.attn_sink_prefill_paged(c2["q"], pk2["k_cache"], pk2["v_cache"], pk2["page_table"],
                                     c2["cu_seqlens_q"], pk2["kv_lens"], c2["sinks"], 2048, 8,
                                     c2["sm_scale"], True, out=out2p)

    def run_chunked(splits):
        kw = dict(out=out6) if splits == 1 else dict(partial_m=p6[0], partial_d=p6[1],
                                                     partial_o=p6[2])
        attn.attn_sink_prefill_paged(c6["q"], c6["k_cache"], c6["v_cache"], c6["page_table"],
                                     c6["cu_seqlens_q"], c6["kv_lens"], c6["sinks"], 512, 8,
                                     c6["sm_scale"], True, num_splits=splits, **kw)

    # One step, in launch order.  The kernel sequence of a step (ours only) is
    # fixed, which is how profile summaries attribute dispatches to workloads.
    # A merge is timed in one bracket with the decode it finishes (third field
    # True): an event recorded between two launches on a stream leaves a gap
    # of a few microseconds that is not part of the work.
    ops = [
        ("prefill", run_prefill, False),
        ("_flush", flush.sum, False),
        ("decode", lambda: run_decode(c3, s3, p3), False),
        ("decode_merge", lambda: attn.attn_sink_merge(*p3, out=o3), True),
        ("_flush", flush.sum, False),
        ("decode_single", run_decode_single, False),
        ("_flush", flush.sum, False),
        ("split", lambda: run_decode(c4, s4, p4), False),
        ("split_merge", lambda: attn.attn_sink_merge(*p4, out=o4), True),
        ("paged_prefill", run_paged_prefill, False),
        ("chunked", lambda: run_chunked(1), False),
        ("chunked_split", lambda: run_chunked(s6), False),
        ("chunked_merge", lambda: attn.attn_sink_merge(*p6, out=o6), True),
        ("ragged_prefill", run_ragged_prefill, False),
    ]

    def step(evs=None, split_pairs=False):
        """One step; with events, evs[i] is recorded before op i unless that op
        continues the previous bracket (and split_pairs is off)."""
        for i, (_, fn, joined) in enumerate(ops):
            if evs and (split_pairs or not joined):
                evs[i].record()
            fn()
        if evs:
            evs[len(ops)].record()

    def timed(n, split_pairs):
        """Mean bracket time (ms) of every op that opens a bracket, the
        per-step samples of each, and the wall time of the n steps."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
               for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            step(evs[i], split_pairs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        marks = [i for i, op in enumerate(ops) if split_pairs or not op[2]] + [len(ops)]
        t, samples = {}, {}
        for a, b in zip(marks, marks[1:]):
            if not ops[a][0].startswith("_"):
                samples[ops[a][0]] = [e[a].elapsed_time(e[b]) for e in evs]
                t[ops[a][0]] = sum(samples[ops[a][0]]) / n
        return t, samples, wall

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The K timed steps; then a few more with an event between every launch,
    # for the per-kernel split of each decode + merge bracket.
    tb, sb, wall = timed(args.steps, False)
    t, _, _ = timed(min(args.steps, 10), True)
    for name in ("prefill", "paged_prefill", "chunked", "ragged_prefill", "decode_single"):
        t[name] = tb[name]

    def spread(name):
        """Mean, median and min of one bracket over the K timed steps (us)."""
        x = sorted(sb[name])
        return {"us_mean": round(tb[name] * 1e3, 2),
                "us_median": round(statistics.median(x) * 1e3, 2),
                "us_min": round(x[0] * 1e3, 2)}

    fl2 = prefill_flops(c2["lens_q"], c2["lens_kv"], hq, 64)
    tflops = fl2 / (t["prefill"] * 1e-3) / 1e12
    b3 = decode_bytes(c3["kv_lens"].tolist(), hq, 8, 64, s3)
    b4 = decode_bytes(c4["kv_lens"].tolist(), hq, 8, 64, s4)
    gbs3 = b3["total"] / (tb["decode"] * 1e-3) / 1e9
    gbs4 = b4["total"] / (tb["split"] * 1e-3) / 1e9
    gbs3_k = b3["decode"] / (t["decode"] * 1e-3) / 1e9
    gbs4_k = b4["decode"] / (t["split"] * 1e-3) / 1e9
    b3s = decode_bytes(c3["kv_lens"].tolist(), hq, 8, 64, 1)
    gbs3s = b3s["total"] / (t["decode_single"] * 1e-3) / 1e9

    fl2p = fl2
    fl6 = prefill_flops(c6["lens_q"], c6["lens_kv"], hq, 64)
    tf2p = fl2p / (t["paged_prefill"] * 1e-3) / 1e12
    tf6 = fl6 / (t["chunked"] * 1e-3) / 1e12
    tf6s = fl6 / (tb["chunked_split"] * 1e-3) / 1e12

    fl5 = prefill_flops(c5["lens_q"], c5["lens_kv"], hq, 64)
    tf5 = fl5 / (t["ragged_prefill"] * 1e-3) / 1e12

    traffic = counted_traffic() or {}
    clock = profiled_clock() or {}
    clk2 = clock.get("prefill")
    power = profiled_power() or {}
    pk = power.get("kernels", {})
    gemm_ref = pk.get("library_gemm_bf16_8192", {}).get("rate")
    result = {
        "metric": "prefill attention TFLOP/s (bf16) + decode KV-read HBM GB/s, % of roofline",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, N(0,2) sinks; random page placement)",
        "config": {"workload": "causal prefill bf16 B=4 x 2048, Hq=64 Hkv=8 D=64 "
                               "(+ per step: paged decode B=64 len U[512,8192]; split-KV "
                               "decode B=4 len 131072 x 64 splits)",
                   "prefill_tokens": 8192, "decode_splits": s3, "split_splits": s4},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic.get("prefill"),
                     "kernel": "prefill_kernel<bf16>", "flops_per_launch": fl2,
                     "us_per_launch": round(t["prefill"] * 1e3, 2),
                     **spread("prefill"),
                     "clock_ghz": clk2,
                     "frac_at_clock": (round(tflops / (PEAK_BF16_TFLOPS * clk2 / 2.4), 4)
                                       if clk2 else None),
                     "power_w": pk.get("prefill", {}).get("power_w"),
                     "power_cap_w": power.get("power_cap_w"),
                     "gemm_reference_tflops": gemm_ref,
                     "frac_of_gemm_reference": (round(tflops / gemm_ref, 4)
                                                if gemm_ref else None)},
        "decode": {"workload": c3["name"], "splits": s3,
                   "us_decode": round(t["decode"] * 1e3, 2),
                   "us_merge": round(t["decode_merge"] * 1e3, 2),
                   "us_decode_merge": round(tb["decode"] * 1e3, 2),
                   "decode_merge": spread("decode"),
                   "clock_ghz": clock.get("decode_paged"),
                   "bytes": b3["total"], "GB/s": round(gbs3, 1),
                   "frac": round(gbs3 / PEAK_HBM_GBS, 4),
                   "decode_kernel_GB/s": round(gbs3_k, 1),
                   "decode_kernel_frac": round(gbs3_k / PEAK_HBM_GBS, 4),
                   "traffic": traffic.get("decode_paged")},
        "decode_single_launch": {"workload": c3["name"] + ", one launch: unsplit, 16 waves "
                                                 "per workgroup merged in LDS",
                                 "splits": 1, "us": round(t["decode_single"] * 1e3, 2),
                                 **spread("decode_single"),
                                 "clock_ghz": clock.get("decode_single"),
                                 "bytes": b3s["total"], "GB/s": round(gbs3s, 1),
                                 "frac": round(gbs3s / PEAK_HBM_GBS, 4),
                                 "traffic": traffic.get("decode_single")},
        "split_decode": {"workload": c4["name"], "splits": s4,
                         "us_decode": round(t["split"] * 1e3, 2),
                         "us_merge": round(t["split_merge"] * 1e3, 2),
                         "us_decode_merge": round(tb["split"] * 1e3, 2),
                         "decode_merge": spread("split"),
                         "clock_ghz": clock.get("decode_split"),
                         "bytes": b4["total"], "GB/s": round(gbs4, 1),
                         "frac": round(gbs4 / PEAK_HBM_GBS, 4),
                         "decode_kernel_GB/s": round(gbs4_k, 1),
                         "decode_kernel_frac": round(gbs4_k / PEAK_HBM_GBS, 4),
                         "traffic": traffic.get("decode_split")},
        "paged_prefill": {"workload": "causal prefill bf16 B=4 x 2048, Hq=64 Hkv=8 D=64, keys "
                                      "and values from a paged cache (16-token pages, random "
                                      "placement)",
                          "us": round(t["paged_prefill"] * 1e3, 2),
                          **spread("paged_prefill"),
                          "TFLOP/s": round(tf2p, 2),
                          "frac": round(tf2p / PEAK_BF16_TFLOPS, 4),
                          "traffic": traffic.get("paged_prefill")},
        "chunked_prefill": {"workload": c6["name"], "flops": fl6,
                            "us_unsplit": round(t["chunked"] * 1e3, 2),
                            "TFLOP/s_unsplit": round(tf6, 2),
                            "frac_unsplit": round(tf6 / PEAK_BF16_TFLOPS, 4),
                            "splits": s6,
                            "us_split": round(t["chunked_split"] * 1e3, 2),
                            "us_merge": round(t["chunked_merge"] * 1e3, 2),
                            "us_split_merge": round(tb["chunked_split"] * 1e3, 2),
                            "TFLOP/s_split": round(tf6s, 2),
                            "frac_split": round(tf6s / PEAK_BF16_TFLOPS, 4)},
        "ragged_prefill": {"workload": c5["name"], "flops": fl5,
                           "us": round(t["ragged_prefill"] * 1e3, 2),
                           **spread("ragged_prefill"),
                           "clock_ghz": clock.get("ragged_prefill"),
                           "TFLOP/s": round(tf5, 2),
                           "frac": round(tf5 / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic.get("ragged_prefill")},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c2, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _smi_sample():
    """Socket power (W) and the mean shader clock over the XCDs (MHz) from amd-smi,
    or None when the tool gives nothing usable."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=15)
        d = json.loads(r.stdout)
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    gpu = (d.get("gpu_data") or [d])[0] if isinstance(d, dict) else d[0]
    try:
        watts = float(gpu["power"]["socket_power"]["value"])
        clocks = [float(v["clk"]["value"]) for k, v in gpu["clock"].items()
                  if k.startswith("gfx_") and isinstance(v, dict) and "clk" in v]
    except (KeyError, TypeError, ValueError):
        return None
    return watts, (sum(clocks) / len(clocks) if clocks else None)


def power_profile(attn, workloads, torch, dev, seconds=4.0):
    """Each main kernel back to back for `seconds`; amd-smi is sampled from a thread
    after the first second.  Prints one JSON line: per kernel the mean socket power,
    shader clock, achieved rate and the dynamic energy per unit of work, beside the
    idle power."""
    import threading
    c2 = workloads.workload(2, device=dev)
    c5 = workloads.workload(5, device=dev)
    c3 = workloads.workload(3, device=dev, cache_device=dev)
    o2, o5 = torch.empty_like(c2["q"]), torch.empty_like(c5["q"])
    mq5 = max(c5["lens_q"])
    kernels = [
        ("prefill", "TFLOP/s", prefill_flops(c2["lens_q"], c2["lens_kv"], 64, 64) / 1e12,
         lambda: attn.attn_sink_prefill(c2["q"], c2["k"], c2["v"], c2["sinks"],
                                        c2["cu_seqlens_q"], c2["cu_seqlens_kv"], 2048, 8,
                                        c2["sm_scale"], True, out=o2)),
        ("ragged_prefill", "TFLOP/s", prefill_flops(c5["lens_q"], c5["lens_kv"], 64, 64) / 1e12,
         lambda: attn.attn_sink_prefill(c5["q"], c5["k"], c5["v"], c5["sinks"],
                                        c5["cu_seqlens_q"], c5["cu_seqlens_kv"], mq5, 8,
                                        c5["sm_scale"], True, out=o5)),
        ("decode_paged_unsplit", "TB/s",
         decode_bytes(c3["kv_lens"].tolist(), 64, 8, 64, 1)["decode"] / 1e12,
         lambda: attn.attn_sink_decode_paged(c3["q"], c3["k_cache"], c3["v_cache"],
                                             c3["page_table"], c3["kv_lens"], c3["sinks"], 8,
                                             c3["sm_scale"], 1)),
    ]
    # reference: a plain bf16 matrix product from the vendor library (hipBLASLt through
    # torch.mm on contiguous operands), the practical MFMA rate under the same power cap
    ga = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    gc = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)
    kernels.append(("library_gemm_bf16_8192", "TFLOP/s", 2.0 * 8192 ** 3 / 1e12,
                    lambda: torch.mm(ga, gb, out=gc)))
    torch.cuda.synchronize()
    time.sleep(2.0)
    idle = [x for x in (_smi_sample() for _ in range(3)) if x]
    res = {"metric": "socket power and shader clock per kernel (back-to-back launches)",
           "idle_w": round(sum(w for w, _ in idle) / len(idle), 1) if idle else None,
           "power_cap_w": 1400.0, "kernels": {}}
    for name, unit, work, fn in kernels:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        samples, stop = [], threading.Event()
        t_start = time.perf_counter()

        def sampler():
            while not stop.is_set():
                if time.perf_counter() - t_start > 1.0:
                    x = _smi_sample()
                    if x:
                        samples.append(x)
                time.sleep(0.2)

        th = threading.Thread(target=sampler)
        th.start()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        n = 0
        while time.perf_counter() - t_start < seconds:
            fn()
            n += 1
        e1.record()
        torch.cuda.synchronize()
        stop.set()
        th.join()
        rate = work * n / (e0.elapsed_time(e1) * 1e-3)
        rec = {"launches": n, "rate": round(rate, 2), "unit": unit, "samples": len(samples)}
        if samples:
            w = sum(x[0] for x in samples) / len(samples)
            clk = [x[1] for x in samples if x[1]]
            rec.update(power_w=round(w, 1),
                       clock_mhz=round(sum(clk) / len(clk), 0) if clk else None)
            if res["idle_w"] is not None:
                per = "pJ/flop" if unit == "TFLOP/s" else "pJ/byte"
                rec["dynamic_energy"] = round((w - res["idle_w"]) / rate, 3)
                rec["dynamic_energy_unit"] = per
        res["kernels"][name] = rec
    print(json.dumps(res), flush=True)


def cpu_baseline(c2, target_s):
    """The fp64 oracle on a bounded sample of the prefill workload: every head
    of a set of query tokens spread evenly over the four sequences."""
    import numpy as np
    import oracle

    host = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in c2.items()}
    hq, lens = 64, host["lens_q"]

    def rows_for(n_tok):
        toks = []
        off = 0
        for L in lens:
            toks += list(off + np.linspace(0, L - 1, n_tok // len(lens)).astype(np.int64))
            off += L
        toks = np.repeat(np.array(toks, dtype=np.int64), hq)
        heads = np.tile(np.arange(hq, dtype=np.int32), len(toks) // hq)
        return toks, heads

    def flops_of(toks):
        cu = np.array(host["cu_seqlens_q"].tolist())
        seq = np.searchsorted(cu, toks, side="right") - 1
        i = toks - cu[seq]
        return float(np.sum(4.0 * 64 * (i + 1)))   # Lq == Lkv: row i sees i+1 keys

    n_tok = 16
    toks, heads = rows_for(n_tok)
    t0 = time.perf_counter()
    oracle.prefill(host["q"], host["k"], host["v"], host["sinks"], host["cu_seqlens_q"],
                   host["cu_seqlens_kv"], 8, 8, host["sm_scale"], True, rows=(toks, heads))
    dt = time.perf_counter() - t0
    # Grow the sample toward target_s; once it is the whole workload (every
    # token of every sequence), repeat whole passes instead.
    total = int(sum(lens))
    scale = max(1, int(target_s / max(dt, 1e-3)))
    n_tok = min(total, n_tok * scale)
    toks, heads = rows_for(n_tok)
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.prefill(host["q"], host["k"], host["v"], host["sinks"], host["cu_seqlens_q"],
                       host["cu_seqlens_kv"], 8, 8, host["sm_scale"], True, rows=(toks, heads))
        passes += 1
        dt = time.perf_counter() - t0
        if n_tok < total or passes == 4 or dt * (passes + 1) / passes > 1.5 * target_s:
            break
    fl = flops_of(toks) * passes
    what = ("the whole prefill workload (%d query tokens x 64 heads), %d pass(es)" % (
        len(toks) // hq, passes) if n_tok == total else
        "%d query tokens x 64 heads of the prefill workload (evenly spaced over the 4 "
        "sequences)" % (len(toks) // hq))
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%s, %.3g GFLOP algorithmic, %.1f s" % (what, fl / 1e9, dt)}


if __name__ == "__main__":
    main()
