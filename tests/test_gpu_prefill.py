"""GPU parity of ragged (causal) prefill with sinks (MI355X)."""
import math

import pytest
import torch

import oracle
import workloads
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_prefill(lib, d, causal=True):
    """Prefill through the C ABI into an output pre-filled with NaN, so that
    any element the grid never writes fails the comparison."""
    dd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    out = torch.full_like(dd["q"], float("nan"))
    lib.attn_sink_prefill(dd["q"], dd["k"], dd["v"], dd["sinks"], dd["cu_seqlens_q"],
                          dd["cu_seqlens_kv"], max(d["lens_q"] + [0]), d["group"],
                          d["sm_scale"], causal, out=out)
    torch.cuda.synchronize()
    return out.cpu()


def oracle_prefill(d, causal=True, rows=None):
    return oracle.prefill(d["q"].cpu(), d["k"].cpu(), d["v"].cpu(), d["sinks"].cpu(),
                          d["cu_seqlens_q"].cpu(), d["cu_seqlens_kv"].cpu(),
                          d["num_kv_heads"], d["group"], d["sm_scale"], causal, rows=rows)


def test_prefill_c1_fp32_matches_oracle(lib):
    """Tiny causal prefill workload, fp32, tolerance 1e-5."""
    d = workloads.workload(1)
    out = run_prefill(lib, d)
    assert_close(out, oracle_prefill(d), torch.float32, "C1")


CASES = [
    # lens_q, lens_kv (None = same), hq, hkv, causal
    ([1], None, 8, 2, True),
    ([63, 64, 65], None, 8, 1, True),
    ([130, 7, 257], None, 16, 2, True),
    ([100, 33], [140, 33], 8, 2, True),          # Lq < Lkv: bottom-right causal
    ([50, 1], [20, 80], 4, 2, True),              # Lkv < Lq: leading rows see no key
    ([70, 129], [150, 3], 8, 4, False),           # non-causal, ragged
    ([0, 40, 0, 9], [0, 40, 5, 9], 4, 1, True),   # empty sequences
    ([300], None, 64, 1, True),                   # group 64: one token per wave
    ([97], None, 6, 2, True),                     # group 3 (does not divide 64)
    ([200], None, 24, 2, False),                  # group 12
    ([129], None, 2, 2, True),                    # group 1 (plain multi-head)
    # kv heads a multiple of 8 with unequal lengths: the sequence-major order
    ([130, 7, 0, 257, 64], [200, 7, 5, 257, 64], 16, 8, True),
    ([100, 33, 300], None, 32, 16, True),         # two kv heads per XCD
    ([70, 129, 1], [150, 3, 40], 16, 8, False),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_sweep_matches_oracle(lib, dtype, case):
    lens_q, lens_kv, hq, hkv, causal = CASES[case]
    d = workloads.prefill_inputs(lens_q, lens_kv, hq=hq, hkv=hkv, dtype=dtype, seed=case,
                                 sink_std=1.5)
    out = run_prefill(lib, d, causal)
    assert_close(out, oracle_prefill(d, causal), dtype, "case %d" % case)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_more_than_64_sequences(lib, dtype):
    """Past 64 sequences the pair index is used as is (no ranking by length)."""
    g = torch.Generator().manual_seed(65)
    lens = torch.randint(0, 40, (70,), generator=g).tolist()
    d = workloads.prefill_inputs(lens, hq=16, hkv=8, dtype=dtype, seed=66, sink_std=1.5)
    assert_close(run_prefill(lib, d), oracle_prefill(d), dtype, "prefill B=70")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_sink_extremes(lib, dtype):
    """Sinks -inf, 0, moderate and +20 with logits up to about +-30."""
    sinks = torch.tensor([-math.inf, 0.0, 1.3, 20.0, -math.inf, -2.0, 20.0, 0.5])
    mults = [1.0, 2.0, 4.0, 7.5, 7.5, 4.0, 2.0, 1.0]
    d = workloads.prefill_inputs([77, 300], hq=8, hkv=2, dtype=dtype, seed=4, sinks=sinks,
                                 q_head_mult=mults)
    out = run_prefill(lib, d)
    ref = oracle_prefill(d)
    assert_close(out, ref, dtype, "sink extremes")


def test_prefill_empty_key_rows_are_zero(lib):
    """Non-causal with no keys: every output row is 0, finite sink or not."""
    d = workloads.prefill_inputs([5, 3], [0, 0], hq=4, hkv=2, dtype=torch.bfloat16, seed=1,
                                 sinks=[-math.inf, 0.0, 3.0, 20.0])
    out = run_prefill(lib, d, causal=False)
    assert torch.all(out == 0)


def test_causal_future_junk_invariance(lib):
    """Overwriting keys/values after position i leaves rows <= i bitwise
    unchanged (masked keys contribute exactly nothing)."""
    L, i = 300, 150
    d = workloads.prefill_inputs([L], hq=16, hkv=2, dtype=torch.bfloat16, seed=9)
    a = run_prefill(lib, d)
    g = torch.Generator().manual_seed(99)
    d2 = dict(d)
    d2["k"] = d["k"].clone()
    d2["v"] = d["v"].clone()
    d2["k"][i + 1:] = (torch.randn(L - i - 1, 2, 64, generator=g) * 50).to(torch.bfloat16)
    d2["v"][i + 1:] = (torch.randn(L - i - 1, 2, 64, generator=g) * 50).to(torch.bfloat16)
    b = run_prefill(lib, d2)
    assert torch.equal(a[:i + 1], b[:i + 1])
    assert not torch.equal(a[i + 1:], b[i + 1:])


def test_prefill_deterministic(lib):
    d = workloads.prefill_inputs([500, 77], hq=16, hkv=2, dtype=torch.bfloat16, seed=2)
    assert torch.equal(run_prefill(lib, d), run_prefill(lib, d))


def test_prefill_c2_full_matches_oracle(lib):
    """Causal prefill workload B=4 x 2048, 64/8 heads, bf16: every element of
    the output against the fp64 oracle (about 5 s of oracle time on 16 host
    cores)."""
    d = workloads.workload(2)
    out = run_prefill(lib, d)
    assert_close(out, oracle_prefill(d), torch.bfloat16, "C2 full")


def test_prefill_c5_full_matches_oracle(lib):
    """Ragged edge-case workload (16 sequences, len U[128,4096], sinks
    {-inf, 0, N(0,1), +20}, logits up to about +-30), the launch the benchmark
    times (sequence-major order per XCD): every element against the fp64
    oracle (about 26 s of oracle time on 16 host cores)."""
    d = workloads.workload(5)
    out = run_prefill(lib, d)
    assert_close(out, oracle_prefill(d), torch.bfloat16, "C5 full")
