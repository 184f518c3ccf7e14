"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/oracle.c -- a dropped or
mis-scaled sink, a wrong GQA head map, top-left causal alignment, the sink
in every split, a wrong chunk rule, a wrong page slot, a dropped merge
weight, a wrong bf16 widening, a missing causal clip -- builds it, and runs
the pin suite (tests/test_oracle_pins.py) against that build in a fresh
process.  The suite must fail for every mutant, and pass for an unmodified
copy built the same way.  The planted copies live in a temporary directory;
oracle/oracle.c itself is never changed.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(HERE, "test_oracle_pins.py")

# (name, original text, planted text, number of occurrences replaced)
MUTANTS = [
    ("sink dropped from the denominator",
     "double den = exp(sink - mx);", "double den = 0.0;", 1),
    ("sink multiplied by sm_scale in prefill",
     "sink_softmax_row((int)n, x, sinks[h], dim, ragged_v_at, &ctx, out);",
     "sink_softmax_row((int)n, x, sinks[h] * scale, dim, ragged_v_at, &ctx, out);", 1),
    ("sink multiplied by sm_scale in decode",
     "sink_softmax_row((int)L, x, sinks[h], dim, paged_v_at, &ctx,",
     "sink_softmax_row((int)L, x, sinks[h] * scale, dim, paged_v_at, &ctx,", 1),
    ("GQA map h % Hkv in prefill",
     "const int g = h / group;                 /* GQA: query head -> kv head */",
     "const int g = h % hkv;", 1),
    ("GQA map h % Hkv in decode",
     "const int g = h / group;            /* GQA: query head -> kv head */",
     "const int g = h % hkv;", 1),
    ("top-left causal alignment",
     "int64_t n = i + (lkv - lq) + 1;", "int64_t n = i + 1;", 1),
    ("sink in every chunk of paged splits",
     "block_state(x, t0, t1, c == 0, sinks[h], dim, paged_v_at, &ctx,",
     "block_state(x, t0, t1, 1, sinks[h], dim, paged_v_at, &ctx,", 2),
    ("sink in every chunk of ragged splits",
     "block_state(x, t0, t1, c == 0, sinks[h], dim, ragged_v_at, &ctx,",
     "block_state(x, t0, t1, 1, sinks[h], dim, ragged_v_at, &ctx,", 1),
    ("sink weight fixed to 1 in chunk 0",
     "den = exp(sink - m);", "den = 1.0;", 1),
    ("wrong chunk size",
     "const int64_t ppc = (nu + splits - 1) / splits;",
     "const int64_t ppc = nu / splits + 1;", 1),
    ("chunk end off by one",
     "e = a + ppc * unit;", "e = a + ppc * unit - 1;", 1),
    ("wrong V slot in a page",
     "t % c->psz);", "(t + 1) % c->psz);", 1),
    ("wrong K slot in a page",
     "* psz + t % psz) * (int64_t)dim;", "* psz + (t + 1) % psz) * (int64_t)dim;", 1),
    ("merge weight dropped from the denominator",
     "D += d[r * splits + c] * w;", "D += d[r * splits + c];", 1),
    ("bf16 widened with the wrong shift",
     "((const uint16_t *)p)[i] << 16;", "((const uint16_t *)p)[i] << 15;", 1),
    ("split prefill not clipped at the causal limit",
     "t1 = n;             /* keys past the row's causal limit */", "(void)n;", 1),
    ("paged prefill queries not taken as the last Lq positions",
     "const int64_t lkv = kv_lens[b];\n        const int64_t n = visible_keys(tok - cu_q[b], "
     "cu_q[b + 1] - cu_q[b], lkv,",
     "const int64_t lkv = kv_lens[b];\n        const int64_t n = visible_keys(tok - cu_q[b], "
     "lkv, lkv,", 1),
    ("merge without the max shift of each chunk",
     "double w = exp(mc - M);", "double w = 1.0;", 1),
]


def _build(src_text, tmp_path, name):
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-shared", "-fPIC", str(c),
                           "-o", str(so), "-lm"])
    return str(so)


def _pins_pass(lib):
    env = dict(os.environ, ORACLE_LIBRARY=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    assert res.returncode in (0, 1), res.stdout[-2000:] + res.stderr[-2000:]
    return res.returncode == 0


def test_unmodified_copy_passes_the_pins(tmp_path):
    assert _pins_pass(_build(open(SRC).read(), tmp_path, "control"))


@pytest.mark.parametrize("case", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, case):
    name, old, new, count = MUTANTS[case]
    text = open(SRC).read()
    assert text.count(old) == count, "anchor for %r not found as expected" % name
    lib = _build(text.replace(old, new), tmp_path, "mutant%d" % case)
    assert not _pins_pass(lib), "the pins did not catch: %s" % name
