"""Host-side planning logic of the binding (CPU only, no GPU call)."""
import gqa_attention_sinks_initialised_amd as m


def test_decode_splits_fill_the_gpu():
    # 64 sequences x 8 kv heads = 512 items: 4 splits give 2048 = 8 per CU
    assert m.default_num_splits([4096] * 64, 8) == 3
    # few long sequences split into many chunks (up to the 256 cap)
    assert m.default_num_splits([131072] * 4, 8) == 48
    assert m.default_num_splits([131072], 1) == 256
    # never more splits than pages
    assert m.default_num_splits([20], 1) == 2
    assert m.default_num_splits([], 8) == 1


def test_prefill_splits():
    # chunked prefill: 512 tokens of one sequence, G = 8 -> 32 tokens per
    # workgroup, 16 tiles x 8 kv heads = 128 workgroups -> 4 splits
    assert m.default_prefill_splits(1, 8, 8, 512, 32768) == 4
    # a full prefill batch already fills the GPU
    assert m.default_prefill_splits(4, 8, 8, 2048, 2048) == 1
    # short key ranges are not cut below 256 keys per chunk
    assert m.default_prefill_splits(1, 1, 8, 16, 600) == 2
    assert m.default_prefill_splits(1, 1, 8, 16, 100) == 1
    assert m.default_prefill_splits(0, 8, 8, 0, 0) == 1


def test_bench_flop_count_matches_enumeration():
    """The benchmark's algorithmic flops (4 * D per visible (query, key) pair
    per head) against an explicit enumeration of the visible pairs, causal
    rows aligned bottom-right."""
    import itertools
    import random

    import bench

    rng = random.Random(7)
    for _ in range(20):
        b = rng.randint(1, 4)
        lq = [rng.randint(0, 40) for _ in range(b)]
        lkv = [rng.randint(0, 60) for _ in range(b)]
        for causal in (True, False):
            pairs = 0
            for q_len, k_len in zip(lq, lkv):
                for i, j in itertools.product(range(q_len), range(k_len)):
                    pairs += (not causal) or j <= i + (k_len - q_len)
            assert bench.prefill_flops(lq, lkv, 3, 64, causal) == 4 * 64 * 3 * pairs
