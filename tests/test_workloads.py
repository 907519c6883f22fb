"""The seeded input generator: shapes, determinism and poisoning (CPU)."""
import math

import numpy as np

from paged_kv_attention_24_amd import workloads as W


def test_tiny_config_layout():
    wl = W.make_config(1)
    assert wl.dtype == "f32" and wl.num_blocks == 8
    assert list(wl.context_lens) == [5, 37]
    assert wl.block_tables.shape == (2, 3)
    assert wl.block_tables[0, 1] == -1 and wl.block_tables[0, 2] == -1
    used = wl.block_tables[wl.block_tables >= 0]
    assert len(set(used.tolist())) == 4 and used.max() < 8
    assert wl.k_cache.shape == (8, 2, 16, 64) and wl.q.shape == (2, 4, 64)
    assert wl.scale == np.float32(0.125)
    # the new token of each sequence goes to the slot of position L-1
    for b, L in enumerate(wl.context_lens):
        pos = int(L) - 1
        assert wl.slot_mapping[b] == wl.block_tables[b, pos // 16] * 16 + pos % 16


def test_deterministic_per_seed():
    a, b = W.make_config(2), W.make_config(2)
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.q, b.q)
    c = W.make_config(2, seed=99)
    assert not np.array_equal(a.context_lens, c.context_lens)


def test_poisoning():
    wl = W.make_config(3)
    nan_bits = W.NAN_BITS["bf16"]
    bs = wl.block_size
    used = set(wl.block_tables[wl.block_tables >= 0].tolist())
    unused = [i for i in range(wl.num_blocks) if i not in used]
    assert len(unused) > 0
    assert np.all(wl.k_cache[unused] == nan_bits)
    for b in range(wl.num_seqs):
        L = int(wl.context_lens[b])
        last = wl.block_tables[b, (L - 1) // bs]
        tail = L - ((L - 1) // bs) * bs
        assert np.all(wl.v_cache[last, :, tail:, :] == nan_bits)
        assert np.all(wl.k_cache[last, :, tail - 1, :] == nan_bits)  # slot awaiting the write
        if tail >= 2:
            assert not np.any(wl.k_cache[last, :, tail - 2, :] == nan_bits)


def test_length_distributions():
    rng = np.random.default_rng(2)
    l2 = W.config_lens(2, rng)
    assert l2.shape == (16,) and l2.min() >= 100 and l2.max() <= 1024
    l3 = W.config_lens(3, np.random.default_rng(3))
    assert l3.shape == (64,) and l3.min() >= 16 and l3.max() <= 4096
    l4 = W.config_lens(4, np.random.default_rng(4))
    assert l4.shape == (128,) and l4.min() >= 2048 and l4.max() <= 8192
    l5 = W.config_lens(5, np.random.default_rng(5))
    assert l5.shape == (256,) and l5[0] == 32768 and l5[1:].max() <= 2048 and l5[1:].min() >= 128


def test_pool_sizing_and_bytes():
    wl = W.make_config(2, poison=False)
    used = int(np.sum((wl.context_lens + 15) // 16))
    assert wl.num_blocks == math.ceil(1.25 * used)
    assert wl.kv_bytes() == int(wl.context_lens.sum()) * 2 * 8 * 64 * 2


def test_half_rounding_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -8], dtype=np.float32)
    f16 = W._round_to_dtype(x, "f16")
    assert list(f16) == [0x3C00, 0x3C02, 0x3C04]
    bf = W._round_to_dtype(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32), "bf16")
    assert list(bf) == [0x3F80, 0x3F82]


def test_prefill_workloads_shapes_and_determinism():
    a, b = W.make_prefill_config(1), W.make_prefill_config(1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_cache, b.k_cache)
    assert a.query_start.tolist() == [0, 7, 8, 28]
    assert a.context_lens.tolist() == [7, 6, 60]
    assert a.q.shape == (28, 8, 64) and a.max_query_len == 20
    w2 = W.make_prefill_config(2, poison=False)
    assert w2.num_query_tokens == 2048 and (np.diff(w2.query_start) == 256).all()
    assert (w2.context_lens >= 256).all() and (w2.context_lens <= 3072 + 256).all()
    # every position of every sequence is backed by a block of the pool
    for s in range(w2.num_seqs):
        nblk = -(-int(w2.context_lens[s]) // w2.block_size)
        assert (w2.block_tables[s, :nblk] >= 0).all()
