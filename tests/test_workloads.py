"""The seeded workload generators: shapes, length statistics, block
allocation and prefix sharing as the five workloads describe them."""

import math

import numpy as np
import pytest
import torch

from paged_kv_cache_32_amd import workloads as W


def _check_tables(w):
    BS = w.block_size
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        n = -(-L // BS)
        row = w.block_tables[s]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < w.num_blocks)
        assert np.all(row[n:] == -1)
        slot = int(w.slot_mapping[s])
        assert slot == int(row[(L - 1) // BS]) * BS + (L - 1) % BS


def test_tiny():
    w = W.config(1)
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks) == (4, 1, 64, 16, 16)
    assert w.seq_lens.tolist() == [17, 40, 5]
    assert [int((r >= 0).sum()) for r in w.block_tables] == [2, 3, 1]
    assert len(set(w.block_tables[w.block_tables >= 0].tolist())) == 6
    assert w.scale == 1 / 8
    _check_tables(w)
    # New tokens land at positions 16 (first slot of a fresh block), 39 and 4.
    assert [int(s) % 16 for s in w.slot_mapping] == [0, 7, 4]
    w2 = W.tiny(new_token_at_end=False)
    assert w2.seq_lens.tolist() == [18, 41, 6]
    assert [int(s) % 16 for s in w2.slot_mapping] == [1, 8, 5]


def test_llama70b_lengths_and_pool():
    w = W.config(2)
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.num_seqs) == (64, 8, 128, 16, 64)
    assert w.seq_lens.min() >= 16 and w.seq_lens.max() <= 32768
    need = sum(-(-int(L) // 16) for L in w.seq_lens)
    assert w.num_blocks == math.ceil(1.25 * need)
    assert len(w.used_blocks()) == need
    _check_tables(w)
    # The lognormal: median 2,400 and p95 18,000 before clipping.
    rng = np.random.default_rng(0)
    x = W.lognormal_lengths(rng, 200_000, lo=0, hi=10 ** 9)
    assert abs(np.median(x) / 2400 - 1) < 0.02
    assert abs(np.quantile(x, 0.95) / 18000 - 1) < 0.03


def test_prefix_shared_rules():
    w = W.config(3)
    assert w.num_seqs == 256 and w.block_size == 32
    _check_tables(w)
    bt = w.block_tables
    # 900 system tokens -> 28 full blocks shared by every sequence.
    assert np.all(bt[:, :28] == bt[0, :28])
    assert len(set(bt[:, 28].tolist())) <= 12
    assert abs(w.notes["pool_share"] - 0.62) < 0.005
    # Blocks holding the last token are private.
    last = [int(bt[s, (int(w.seq_lens[s]) - 1) // 32]) for s in range(256)]
    assert len(set(last)) == 256
    s = w.summary()
    assert 2.0 < s["sharing_factor"] < 4.0
    assert w.physical_kv_bytes() < w.logical_kv_bytes()
    assert w.num_blocks == math.ceil(1.25 * len(w.used_blocks()))


def test_long_context_and_fp8_shapes():
    w = W.config(4)
    assert w.seq_lens.tolist() == [131072] * 4 and w.num_blocks == 40960
    _check_tables(w)
    w5 = W.config(5)
    assert w5.kv_dtype == "fp8" and w5.num_layers == 80 and w5.num_seqs == 128
    _check_tables(w5)


def test_deterministic():
    a, b = W.config(2), W.config(2)
    assert np.array_equal(a.block_tables, b.block_tables) and np.array_equal(a.seq_lens, b.seq_lens)
    ta = W.config(1).make_tensors("cpu")
    tb = W.config(1).make_tensors("cpu")
    for k in ta:
        x, y = ta[k], tb[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_poison_covers_exactly_the_unreadable_slots(kv_dtype):
    w = W.random_workload(3, 5, 8, 2, 32, 32, 70, kv_dtype=kv_dtype, min_len=1)
    t = w.make_tensors("cpu")
    kc = t["k_cache"][0]
    kc = (kc.view(torch.int16).numpy().view(np.uint16) if kv_dtype == "bf16" else kc.numpy())
    nan = W.BF16_NAN if kv_dtype == "bf16" else W.FP8_NAN
    from oracle import paged
    g = paged.Geom(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, kv_dtype)
    readable = np.zeros(g.cache_elems, dtype=bool)
    for s in range(w.num_seqs):
        for tok in range(int(w.seq_lens[s]) - 1):          # the new token's slot is poisoned
            blk = int(w.block_tables[s, tok // w.block_size])
            for h in range(2):
                readable[[paged.k_offset(g, blk, h, tok % w.block_size, d) for d in range(32)]] = True
    assert not np.any(kc[readable] == nan)
    assert np.all(kc[~readable] == nan)
    if kv_dtype == "fp8":
        assert t["k_scale"].shape == (1,) and float(t["k_scale"][0]) > 0
