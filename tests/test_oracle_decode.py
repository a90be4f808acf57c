"""The oracle's paged decode pinned to things other than itself: a textbook
contiguous-cache attention, invariance under relabelling physical blocks,
shared versus duplicated blocks, brute force with scalar loops, closed forms,
and the split-K log-sum-exp identity.  The last tests plant mistakes in the
oracle (on the CPU) and check that these pins catch them."""

import math

import numpy as np
import pytest

from oracle import e4m3, paged

rng0 = np.random.default_rng(12345)


def bf16_bits(x):
    """float -> bf16 bit patterns (truncation; any pattern is a valid input)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def make_paged(rng, lens, Hq, Hkv, D, BS, kv_dtype="bf16", extra_blocks=2, scales=(1.0, 1.0)):
    """Contiguous per-sequence K/V, the same data scattered into a paged cache
    through shuffled block tables (using the oracle's own cache_write), and
    the query.  Returns everything both sides need."""
    g_blocks = sum(-(-L // BS) for L in lens) + extra_blocks
    g = paged.Geom(g_blocks, BS, Hkv, D, kv_dtype)
    perm = rng.permutation(g_blocks)
    maxb = max(max(-(-L // BS) for L in lens), 1)
    bt = np.full((len(lens), maxb), -1, dtype=np.int32)
    p = 0
    for s, L in enumerate(lens):
        n = -(-L // BS)
        bt[s, :n] = perm[p:p + n]
        p += n
    kc = np.full(g.cache_elems, 0x7FC0 if kv_dtype == "bf16" else 0x7F, dtype=g.np_dtype)
    vc = kc.copy()
    dense = []
    for s, L in enumerate(lens):
        kb = bf16_bits(rng.standard_normal((L, Hkv, D)))
        vb = bf16_bits(rng.standard_normal((L, Hkv, D)))
        slots = np.array([bt[s, t // BS] * BS + t % BS for t in range(L)], dtype=np.int64)
        if kv_dtype == "bf16":
            paged.cache_write_bf16(g, kb, vb, slots, kc, vc)
            K, V = paged.bf16_bits_to_f64(kb), paged.bf16_bits_to_f64(vb)
        else:
            paged.cache_write_fp8(g, kb, vb, slots, kc, vc, *scales)
            K = e4m3.dequantize(e4m3.quantize(paged.bf16_bits_to_f64(kb).astype(np.float32), scales[0]), scales[0])
            V = e4m3.dequantize(e4m3.quantize(paged.bf16_bits_to_f64(vb).astype(np.float32), scales[1]), scales[1])
        dense.append((K, V))
    q = bf16_bits(rng.standard_normal((len(lens), Hq, D)))
    return g, kc, vc, bt, np.array(lens, dtype=np.int32), q, dense


@pytest.mark.parametrize("Hq,Hkv,D,BS", [(4, 1, 64, 16), (8, 2, 32, 32), (16, 8, 128, 16), (6, 6, 64, 48)])
def test_matches_dense_contiguous_attention(Hq, Hkv, D, BS):
    rng = np.random.default_rng(Hq * 100 + BS)
    lens = [1, 17, 40, 5, 33]
    g, kc, vc, bt, sl, q, dense = make_paged(rng, lens, Hq, Hkv, D, BS)
    scale = 1 / math.sqrt(D)
    out = paged.decode(g, q, kc, vc, bt, sl, scale)
    qf = paged.bf16_bits_to_f64(q)
    for s, (K, V) in enumerate(dense):
        ref = paged.dense_attention(qf[s], K, V, scale)
        assert np.max(np.abs(out[s] - ref)) <= 1e-12


def test_fp8_matches_dense_on_dequantized_values():
    rng = np.random.default_rng(7)
    lens = [3, 40, 16]
    scales = (np.float32(0.011), np.float32(0.0093))
    g, kc, vc, bt, sl, q, dense = make_paged(rng, lens, 8, 2, 64, 16, "fp8", scales=scales)
    out = paged.decode(g, q, kc, vc, bt, sl, 0.125, k_scale=scales[0], v_scale=scales[1])
    qf = paged.bf16_bits_to_f64(q)
    for s, (K, V) in enumerate(dense):
        assert np.max(np.abs(out[s] - paged.dense_attention(qf[s], K, V, 0.125))) <= 1e-12


def test_offsets_and_reshape_describe_the_same_layout():
    for kv_dtype in ("bf16", "fp8"):
        g = paged.Geom(3, 32, 2, 64, kv_dtype)
        k = np.zeros(g.cache_elems, dtype=np.int64)
        v = np.zeros(g.cache_elems, dtype=np.int64)
        for blk in range(3):
            for h in range(2):
                for t in range(32):
                    for d in range(64):
                        tag = ((blk * 2 + h) * 32 + t) * 64 + d
                        k[paged.k_offset(g, blk, h, t, d)] = tag
                        v[paged.v_offset(g, blk, h, t, d)] = tag
        assert sorted(k.tolist()) == list(range(g.cache_elems))
        assert sorted(v.tolist()) == list(range(g.cache_elems))
        r = g.r
        kt = k.reshape(3, 2, 2, 64 // g.x, 16, g.x)
        vt = v.reshape(3, 2, 2, 64 // (16 * r), 16, 4, r, 4)
        for blk in range(3):
            for h in range(2):
                K = kt[blk, h].transpose(0, 2, 1, 3).reshape(32, 64)
                V = vt[blk, h].transpose(0, 3, 5, 1, 4, 2).reshape(32, 64)
                want = ((blk * 2 + h) * 32 + np.arange(32)[:, None]) * 64 + np.arange(64)[None, :]
                assert np.array_equal(K, want) and np.array_equal(V, want)


def test_invariant_under_physical_block_relabelling():
    rng = np.random.default_rng(3)
    g, kc, vc, bt, sl, q, _ = make_paged(rng, [17, 40, 5, 64], 8, 2, 64, 16, extra_blocks=5)
    out = paged.decode(g, q, kc, vc, bt, sl, 0.125)
    perm = rng.permutation(g.num_blocks)            # new id of old block b is perm[b]
    per_block = g.cache_elems // g.num_blocks
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    for b in range(g.num_blocks):
        kc2[perm[b] * per_block:(perm[b] + 1) * per_block] = kc[b * per_block:(b + 1) * per_block]
        vc2[perm[b] * per_block:(perm[b] + 1) * per_block] = vc[b * per_block:(b + 1) * per_block]
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    out2 = paged.decode(g, q, kc2, vc2, bt2, sl, 0.125)
    assert np.array_equal(out, out2)


def test_shared_blocks_equal_duplicated_blocks():
    rng = np.random.default_rng(4)
    BS, Hkv, D = 16, 2, 32
    # Three sequences share their first three blocks.
    g = paged.Geom(20, BS, Hkv, D)
    kc = bf16_bits(rng.standard_normal(g.cache_elems))
    vc = bf16_bits(rng.standard_normal(g.cache_elems))
    bt = np.array([[0, 1, 2, 3, 4], [0, 1, 2, 5, -1], [0, 1, 2, 6, 7]], dtype=np.int32)
    sl = np.array([70, 60, 80], dtype=np.int32)
    q = bf16_bits(rng.standard_normal((3, 4, D)))
    out = paged.decode(g, q, kc, vc, bt, sl, 0.2)
    per_block = g.cache_elems // g.num_blocks
    kc2, vc2 = kc.copy(), vc.copy()
    bt2 = bt.copy()
    nxt = 8
    for s in (1, 2):
        for j in range(3):
            src = bt[s, j]
            kc2[nxt * per_block:(nxt + 1) * per_block] = kc[src * per_block:(src + 1) * per_block]
            vc2[nxt * per_block:(nxt + 1) * per_block] = vc[src * per_block:(src + 1) * per_block]
            bt2[s, j] = nxt
            nxt += 1
    assert len(set(bt2[:, :3].ravel().tolist())) == 9
    out2 = paged.decode(g, q, kc2, vc2, bt2, sl, 0.2)
    assert np.array_equal(out, out2)


def test_brute_force_tiny_scalar_loops():
    """The tiny workload's shapes (4 query heads on 1 KV head, head_dim 64,
    block 16, lengths 17, 40, 5), computed with scalar loops, math.exp and
    math.fsum straight off the block table."""
    rng = np.random.default_rng(1)
    g, kc, vc, bt, sl, q, _ = make_paged(rng, [17, 40, 5], 4, 1, 64, 16, extra_blocks=10)
    scale = 1 / 8
    out = paged.decode(g, q, kc, vc, bt, sl, scale)
    qf = paged.bf16_bits_to_f64(q)
    kf = paged.bf16_bits_to_f64(kc)
    vf = paged.bf16_bits_to_f64(vc)
    for s in range(3):
        for i in range(4):
            logits = []
            for t in range(int(sl[s])):
                blk = int(bt[s][t // 16])
                dot = math.fsum(qf[s, i, d] * kf[paged.k_offset(g, blk, 0, t % 16, d)] for d in range(64))
                logits.append(scale * dot)
            mx = max(logits)
            w = [math.exp(z - mx) for z in logits]
            den = math.fsum(w)
            for d in range(64):
                num = math.fsum(w[t] * vf[paged.v_offset(g, int(bt[s][t // 16]), 0, t % 16, d)]
                                for t in range(len(w)))
                assert abs(out[s, i, d] - num / den) <= 1e-12


def test_closed_forms():
    rng = np.random.default_rng(5)
    D = 32
    K = rng.standard_normal((50, D))
    V = rng.standard_normal((50, D))
    q = rng.standard_normal((3, D))
    # One token: the output is that token's value.
    assert np.array_equal(paged.softmax_attention(q, K[:1], V[:1], 0.3), np.repeat(V[:1], 3, 0))
    # Zero query or zero scale: the mean of the values.
    assert np.allclose(paged.softmax_attention(np.zeros((2, D)), K, V, 0.3), V.mean(0), atol=1e-14)
    assert np.allclose(paged.softmax_attention(q, K, V, 0.0), V.mean(0), atol=1e-14)
    # All keys equal: the mean of the values.
    assert np.allclose(paged.softmax_attention(q, np.repeat(K[:1], 50, 0), V, 0.3), V.mean(0), atol=1e-14)
    # One logit ahead of the rest by >= 50: that token's value.
    Kp = np.zeros((50, D))
    Kp[17, 0] = 60.0
    qp = np.zeros((1, D))
    qp[0, 0] = 1.0
    assert np.max(np.abs(paged.softmax_attention(qp, Kp, V, 1.0)[0] - V[17])) < 1e-17 * 50 * 10
    # Empty sequence: zeros.
    assert np.array_equal(paged.softmax_attention(q, K[:0], V[:0], 0.3), np.zeros((3, D)))


def test_gqa_reduces_to_per_head_mha_and_shares_groups():
    rng = np.random.default_rng(6)
    lens = [9, 31, 50]
    g, kc, vc, bt, sl, q, dense = make_paged(rng, lens, 4, 4, 32, 16)
    out = paged.decode(g, q, kc, vc, bt, sl, 0.25)
    qf = paged.bf16_bits_to_f64(q)
    for s, (K, V) in enumerate(dense):
        for i in range(4):
            assert np.max(np.abs(out[s, i] - paged.softmax_attention(qf[s, i:i + 1], K[:, i], V[:, i], 0.25)[0])) < 1e-13
    # Identical query rows inside one group give identical outputs.
    g2, kc2, vc2, bt2, sl2, q2, _ = make_paged(rng, lens, 8, 2, 32, 16)
    q2[:, 1] = q2[:, 0]
    q2[:, 6] = q2[:, 5]
    out2 = paged.decode(g2, q2, kc2, vc2, bt2, sl2, 0.25)
    assert np.array_equal(out2[:, 1], out2[:, 0]) and np.array_equal(out2[:, 6], out2[:, 5])


def test_split_k_identity():
    """Merging the softmax states of any partition of the tokens equals the
    single pass (a self-test of the merge rule; the reference stays the
    single pass)."""
    rng = np.random.default_rng(8)
    K = rng.standard_normal((1000, 64))
    K[rng.choice(1000, 10, replace=False)] *= 8
    V = rng.standard_normal((1000, 64))
    q = rng.standard_normal((8, 64))
    ref = paged.softmax_attention(q, K, V, 1 / 8)
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 1000), size=rng.integers(1, 20), replace=False))
        edges = [0, *cuts.tolist(), 1000]
        states = [paged.partial_state(q, K[a:b], V[a:b], 1 / 8) for a, b in zip(edges[:-1], edges[1:])]
        assert np.max(np.abs(paged.lse_merge(states) - ref)) < 1e-13


def test_cache_write_touches_only_its_slots():
    rng = np.random.default_rng(9)
    g = paged.Geom(6, 32, 2, 64)
    kc = bf16_bits(rng.standard_normal(g.cache_elems))
    vc = bf16_bits(rng.standard_normal(g.cache_elems))
    k0, v0 = kc.copy(), vc.copy()
    kn = bf16_bits(rng.standard_normal((4, 2, 64)))
    vn = bf16_bits(rng.standard_normal((4, 2, 64)))
    slots = np.array([5, -1, 33, 6 * 32], dtype=np.int64)   # one skipped, one out of range
    paged.cache_write_bf16(g, kn, vn, slots, kc, vc)
    changed_k = np.nonzero(kc != k0)[0]
    expect = sorted(paged.k_offset(g, b, h, o, d) for (b, o) in [(0, 5), (1, 1)]
                    for h in range(2) for d in range(64))
    assert set(changed_k.tolist()) <= set(expect)
    for j, (b, o) in ((0, (0, 5)), (2, (1, 1))):
        for h in range(2):
            idx = [paged.k_offset(g, b, h, o, d) for d in range(64)]
            assert np.array_equal(kc[idx], kn[j, h])
            idx = [paged.v_offset(g, b, h, o, d) for d in range(64)]
            assert np.array_equal(vc[idx], vn[j, h])


# ---------------------------------------------------------------- planted mistakes
def _dense_pin_fails():
    try:
        test_matches_dense_contiguous_attention(8, 2, 32, 32)
    except AssertionError:
        return True
    return False


def test_planted_wrong_head_mapping_is_caught(monkeypatch):
    orig = paged.gather

    def bad(g, kc, vc, row, L, h, *a, **k):
        return orig(g, kc, vc, row, L, (h + 1) % g.num_kv_heads, *a, **k)
    monkeypatch.setattr(paged, "gather", bad)
    assert _dense_pin_fails()


def test_planted_missing_scale_is_caught(monkeypatch):
    orig = paged.softmax_attention
    monkeypatch.setattr(paged, "softmax_attention", lambda q, K, V, scale: orig(q, K, V, 1.0))
    assert _dense_pin_fails()


def test_planted_transposed_k_tile_is_caught(monkeypatch):
    def bad_gather(g, kc, vc, row, L, h, k_scale=1.0, v_scale=1.0):
        nblk = -(-L // g.block_size)
        sb = g.block_size // 16
        kt = kc.reshape(g.num_blocks, g.num_kv_heads, sb, g.head_dim // g.x, 16, g.x)[row[:nblk], h]
        vt = vc.reshape(g.num_blocks, g.num_kv_heads, sb, g.head_dim, 16)[row[:nblk], h]
        K = kt.reshape(nblk * g.block_size, g.head_dim)      # forgot the transpose
        V = vt.transpose(0, 1, 3, 2).reshape(nblk * g.block_size, g.head_dim)
        return paged.bf16_bits_to_f64(K[:L]), paged.bf16_bits_to_f64(V[:L])
    monkeypatch.setattr(paged, "gather", bad_gather)
    assert _dense_pin_fails()


def test_planted_off_by_one_block_index_is_caught(monkeypatch):
    orig = paged.slot_to_block
    monkeypatch.setattr(paged, "slot_to_block", lambda slot, bs: orig(slot + 1, bs))
    with pytest.raises(AssertionError):
        test_cache_write_touches_only_its_slots()


# ---------------------------------------------------------------- sliding window
def test_window_positions_follow_the_pages_trace(pages):
    """A four-token window over ten tokens keeps the printed positions after
    every token ("KV Cache Engineering for LLM Serving", section 3)."""
    c = pages["sliding_window_trace"]
    for p in range(c["tokens"]):
        assert paged.window_positions(p + 1, c["window"]) == c["retained_after_token"][p]
    assert max(len(paged.window_positions(L, c["window"])) for L in range(50)) == c["max_retained"]
    assert paged.window_positions(7, 0) == list(range(7))


@pytest.mark.parametrize("W", [1, 5, 16, 17, 33, 64, 1000])
def test_window_decode_is_dense_attention_over_the_window(W):
    rng = np.random.default_rng(40 + W)
    lens = [1, 9, 40, 77, 130]
    g, kc, vc, bt, sl, q, dense = make_paged(rng, lens, 8, 2, 32, 16)
    out = paged.decode(g, q, kc, vc, bt, sl, 0.3, window=W)
    qf = paged.bf16_bits_to_f64(q)
    for s, (K, V) in enumerate(dense):
        lo = max(0, lens[s] - W)
        ref = paged.dense_attention(qf[s], K[lo:], V[lo:], 0.3)
        assert np.max(np.abs(out[s] - ref)) < 1e-12, (W, s)
    if W >= max(lens):        # a window at least as long as every sequence is full attention
        assert np.array_equal(out, paged.decode(g, q, kc, vc, bt, sl, 0.3))


def test_window_of_one_returns_the_last_value_and_ignores_released_blocks():
    rng = np.random.default_rng(77)
    lens = [20, 47, 64]
    g, kc, vc, bt, sl, q, dense = make_paged(rng, lens, 4, 1, 32, 16)
    out = paged.decode(g, q, kc, vc, bt, sl, 0.3, window=1)
    for s, (K, V) in enumerate(dense):
        assert np.array_equal(out[s], np.repeat(V[-1:, 0], 4, 0))
    # Table entries of blocks before the window are never read.
    W = 20
    ref = paged.decode(g, q, kc, vc, bt, sl, 0.3, window=W)
    bt2 = bt.copy()
    for s, L in enumerate(lens):
        bt2[s, :max(0, L - W) // 16] = -1
    assert np.array_equal(paged.decode(g, q, kc, vc, bt2, sl, 0.3, window=W), ref)


def test_a_lost_or_doubled_piece_leaves_the_parity_envelope():
    """Why the GPU parity tests check an accuracy envelope beside the
    contract bounds.  Planted in the oracle: a long unit (9,000 tokens, the
    length the many-piece GPU test uses) merged by log-sum-exp with one
    16-token piece dropped, or counted twice.  With N(0, 1) queries, keys and
    values the output moves by about 1/563 of a value, which the contract's
    max-abs 1e-2 can miss but the envelope's 1e-4 cannot."""
    from tests.gpu_helpers import BF16_ENVELOPE, BF16_TOL
    rng = np.random.default_rng(7)
    L, G, D, P = 9000, 8, 128, 16
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    scale = 1 / math.sqrt(D)
    pieces = [paged.partial_state(q, K[i:i + P], V[i:i + P], scale) for i in range(0, L, P)]
    whole = paged.lse_merge(pieces)
    assert np.abs(whole - paged.softmax_attention(q, K, V, scale)).max() < 1e-12
    moved = []
    for j in (0, 100, 400, len(pieces) - 1):
        lost = paged.lse_merge(pieces[:j] + pieces[j + 1:])
        twice = paged.lse_merge(pieces + [pieces[j]])
        for bad in (lost, twice):
            moved.append(np.abs(bad - whole).max())
    assert min(moved) > 10 * BF16_ENVELOPE
    assert min(moved) < BF16_TOL[0]          # the contract bound alone would not have caught some


@pytest.mark.parametrize("W,BS", [(1, 16), (16, 16), (33, 16), (64, 32), (100, 48)])
def test_ring_decode_through_the_manager_is_dense_attention_over_the_window(W, BS):
    """Local-layer sequences in ring tables kept by the manager model: each
    token's K/V goes to the slot the manager hands out, and after every step
    the ring decode (logical block b at entry b % entries) equals dense
    attention over the raw rows of the last W positions, which never pass
    through the cache.  The sequences go round their rings several times,
    one of them from a prompt that starts part-way round."""
    from oracle import blocks as B
    rng = np.random.default_rng(900 + W + BS)
    Hq, Hkv, D = 4, 2, 32
    nblk = 40
    g = paged.Geom(nblk, BS, Hkv, D)
    kc = np.full(g.cache_elems, 0x7FC0, dtype=np.uint16)       # NaN everywhere not written
    vc = kc.copy()
    bm = B.BlockManager(nblk, BS)
    prompts = [0, 5, 3 * W + 7]
    raw = []
    for s, n in enumerate(prompts):
        E = bm.add_ring_sequence(s, n, W)
        kb = bf16_bits(rng.standard_normal((n, Hkv, D)))
        vb = bf16_bits(rng.standard_normal((n, Hkv, D)))
        paged.cache_write_bf16(g, kb, vb, np.array(bm.slots(s, 0, n), dtype=np.int64), kc, vc)
        raw.append([kb, vb])
    assert E == -(-W // BS) + 1
    q = bf16_bits(rng.standard_normal((len(prompts), Hq, D)))
    qf = paged.bf16_bits_to_f64(q)
    steps = 2 * E * BS + 3
    for step in range(steps):
        for s in range(len(prompts)):
            slot, src, dst = bm.append_token(s, 0)
            assert src == -1
            kb = bf16_bits(rng.standard_normal((1, Hkv, D)))
            vb = bf16_bits(rng.standard_normal((1, Hkv, D)))
            paged.cache_write_bf16(g, kb, vb, np.array([slot], dtype=np.int64), kc, vc)
            raw[s] = [np.concatenate([raw[s][0], kb]), np.concatenate([raw[s][1], vb])]
        if step % 3 and step != steps - 1:
            continue
        bt = np.array([bm.table(s) for s in range(len(prompts))], dtype=np.int32)
        sl = np.array([bm.length(s) for s in range(len(prompts))], dtype=np.int32)
        assert bt.shape[1] == E
        out = paged.decode(g, q, kc, vc, bt, sl, 0.3, window=W, ring=True)
        for s in range(len(prompts)):
            K = paged.bf16_bits_to_f64(raw[s][0][-W:])
            V = paged.bf16_bits_to_f64(raw[s][1][-W:])
            ref = paged.dense_attention(qf[s], K, V, 0.3)
            assert np.max(np.abs(out[s] - ref)) < 1e-12, (step, s)
