"""The Quest oracle (query-aware page selection), pinned to the page's
printed example, to the bound the score is defined to be, to brute force on
tiny inputs, and to plain decode and textbook attention."""

import itertools
import random

import numpy as np
import pytest

from oracle import paged
from oracle import quest as Q


def bf16_bits(x):
    """float64 -> bf16 bit patterns, round to nearest even (test inputs)."""
    f = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def test_page_example_scores_and_choice(pages):
    """Four pages of two 2-d keys, query (1, 0.5): scores 2.5, 6.0, 4.0,
    -1.0; the two best pages are 1 and 2, so 4 of the 8 stored entries are
    read ("KV Cache Engineering for LLM Serving", section 7, printed output)."""
    c = pages["quest_example"]
    keys = np.array(c["pages"], dtype=np.float64)          # [page, key, dim]
    sc = Q.page_scores(np.array([c["query"]]), keys.min(axis=1), keys.max(axis=1))
    assert sc.tolist() == c["scores"]
    sel = Q.select_pages(sc, c["keep"])
    assert sel == c["selected"]
    assert len(sel) * keys.shape[1] == c["entries_read"] and keys.shape[0] * keys.shape[1] == c["entries_stored"]


def example_in_cache(c, kv_dtype="bf16"):
    """The example's four pages as four 16-token blocks of a cache with
    head_dim 32: block p holds page p's two keys in its first two tokens and
    copies of them after (copies change no minimum or maximum); the other
    dimensions are 0, and so is the query there.  Blocks are placed in the
    pool in a shuffled order."""
    keys = np.array(c["pages"], dtype=np.float64)
    D, BS = 32, 16
    g = paged.Geom(num_blocks=6, block_size=BS, num_kv_heads=1, head_dim=D, kv_dtype=kv_dtype)
    table = [4, 0, 5, 2]
    L = 4 * BS
    K = np.zeros((L, 1, D))
    for p in range(4):
        for t in range(BS):
            K[p * BS + t, 0, :2] = keys[p, t % 2]
    rng = np.random.default_rng(0)
    V = rng.standard_normal((L, 1, D))
    kc = np.zeros(g.cache_elems, g.np_dtype)
    vc = np.zeros(g.cache_elems, g.np_dtype)
    slots = [table[i // BS] * BS + i % BS for i in range(L)]
    paged.cache_write_bf16(g, bf16_bits(K), bf16_bits(V), slots, kc, vc)
    q = np.zeros((1, 1, D))
    q[0, 0, :2] = c["query"]
    return g, kc, vc, np.array([table], np.int32), np.array([L], np.int32), bf16_bits(q), K, \
        paged.bf16_bits_to_f64(bf16_bits(V))


def test_page_example_through_the_cache(pages):
    """The same example end to end: summaries rebuilt from the paged cache
    layout, scores, choice, and attention over the chosen blocks' tokens."""
    c = pages["quest_example"]
    g, kc, vc, bt, sl, qb, K, V = example_in_cache(c)
    mn, mx = Q.empty_summaries(g)
    Q.summarize(g, kc, bt[0], [16] * 4, mn, mx)
    assert Q.selection(g, qb, mn, mx, bt, sl, c["keep"]) == [[c["selected"]]]
    out, _ = Q.decode(g, qb, kc, vc, bt, sl, mn, mx, c["keep"], 0.5)
    rows = [p * 16 + t for p in c["selected"] for t in range(16)]
    ref = paged.dense_attention(paged.bf16_bits_to_f64(qb)[0], K[rows], V[rows], 0.5)
    assert np.max(np.abs(out[0] - ref)) < 1e-12
    full, _ = Q.decode(g, qb, kc, vc, bt, sl, mn, mx, 4, 0.5)
    assert np.max(np.abs(full[0] - paged.dense_attention(paged.bf16_bits_to_f64(qb)[0], K, V, 0.5))) < 1e-12


def exact_score(q, mn, mx):
    """The score in float64 (exact for these bf16 inputs: 2-d products of
    8-bit significands summed well inside 53 bits), for the bound checks."""
    return np.maximum(q * mn, q * mx).sum()


@pytest.mark.parametrize("seed", range(3))
def test_score_bounds_every_key_of_the_page(seed):
    """Every key k of a page has q.k <= the page's score (the box bound);
    a page of one key scores exactly q.k; the float32 score is within its
    rounding bound of the exact one."""
    rng = np.random.default_rng(seed)
    D, n, per = 64, 40, 16
    keys = paged.bf16_bits_to_f64(bf16_bits(rng.standard_normal((n, per, D)) * rng.uniform(0.1, 3, (n, 1, 1))))
    q = paged.bf16_bits_to_f64(bf16_bits(rng.standard_normal(D)))
    mn, mx = keys.min(axis=1), keys.max(axis=1)
    sc = Q.page_scores(q[None], mn, mx)
    for p in range(n):
        ex = exact_score(q, mn[p], mx[p])
        terms = np.abs(np.maximum(q * mn[p], q * mx[p])).sum()
        assert abs(float(sc[p]) - ex) <= D * 2.0 ** -24 * terms
        assert (keys[p] @ q <= ex + 1e-12).all()
    one = Q.page_scores(q[None], keys[:, 0], keys[:, 0])
    ex1 = keys[:, 0] @ q
    assert np.all(np.abs(one - ex1) <= D * 2.0 ** -24 * np.abs(keys[:, 0] * q).sum(axis=1))


def test_score_sums_in_dimension_order_in_float32():
    """The float32 sum runs in dimension order: with terms 2^24, 1, -2^24
    the 1 is lost (float32 gives 0); any other order or a float64 sum would
    give 1."""
    q = np.array([[1.0, 1.0, 1.0]])
    v = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)]])
    assert Q.page_scores(q, v, v).tolist() == [0.0]
    v2 = np.array([[2.0 ** 24, -(2.0 ** 24), 1.0]])
    assert Q.page_scores(q, v2, v2).tolist() == [1.0]


def test_group_score_is_the_largest_head_score():
    rng = np.random.default_rng(5)
    D, n, G = 32, 25, 4
    q = paged.bf16_bits_to_f64(bf16_bits(rng.standard_normal((G, D))))
    mn = paged.bf16_bits_to_f64(bf16_bits(rng.standard_normal((n, D)) - 1))
    mx = mn + np.abs(paged.bf16_bits_to_f64(bf16_bits(rng.standard_normal((n, D)))))
    mx = paged.bf16_bits_to_f64(bf16_bits(mx))
    per_head = np.stack([Q.page_scores(q[g:g + 1], mn, mx) for g in range(G)])
    assert np.array_equal(Q.page_scores(q, mn, mx), per_head.max(axis=0))


@pytest.mark.parametrize("seed", range(20))
def test_choice_against_brute_force(seed):
    """Among all subsets of the budget's size, the chosen one is the single
    subset whose every member beats every non-member on (score, -index)."""
    r = random.Random(seed)
    n = r.randrange(1, 9)
    scores = np.array([r.choice([-1.0, 0.0, 2.5, 2.5, 7.0]) for _ in range(n)], np.float32)
    budget = r.randrange(0, n + 2)
    got = Q.select_pages(scores, budget)
    if budget >= n:
        assert got == list(range(n))
        return
    good = [list(c) for c in itertools.combinations(range(n), budget)
            if all((scores[i], -i) > (scores[j], -j) for i in c for j in range(n) if j not in c)]
    assert good == [got]


def test_budget_covering_every_page_is_plain_decode():
    rng = np.random.default_rng(7)
    g = paged.Geom(num_blocks=30, block_size=16, num_kv_heads=2, head_dim=64)
    S, G = 4, 3
    lens = np.array([1, 16, 37, 100], np.int32)
    perm = rng.permutation(g.num_blocks).astype(np.int32)
    bt = perm[:S * 7].reshape(S, 7)
    kc = bf16_bits(rng.standard_normal(g.cache_elems))
    vc = bf16_bits(rng.standard_normal(g.cache_elems))
    qb = bf16_bits(rng.standard_normal((S, G * 2, 64)))
    mn, mx = Q.empty_summaries(g)
    for s in range(S):
        pages = -(-int(lens[s]) // 16)
        counts = [16] * (pages - 1) + [int(lens[s]) - 16 * (pages - 1)]
        Q.summarize(g, kc, bt[s, :pages], counts, mn, mx)
    out, chosen = Q.decode(g, qb, kc, vc, bt, lens, mn, mx, 7, 0.125)
    ref = paged.decode(g, qb, kc, vc, bt, lens, 0.125)
    assert np.max(np.abs(out - ref)) < 1e-13
    assert all(chosen[s][h] == list(range(-(-int(lens[s]) // 16))) for s in range(S) for h in range(2))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_quest_decode_is_attention_over_the_chosen_tokens(kv_dtype):
    """With a small budget, each (sequence, KV head) output equals textbook
    attention over the tokens of its chosen pages, rebuilt from the dense
    keys the cache was written from; the chosen pages are the best by the
    page scores of the summaries, recomputed here from dense keys."""
    rng = np.random.default_rng(11)
    BS, D, Hkv, G = 16, 64, 2, 4
    g = paged.Geom(num_blocks=40, block_size=BS, num_kv_heads=Hkv, head_dim=D, kv_dtype=kv_dtype)
    lens = [150, 33, 200]
    S = len(lens)
    perm = rng.permutation(g.num_blocks)
    tables = np.full((S, 13), -1, np.int32)
    kc = np.zeros(g.cache_elems, g.np_dtype)
    vc = np.zeros(g.cache_elems, g.np_dtype)
    Ks, Vs, used = [], [], 0
    ks = vs = 1.0
    if kv_dtype == "fp8":
        ks, vs = 3.0 / 448, 2.5 / 448
    for s, L in enumerate(lens):
        nb = -(-L // BS)
        tables[s, :nb] = perm[used:used + nb]
        used += nb
        K = rng.standard_normal((L, Hkv, D)) * np.where(rng.random((L, 1, 1)) < 0.1, 3.0, 0.5)
        V = rng.standard_normal((L, Hkv, D))
        slots = [tables[s, i // BS] * BS + i % BS for i in range(L)]
        if kv_dtype == "bf16":
            paged.cache_write_bf16(g, bf16_bits(K), bf16_bits(V), slots, kc, vc)
        else:
            paged.cache_write_fp8(g, bf16_bits(K), bf16_bits(V), slots, kc, vc, np.float32(ks), np.float32(vs))
        Ks.append(K)
        Vs.append(V)
    qb = bf16_bits(rng.standard_normal((S, Hkv * G, D)))
    mn, mx = Q.empty_summaries(g)
    for s, L in enumerate(lens):
        nb = -(-L // BS)
        Q.summarize(g, kc, tables[s, :nb], [BS] * (nb - 1) + [L - BS * (nb - 1)], mn, mx)
    budget = 3
    out, chosen = Q.decode(g, qb, kc, vc, tables, lens, mn, mx, budget, 0.1, ks, vs)
    q = paged.bf16_bits_to_f64(qb)
    for s, L in enumerate(lens):
        for h in range(Hkv):
            Kh, Vh = paged.gather(g, kc, vc, tables[s], L, h, ks, vs)
            vals = Kh / ks                        # stored values, recomputed from the gather

            nb = -(-L // BS)
            pmn = np.array([vals[p * BS:min(L, (p + 1) * BS)].min(axis=0) for p in range(nb)])
            pmx = np.array([vals[p * BS:min(L, (p + 1) * BS)].max(axis=0) for p in range(nb)])
            sc = Q.page_scores(q[s, h * G:(h + 1) * G].astype(np.float32), pmn, pmx)
            assert chosen[s][h] == Q.select_pages(sc, budget)
            rows = [p * BS + t for p in chosen[s][h] for t in range(BS) if p * BS + t < L]
            ref = paged.dense_attention(q[s, h * G:(h + 1) * G], Kh[rows][:, None], Vh[rows][:, None], 0.1)
            assert np.max(np.abs(out[s, h * G:(h + 1) * G] - ref)) < 1e-12
        assert len(chosen[s][0]) == min(budget, -(-L // BS))


def test_fp8_summaries_hold_code_values_without_the_scale():
    g = paged.Geom(num_blocks=2, block_size=16, num_kv_heads=1, head_dim=32, kv_dtype="fp8")
    kc = np.zeros(g.cache_elems, np.uint8)
    vc = np.zeros(g.cache_elems, np.uint8)
    k = np.zeros((3, 1, 32))
    k[:, 0, 0] = [1.0, -2.0, 0.5]
    paged.cache_write_fp8(g, bf16_bits(k), bf16_bits(k), [16, 17, 18], kc, vc, np.float32(0.5), np.float32(1))
    mn, mx = Q.block_summary(g, kc, 1, 3)
    assert mn[0, 0] == -4.0 and mx[0, 0] == 2.0 and mn[0, 1] == 0.0 and mx[0, 1] == 0.0


def test_nan_keys_are_ignored_and_empty_blocks_are_inf():
    g = paged.Geom(num_blocks=2, block_size=16, num_kv_heads=1, head_dim=32)
    kc = np.zeros(g.cache_elems, np.uint16)
    vc = np.zeros(g.cache_elems, np.uint16)
    k = np.zeros((2, 1, 32))
    k[0, 0, 3] = np.nan
    k[1, 0, 3] = -1.5
    paged.cache_write_bf16(g, bf16_bits(k), bf16_bits(k), [0, 1], kc, vc)
    mn, mx = Q.block_summary(g, kc, 0, 2)
    assert mn[0, 3] == -1.5 and mx[0, 3] == -1.5
    e0, e1 = Q.block_summary(g, kc, 1, 0)
    assert np.isposinf(e0).all() and np.isneginf(e1).all()


@pytest.mark.parametrize("seed", range(3))
def test_write_maintained_summaries_equal_recomputed(seed):
    """Q6: summaries kept by the writes (a reset at offset 0, then a merge
    per written token) equal summaries recomputed over each block's written
    tokens, through prefill writes of many tokens per block, one-token decode
    writes, padding slots, and blocks freed and reused by new sequences."""
    rng = np.random.default_rng(seed)
    r = random.Random(seed)
    BS = 16
    g = paged.Geom(num_blocks=12, block_size=BS, num_kv_heads=2, head_dim=32)
    kc = bf16_bits(rng.standard_normal(g.cache_elems) * 7)   # stale contents everywhere
    vc = np.zeros(g.cache_elems, np.uint16)
    mn, mx = Q.empty_summaries(g)
    free = list(range(g.num_blocks))
    seqs = {}                                      # seq -> [table, length]
    count = {}                                     # block -> tokens written since offset 0
    for step in range(80):
        slots = []
        if not seqs or r.random() < 0.3:           # a prefill
            L = r.randrange(1, 50)
            nb = -(-L // BS)
            if nb <= len(free):
                table = [free.pop(0) for _ in range(nb)]
                seqs[step] = [table, L]
                slots = [table[i // BS] * BS + i % BS for i in range(L)]
        elif r.random() < 0.2:                     # a sequence ends
            s = r.choice(list(seqs))
            free.extend(seqs.pop(s)[0])
        else:                                      # a decode step
            for s, (table, L) in list(seqs.items()):
                if L % BS == 0:
                    if not free:
                        continue
                    table.append(free.pop(0))
                slots.append(table[L // BS] * BS + L % BS)
                seqs[s][1] = L + 1
        for _ in range(r.randrange(0, 3)):                         # padding and out-of-pool slots
            slots.insert(r.randrange(len(slots) + 1), r.choice([-1, -7, g.num_blocks * BS]))
        if r.random() < 0.5:
            r.shuffle(slots)
        k = bf16_bits(rng.standard_normal((len(slots), 2, 32)))
        paged.cache_write_bf16(g, k, k, slots, kc, vc)
        Q.update_summaries(g, kc, slots, mn, mx)
        offs = {}
        for x in slots:
            if 0 <= x < g.num_blocks * BS:
                offs.setdefault(x // BS, []).append(x % BS)
        for b, o in offs.items():                  # tokens written since the block's offset 0
            count[b] = max(o) + 1 if 0 in o else max(count.get(b, 0), max(o) + 1)
        for b, c in count.items():
            a, z = Q.block_summary(g, kc, b, c)
            assert np.array_equal(mn[b], a) and np.array_equal(mx[b], z), (step, b)
        assert all(np.isposinf(mn[b]).all() for b in range(g.num_blocks) if b not in count)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sequence_page_summaries_equal_block_summaries(kv_dtype):
    rng = np.random.default_rng(3)
    g = paged.Geom(num_blocks=9, block_size=32, num_kv_heads=2, head_dim=64, kv_dtype=kv_dtype)
    if kv_dtype == "bf16":
        kc = bf16_bits(rng.standard_normal(g.cache_elems))
    else:
        kc = rng.integers(0, 256, g.cache_elems).astype(np.uint8)
        kc[(kc & 0x7F) == 0x7F] = 0x11                    # no NaN codes
    row = [7, 2, 5, 0]
    for L in (1, 32, 33, 100, 128):
        for h in range(2):
            mn, mx = Q.sequence_page_summaries(g, kc, row, L, h)
            pages = -(-L // 32)
            assert mn.shape == (pages, 64)
            for p in range(pages):
                a, z = Q.block_summary(g, kc, row[p], min(32, L - 32 * p))
                assert np.array_equal(mn[p], a[h]) and np.array_equal(mx[p], z[h])
