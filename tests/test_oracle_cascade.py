"""The shared-prefix (cascade) decomposition in the oracle: the segments of
a hand-built batch, brute-force pairwise common prefixes, maximality, and
the merged parts equal to plain decode."""

import itertools
import random

import numpy as np
import pytest

from oracle import cascade as C
from oracle import paged
from paged_kv_cache_32_amd import workloads as W


def canon(segments):
    return sorted((s["first"], tuple(s["blocks"]), tuple(sorted(s["members"]))) for s in segments)


def test_hand_built_batch():
    BS = 4
    tables = [[1, 2, 3, 4, 9, 10],     # A
              [1, 2, 3, 4, 7, 0],      # B
              [1, 2, 3, 5, 0, 0],      # C
              [1, 2, 6, 0, 0, 0],      # D
              [8, 0, 0, 0, 0, 0]]      # E
    lens = [5 * BS + 1, 4 * BS + 3, 4 * BS, 3 * BS, 2]
    segs, prefix = C.shared_segments(tables, lens, BS)
    assert canon(segs) == [(0, (1, 2), (0, 1, 2, 3)), (2, (3,), (0, 1, 2)), (3, (4,), (0, 1))]
    assert prefix == [4 * BS, 4 * BS, 3 * BS, 2 * BS, 0]
    # B's block 7 at position 4 is partial (4 * BS + 3 tokens): never shared,
    # even with a sequence holding the same id there
    tables2 = [t[:] for t in tables]
    tables2[0][4] = 7
    segs2, prefix2 = C.shared_segments(tables2, lens, BS)
    assert canon(segs2) == canon(segs) and prefix2 == prefix
    # with three members required, the A-B run is private again
    segs3, prefix3 = C.shared_segments(tables, lens, BS, min_members=3)
    assert canon(segs3) == [(0, (1, 2), (0, 1, 2, 3)), (2, (3,), (0, 1, 2))]
    assert prefix3 == [3 * BS, 3 * BS, 3 * BS, 2 * BS, 0]


def common_full_prefix(tables, lens, BS, s, t):
    n = 0
    while n < lens[s] // BS and n < lens[t] // BS and tables[s][n] == tables[t][n]:
        n += 1
    return n


@pytest.mark.parametrize("seed", range(6))
def test_segments_against_brute_force(seed):
    """On random trees of shared prefixes: segment blocks are each member's
    blocks there; any two sequences share exactly their common full-block
    prefix through segments they both belong to; runs are maximal; each
    sequence's private part starts at its deepest shared block."""
    r = random.Random(seed)
    BS = r.choice([2, 4, 16])
    S = r.randrange(2, 14)
    next_id = [100]

    def fresh():
        next_id[0] += 1
        return next_id[0]
    stems = [[fresh() for _ in range(r.randrange(0, 6))] for _ in range(3)]
    branches = {}
    tables, lens = [], []
    for s in range(S):
        st = r.choice(stems)[:r.randrange(0, 7)]
        bkey = (tuple(st), r.randrange(3))
        if bkey not in branches:
            branches[bkey] = [fresh() for _ in range(r.randrange(0, 4))]
        row = st + branches[bkey][:r.randrange(0, 5)] + [fresh() for _ in range(r.randrange(0, 3))]
        nfull = len(row)
        L = nfull * BS + r.randrange(0, BS)
        if L % BS:
            row = row + [fresh()]
        tables.append(row + [0] * (12 - len(row)))
        lens.append(L)
    segs, prefix = C.shared_segments(tables, lens, BS)
    for seg in segs:
        assert len(seg["members"]) >= 2
        for s in seg["members"]:
            j = seg["first"]
            assert tables[s][j:j + len(seg["blocks"])] == seg["blocks"]
            assert j + len(seg["blocks"]) <= lens[s] // BS
    for s, t in itertools.combinations(range(S), 2):
        n = common_full_prefix(tables, lens, BS, s, t)
        both = [seg for seg in segs if s in seg["members"] and t in seg["members"]]
        covered = sorted((seg["first"], seg["first"] + len(seg["blocks"])) for seg in both)
        pos = 0
        for a, b in covered:                       # contiguous from 0
            assert a == pos
            pos = b
        assert pos == n, (s, t)
    for seg in segs:                               # maximal: no further common block, no extra member
        end = seg["first"] + len(seg["blocks"])
        m = seg["members"]
        nxt = {tables[s][end] if end < lens[s] // BS else None for s in m}
        assert not (len(nxt) == 1 and None not in nxt and all(
            common_full_prefix(tables, lens, BS, s2, m[0]) >= end + 1 for s2 in m))
        others = [s2 for s2 in range(S) if s2 not in m and common_full_prefix(tables, lens, BS, s2, m[0]) >= end]
        assert not others
    for s in range(S):
        deepest = max([common_full_prefix(tables, lens, BS, s, t) for t in range(S) if t != s] + [0])
        assert prefix[s] == deepest * BS


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_decode_by_parts_equals_plain_decode(kv_dtype):
    """The prefix-shared workload's structure at a small size: a system
    prompt, prefix pools, private suffixes; the merged parts equal plain
    decode, and the shared segments are the ones the generator built."""
    w = W.prefix_shared(num_seqs=12, system_tokens=70, num_pools=3, pool_range=(40, 90), suffix_median=20,
                        max_len=400, block_size=16, num_kv_heads=2, num_q_heads=8, head_dim=64, seed=5,
                        kv_dtype=kv_dtype, pool_share=0.5)
    g = paged.Geom(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, kv_dtype)
    rng = np.random.default_rng(1)
    if kv_dtype == "bf16":
        kc = (rng.integers(0, 1 << 16, g.cache_elems).astype(np.uint16) & 0xBFFF)   # finite values
        vc = (rng.integers(0, 1 << 16, g.cache_elems).astype(np.uint16) & 0xBFFF)
        ks = vs = 1.0
    else:
        kc = rng.integers(0, 126, g.cache_elems).astype(np.uint8)
        vc = rng.integers(0, 126, g.cache_elems).astype(np.uint8)
        ks, vs = 0.02, 0.03
    qb = (rng.integers(0, 1 << 16, (w.num_seqs, 8, 64)).astype(np.uint16) & 0xBFFF)
    ref = paged.decode(g, qb, kc, vc, w.block_tables, w.seq_lens, 0.1, k_scale=ks, v_scale=vs)
    got = C.decode(g, qb, kc, vc, w.block_tables, w.seq_lens, 0.1, ks, vs)
    assert np.max(np.abs(got - ref)) < 1e-12
    segs, prefix = C.shared_segments(w.block_tables, w.seq_lens, w.block_size)
    assert segs and max(len(s["members"]) for s in segs) == w.num_seqs    # the system prompt
    assert all(p % w.block_size == 0 for p in prefix)
