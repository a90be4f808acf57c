"""The block-manager model in the oracle, pinned to the pages' printed traces
and to the invariants the rules imply."""

import random

import numpy as np
import pytest

from oracle import blocks as B
from oracle import paged


def unique_tokens(start, n):
    return list(range(start, start + n))


def test_free_list_trace_of_the_paging_section(pages):
    """Six free blocks; A takes three, B two; A finishes; C takes two
    ("KV Cache Engineering for LLM Serving", section 10, printed output)."""
    c = pages["free_list_trace"]
    bm = B.BlockManager(len(c["free"]), 4)
    bm.add_sequence("A", unique_tokens(100, 12))
    bm.add_sequence("B", unique_tokens(200, 8))
    assert bm.table("A") == c["request_a"] and bm.table("B") == c["request_b"]
    bm.free_sequence("A")
    assert bm.free == c["free_after_a"]
    bm.add_sequence("C", unique_tokens(300, 8))
    assert bm.table("C") == c["request_c"]


def test_prefix_reuse_of_the_prefix_section(pages):
    """Four-token blocks: the first request reuses 0 of 3 blocks, the second
    (same first 8 tokens) 2 of 3 and computes 1 new block (same page,
    section 11, printed output)."""
    c = pages["prefix_reuse"]
    bm = B.BlockManager(16, c["block_size"])
    assert bm.add_sequence(1, c["first"]) == c["first_reused"]
    assert len(bm.table(1)) == c["blocks"]
    assert bm.add_sequence(2, c["second"]) == c["second_reused"]
    assert bm.misses - c["blocks"] == c["second_new"]
    t1, t2 = bm.table(1), bm.table(2)
    assert t2[:2] == t1[:2] and t2[2] != t1[2]
    assert [bm.ref[b] for b in t1] == [2, 2, 1]


def test_whole_prefix_and_model_key_must_match():
    """Matching tokens in the middle reuse nothing; identical tokens under
    another model / adapter key reuse nothing (rajatmohan.com, "Prefix
    sharing is where the real win lives")."""
    bm = B.BlockManager(32, 4)
    first = [10, 11, 12, 13, 20, 21, 22, 23, 30, 31, 32, 33]
    bm.add_sequence(1, first)
    assert bm.add_sequence(2, [99, 98, 97, 96] + first[4:]) == 0
    assert set(bm.table(2)).isdisjoint(bm.table(1))
    assert bm.add_sequence(3, first, model=7) == 0
    assert bm.add_sequence(4, first, model=0) == 3


def test_partial_blocks_are_never_shared_by_key():
    bm = B.BlockManager(8, 4)
    bm.add_sequence(1, [1, 2, 3, 4, 5, 6])
    assert bm.add_sequence(2, [1, 2, 3, 4, 5, 6]) == 1
    assert bm.table(1)[0] == bm.table(2)[0] and bm.table(1)[1] != bm.table(2)[1]


def test_block_address_rule_for_appends():
    """The slot of position i is table[i // bs] * bs + i % bs ("Taming the
    token torrent", "The Block Table Logic")."""
    bm = B.BlockManager(8, 4)
    bm.add_sequence(1, [5, 6, 7])
    slots = [bm.append_token(1, t)[0] for t in range(10)]
    t = bm.table(1)
    assert slots == [t[i // 4] * 4 + i % 4 for i in range(3, 13)]


def test_fork_and_copy_on_write():
    bm = B.BlockManager(8, 4)
    bm.add_sequence("p", [1, 2, 3, 4, 5, 6])          # one full block, one partial
    bm.fork("p", "c")
    full, part = bm.table("p")
    assert bm.ref[full] == 2 and bm.ref[part] == 2
    slot, src, dst = bm.append_token("c", 9)          # c writes into the shared partial block
    assert src == part and dst not in (full, part) and bm.table("c") == [full, dst]
    assert slot == dst * 4 + 2 and bm.ref[part] == 1 and bm.ref[dst] == 1
    slot, src, dst = bm.append_token("p", 8)          # p now holds its block alone: no copy
    assert (src, dst) == (-1, -1) and slot == part * 4 + 2
    # completing the block stores it under its key: an equal prompt reuses it
    bm.append_token("p", 7)
    assert bm.add_sequence("q", [1, 2, 3, 4, 5, 6, 8, 7]) == 2


def test_out_of_blocks_changes_nothing():
    bm = B.BlockManager(3, 4)
    bm.add_sequence(1, unique_tokens(0, 8))
    before = (list(bm.free), list(bm.ref), dict(bm.key_block))
    with pytest.raises(B.OutOfBlocks):
        bm.add_sequence(2, unique_tokens(50, 9))
    assert (list(bm.free), list(bm.ref), dict(bm.key_block)) == before and 2 not in bm.seqs
    bm.add_sequence(3, unique_tokens(90, 4))
    with pytest.raises(B.OutOfBlocks):
        bm.append_token(3, 1)
    assert bm.length(3) == 4


def random_ops(bm, rng, steps, vocab=3, max_prompt=14):
    """Random mix of adds (small vocabulary, so prefixes repeat), forks,
    appends and frees; yields the result of each operation."""
    live, next_id = [], 0
    for _ in range(steps):
        op = rng.random()
        try:
            if op < 0.3 or not live:
                n = rng.randrange(0, max_prompt)
                toks = [rng.randrange(vocab) for _ in range(n)]
                model = rng.randrange(2)
                r = bm.add_sequence(next_id, toks, model)
                live.append(next_id)
                yield ("add", next_id, r)
                next_id += 1
            elif op < 0.4:
                p = rng.choice(live)
                bm.fork(p, next_id)
                live.append(next_id)
                yield ("fork", p, next_id)
                next_id += 1
            elif op < 0.85:
                s = rng.choice(live)
                yield ("append", s, bm.append_token(s, rng.randrange(vocab)))
            else:
                s = live.pop(rng.randrange(len(live)))
                bm.free_sequence(s)
                yield ("free", s)
        except (B.OutOfBlocks, B.Swapped) as e:
            yield (type(e).__name__,)


def check_invariants(bm, num_blocks):
    counts = [0] * num_blocks
    for s in bm.seqs.values():
        for b in s["table"]:
            counts[b] += 1
        assert len(s["table"]) == -(-len(s["tokens"]) // bm.block_size)
    assert counts == bm.ref                       # reference count = tables naming the block
    assert sorted(bm.free) == [b for b in range(num_blocks) if counts[b] == 0]
    for key, b in bm.key_block.items():           # a stored block holds exactly its key's tokens
        model, prefix = key
        assert bm.ref[b] > 0 and len(prefix) % bm.block_size == 0
        holders = [s for s in bm.seqs.values() if b in s["table"]]
        for s in holders:
            i = s["table"].index(b)
            assert tuple(s["tokens"][:(i + 1) * bm.block_size]) == prefix and s["model"] == model


@pytest.mark.parametrize("seed", range(4))
def test_random_operations_keep_the_invariants(seed):
    rng = random.Random(seed)
    bm = B.BlockManager(40, 4)
    for i, _ in enumerate(random_ops(bm, rng, 600)):
        if i % 25 == 0:
            check_invariants(bm, 40)
    check_invariants(bm, 40)


def test_copy_blocks_moves_exactly_the_blocks_elements():
    """A block of the cache layout is one contiguous run of
    Hkv * block_size * D elements: the oracle's layout offsets of every
    (head, token, dim) of block b fill exactly that run."""
    g = paged.Geom(num_blocks=5, block_size=32, num_kv_heads=2, head_dim=64)
    E = g.num_kv_heads * g.block_size * g.head_dim
    h, t, d = np.meshgrid(np.arange(g.num_kv_heads), np.arange(g.block_size), np.arange(g.head_dim),
                          indexing="ij")
    for b in range(g.num_blocks):
        for off in (paged.k_offset, paged.v_offset):
            o = np.sort(off(g, b, h, t, d).ravel())
            assert np.array_equal(o, np.arange(b * E, (b + 1) * E))
    k = np.arange(g.cache_elems, dtype=np.int64)
    v = -k
    B.copy_blocks(k, v, [(1, 3), (4, 0)], E)
    assert np.array_equal(k[3 * E:4 * E], np.arange(E, 2 * E)) and np.array_equal(k[0:E], np.arange(4 * E, 5 * E))
    assert np.array_equal(v[3 * E:4 * E], -np.arange(E, 2 * E))
    assert np.array_equal(k[E:3 * E], np.arange(E, 3 * E))   # sources untouched


def test_trim_releases_blocks_outside_the_window():
    bm = B.BlockManager(12, 4)
    sysp = unique_tokens(0, 8)                       # two full shared blocks
    bm.add_sequence("a", sysp + unique_tokens(100, 9))
    bm.add_sequence("b", sysp + unique_tokens(200, 3))
    ta, tb = bm.table("a"), bm.table("b")
    assert ta[:2] == tb[:2]
    free0 = bm.num_free()
    # a has 17 tokens; keeping the last 6 keeps positions 11..16 (blocks 2..4)
    assert bm.trim("a", 6) == 2
    assert bm.table("a")[:2] == [-1, -1] and bm.table("a")[2:] == ta[2:]
    assert bm.num_free() == free0                    # the shared blocks are still held by b
    assert [bm.ref[b] for b in tb[:2]] == [1, 1]
    assert bm.trim("a", 6) == 0                      # idempotent
    slot, _, _ = bm.append_token("a", 5)             # positions keep their logical blocks
    assert slot == ta[4] * 4 + 1
    bm.free_sequence("b")
    assert bm.free[-3:] == tb                        # b's blocks, now unreferenced, in table order
    bm.free_sequence("a")
    check_invariants_with_trims(bm, 12)
    with pytest.raises(ValueError):
        bm.trim("x", 0)


def check_invariants_with_trims(bm, num_blocks):
    counts = [0] * num_blocks
    for s in bm.seqs.values():
        for b in s["table"]:
            if b >= 0:
                counts[b] += 1
    assert counts == bm.ref
    assert sorted(bm.free) == [b for b in range(num_blocks) if counts[b] == 0]


@pytest.mark.parametrize("seed", range(3))
def test_random_operations_with_trims_keep_the_invariants(seed):
    rng = random.Random(100 + seed)
    bm = B.BlockManager(30, 4)
    for i, _ in enumerate(random_ops(bm, rng, 500)):
        if bm.seqs and rng.random() < 0.2:
            s = rng.choice(list(bm.seqs))
            bm.trim(s, rng.randrange(1, 12))
        if i % 20 == 0:
            check_invariants_with_trims(bm, 30)
    check_invariants_with_trims(bm, 30)


def test_offload_trace_of_the_offloading_section(pages):
    """A pool with room for two sessions: C's arrival moves A out, A's return
    moves B out ("KV Cache Engineering for LLM Serving", section 12, printed
    output).  On each side of the trace, the sessions whose blocks are on the
    GPU and those swapped to the host are the ones the page prints."""
    c = pages["offload_trace"]
    per = 3                                            # blocks per session
    bm = B.BlockManager(c["gpu_sessions"] * per, 4)
    name = {"a": "cache-a", "b": "cache-b", "c": "cache-c"}
    toks = {s: unique_tokens(100 * i, 4 * per) for i, s in enumerate("abc")}
    host = {}

    def state():
        gpu = [name[s] for s in bm.seqs if not bm.seqs[s]["swapped"]]
        cpu = [name[s] for s in bm.seqs if bm.seqs[s]["swapped"]]
        return gpu, cpu

    bm.add_sequence("a", toks["a"])
    bm.add_sequence("b", toks["b"])
    with pytest.raises(B.OutOfBlocks):
        bm.add_sequence("c", toks["c"])
    table_a = bm.table("a")
    host["a"] = bm.swap_out("a")
    assert host["a"] == table_a and bm.table("a") == [B.SWAPPED] * per
    bm.add_sequence("c", toks["c"])
    gpu, cpu = state()
    assert sorted(gpu) == sorted(c["gpu_after_c_arrives"]) and cpu == c["cpu_after_c_arrives"]
    with pytest.raises(B.OutOfBlocks):
        bm.swap_in("a")
    assert bm.table("a") == [B.SWAPPED] * per        # nothing changed
    host["b"] = bm.swap_out("b")
    back = bm.swap_in("a")
    assert bm.table("a") == back and len(back) == per
    gpu, cpu = state()
    assert sorted(gpu) == sorted(c["gpu_after_a_returns"]) and cpu == c["cpu_after_a_returns"]
    # A's full blocks are stored under their keys again: an equal prompt reuses them
    assert bm.num_free() == 0 and bm.add_sequence("a2", toks["a"][:8]) == 2
    check_invariants_with_swaps(bm, c["gpu_sessions"] * per)


def test_swap_keeps_shared_blocks_and_refuses_updates():
    """Only blocks no other sequence holds move out; the shared prefix stays
    ("Taming the token torrent", "The Swapping Mechanism").  A swapped
    sequence takes no appends, forks or trims until it is swapped in."""
    bm = B.BlockManager(16, 4)
    sysp = unique_tokens(0, 8)
    bm.add_sequence("a", sysp + unique_tokens(100, 6))
    bm.add_sequence("b", sysp + unique_tokens(200, 2))
    ta = bm.table("a")
    free0 = bm.num_free()
    out = bm.swap_out("a")
    assert out == ta[2:] and bm.table("a") == ta[:2] + [B.SWAPPED, B.SWAPPED]
    assert bm.num_free() == free0 + 2 and [bm.ref[b] for b in ta[:2]] == [2, 2]
    for op in (lambda: bm.append_token("a", 1), lambda: bm.fork("a", "z"), lambda: bm.trim("a", 2),
               lambda: bm.swap_out("a")):
        with pytest.raises(B.Swapped):
            op()
    with pytest.raises(B.Swapped):
        bm.swap_in("b")
    back = bm.swap_in("a")
    assert bm.table("a") == ta[:2] + back
    slot, src, dst = bm.append_token("a", 7)          # the partial block is private again
    assert (src, dst) == (-1, -1) and slot == back[1] * 4 + 2
    # a swapped sequence's table entries are not references: freeing it
    # releases only what it still holds
    bm.swap_out("b")
    bm.free_sequence("b")
    check_invariants_with_swaps(bm, 16)


def check_invariants_with_swaps(bm, num_blocks):
    check_invariants_with_trims(bm, num_blocks)
    for s in bm.seqs.values():
        assert (B.SWAPPED in s["table"]) <= s["swapped"]


@pytest.mark.parametrize("seed", range(3))
def test_random_operations_with_swaps_keep_the_invariants(seed):
    rng = random.Random(200 + seed)
    bm = B.BlockManager(30, 4)
    ops = random_ops(bm, rng, 500)
    for i in range(500):
        swapped = [s for s in bm.seqs if bm.seqs[s]["swapped"]]
        try:
            if swapped and rng.random() < 0.3:
                bm.swap_in(rng.choice(swapped))
            elif bm.seqs and rng.random() < 0.1:
                bm.swap_out(rng.choice([s for s in bm.seqs if s not in swapped] or [None]))
            else:
                next(ops)
        except (B.OutOfBlocks, B.Swapped, KeyError):
            pass
        if i % 20 == 0:
            check_invariants_with_swaps(bm, 30)
    check_invariants_with_swaps(bm, 30)


def test_swap_image_round_trip():
    """A host copy holds each listed block's K elements, then its V elements,
    every (head, token, dim) of the block (located through the oracle's
    layout offsets); restoring it into other blocks moves exactly those."""
    g = paged.Geom(num_blocks=7, block_size=16, num_kv_heads=2, head_dim=64)
    E = g.num_kv_heads * g.block_size * g.head_dim
    k = np.arange(g.cache_elems, dtype=np.int64)
    v = 10 ** 6 + k
    blocks = [5, 1, 4]
    img = B.swap_image(k, v, blocks, E)
    assert img.shape == (2 * len(blocks) * E,)
    h, t, d = 1, 9, 33
    for i, b in enumerate(blocks):
        assert img[i * E + paged.k_offset(g, b, h, t, d) - b * E] == k[paged.k_offset(g, b, h, t, d)]
        j = len(blocks) + i
        assert img[j * E + paged.v_offset(g, b, h, t, d) - b * E] == v[paged.v_offset(g, b, h, t, d)]
    k2, v2 = np.zeros_like(k), np.zeros_like(v)
    B.swap_restore(k2, v2, [0, 6, 2], img, E)
    for src, dst in zip(blocks, [0, 6, 2]):
        assert np.array_equal(k2[dst * E:(dst + 1) * E], k[src * E:(src + 1) * E])
        assert np.array_equal(v2[dst * E:(dst + 1) * E], v[src * E:(src + 1) * E])
    assert not k2[E:2 * E].any() and not v2[3 * E:6 * E].any()
    assert B.swap_image(k, v, [], E).size == 0


# ---------------------------------------------------------------- ring tables
def test_ring_sequence_keeps_its_window_and_takes_no_blocks_once_full():
    """A local layer's sequence in a ring of ceil(W / BS) + 1 entries ("KV
    Cache Engineering for LLM Serving", section 3: each new entry displaces
    the oldest).  After every append, each of the last W positions still
    reads back the value it wrote (no later token wrote over its slot), the
    ring's blocks are the only blocks it holds, and once the ring is full
    the pool no longer changes."""
    bs, W = 4, 8
    bm = B.BlockManager(30, bs)
    E = bm.add_ring_sequence("a", 0, W)
    assert E == 3 and bm.table("a") == [-1, -1, -1]
    content = {}                                    # slot -> position written there last
    written = []
    for p in range(60):
        slot, src, dst = bm.append_token("a", 7)
        assert (src, dst) == (-1, -1)
        content[slot] = p
        written.append(slot)
        L = p + 1
        lo = max(0, L - W)
        got = bm.slots("a", lo, L - lo)
        assert got == written[lo:L]
        assert all(content[s] == q for q, s in zip(range(lo, L), got)), p
        assert len(bm.table("a")) == E
        held = [b for b in bm.table("a") if b >= 0]
        assert len(held) == min(-(-L // bs), E) and 30 - bm.num_free() == len(held)
    # positions whose block has left the ring have no slot
    nb = -(-60 // bs)
    assert bm.slots("a", 0, (nb - E) * bs) == [-1] * ((nb - E) * bs)
    assert bm.slots("a", (nb - E) * bs, 1)[0] >= 0
    bm.free_sequence("a")
    assert bm.num_free() == 30


def test_ring_prompt_holds_its_last_blocks():
    bm = B.BlockManager(10, 4)
    assert bm.add_ring_sequence("b", 23, 8) == 3    # 6 logical blocks; the last 3 are held
    t = bm.table("b")
    assert sorted(t) == [0, 1, 2] and t == [0, 1, 2]  # logical 3, 4, 5 at entries 0, 1, 2
    s = bm.slots("b", 0, 23)
    assert s[:12] == [-1] * 12 and s[12:] == [0 * 4 + i for i in range(4)] + [4 + i for i in range(4)] + [8, 9, 10]
    with pytest.raises(B.OutOfBlocks):
        bm.add_ring_sequence("c", 100, 40)          # 11 entries, 7 free blocks
    assert bm.num_free() == 7 and "c" not in bm.seqs
    with pytest.raises(ValueError):
        bm.add_ring_sequence("d", 5, 0)


def test_ring_fork_copies_shared_blocks_before_writing_them():
    bm = B.BlockManager(12, 4)
    bm.add_ring_sequence("c", 10, 8)                # logical blocks 0, 1, 2 at entries 0, 1, 2
    t0 = bm.table("c")
    bm.fork("c", "d")
    assert all(bm.ref[b] == 2 for b in t0)
    # c writes position 10 into shared logical block 2: copy first
    slot, src, dst = bm.append_token("c", 1)
    assert src == t0[2] and dst not in t0 and slot == dst * 4 + 2
    # d now holds block t0[2] alone: written in place
    assert bm.append_token("d", 1) == (t0[2] * 4 + 2, -1, -1)
    bm.append_token("c", 1)
    # c starts logical block 3 on entry 0, whose block d still shares: a fresh block
    slot, src, dst = bm.append_token("c", 1)
    assert (src, dst) == (-1, -1) and slot // 4 not in t0 and bm.ref[t0[0]] == 1
    bm.append_token("d", 1)
    # d starts logical block 3 on entry 0, whose block only d holds now: reused in place
    assert bm.append_token("d", 1) == (t0[0] * 4, -1, -1)
    check_invariants_with_trims(bm, 12)


def test_ring_trim_releases_blocks_before_the_kept_tokens():
    bm = B.BlockManager(10, 4)
    bm.add_ring_sequence("e", 20, 8)                # logical 2, 3, 4 held
    t = bm.table("e")
    assert bm.trim("e", 3) == 2                     # keeps positions 17..19: logical block 4 only
    assert bm.table("e") == [-1, t[1], -1]          # entries 2 % 3 and 3 % 3 released; 4 % 3 kept
    assert bm.slots("e", 16, 4) == [t[1] * 4 + i for i in range(4)]
    assert bm.slots("e", 12, 4) == [-1] * 4
    slot, _, _ = bm.append_token("e", 0)            # position 20: logical 5, entry 2: a fresh block
    assert slot % 4 == 0 and bm.table("e")[2] == slot // 4
    check_invariants_with_trims(bm, 10)


def ring_ops_with_contents(seed, num_blocks, bs, steps):
    """Random ring adds, forks, appends (with their copy-on-write copies),
    trims, swaps out and in and frees on the model, simulating what each
    slot holds: every token written gets a unique id, block copies and swap
    images move the ids, and after each operation every live sequence's
    window positions must read back their own ids."""
    rng = random.Random(seed)
    bm = B.BlockManager(num_blocks, bs)
    content = {}                 # slot -> token id
    ids = {}                     # seq -> token id of every position
    window = {}
    images = {}
    nid = [0]

    def fresh_id():
        nid[0] += 1
        return nid[0]

    def copy_block(src, dst):
        for o in range(bs):
            if src * bs + o in content:
                content[dst * bs + o] = content[src * bs + o]

    live, swapped, nxt = [], set(), 0
    for step in range(steps):
        op = rng.random()
        resident = [s for s in live if s not in swapped]
        if op < 0.12 or not resident:
            n, W = rng.randrange(0, 6 * bs), rng.randrange(1, 3 * bs)
            try:
                bm.add_ring_sequence(nxt, n, W)
            except B.OutOfBlocks:
                continue
            ids[nxt] = [fresh_id() for _ in range(n)]
            window[nxt] = W
            for p, s in enumerate(bm.slots(nxt, 0, n)):
                if s >= 0:
                    content[s] = ids[nxt][p]
            live.append(nxt)
            nxt += 1
        elif op < 0.2:
            p = rng.choice(resident)
            bm.fork(p, nxt)
            ids[nxt], window[nxt] = list(ids[p]), window[p]
            live.append(nxt)
            nxt += 1
        elif op < 0.75:
            s = rng.choice(resident)
            try:
                slot, src, dst = bm.append_token(s, 0)
            except B.OutOfBlocks:
                continue
            if src >= 0:
                copy_block(src, dst)
            ids[s].append(fresh_id())
            content[slot] = ids[s][-1]
        elif op < 0.8:
            s = rng.choice(resident)
            bm.trim(s, rng.randrange(window[s], 3 * bs + window[s]))
        elif op < 0.86:
            s = rng.choice(resident)
            out = bm.swap_out(s)
            images[s] = [[content.get(b * bs + o) for o in range(bs)] for b in out]
            swapped.add(s)
        elif op < 0.93 and swapped:
            s = rng.choice(sorted(swapped))
            try:
                new = bm.swap_in(s)
            except B.OutOfBlocks:
                continue
            for b, img in zip(new, images.pop(s)):
                for o, v in enumerate(img):
                    if v is not None:
                        content[b * bs + o] = v
            swapped.discard(s)
        else:
            s = live.pop(rng.randrange(len(live)))
            swapped.discard(s)
            images.pop(s, None)
            bm.free_sequence(s)
        check_invariants_with_trims(bm, num_blocks)
        for s in live:
            if s in swapped:
                continue
            L = len(ids[s])
            lo = max(0, L - window[s])
            for p, slot in zip(range(lo, L), bm.slots(s, lo, L - lo)):
                assert slot >= 0 and content[slot] == ids[s][p], (step, s, p)
    return bm


@pytest.mark.parametrize("seed,num_blocks,bs", [(0, 40, 4), (1, 25, 3), (2, 64, 16), (3, 12, 2)])
def test_random_ring_operations_keep_every_window_readable(seed, num_blocks, bs):
    ring_ops_with_contents(seed, num_blocks, bs, 1200)
