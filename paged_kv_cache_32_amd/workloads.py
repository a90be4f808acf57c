"""Seeded synthetic workloads for paged decode.

This module only builds inputs: sequence lengths, block pools and block
tables, slot mappings and random tensors.  It holds none of the decode or
quantizer arithmetic and imports neither the HIP binding nor the oracle, so
the kernels and the oracle can both be fed from it.

The five workloads follow the traffic the pages describe: a 70B-class layer
with 64 query heads, 8 KV heads and head dimension 128; prompt lengths with a
median of 2,400 tokens and a p95 around 18,000 (rajatmohan.com serving
design, "traffic"); a 900-token system prompt on every chat request and about
62% of prompt tokens already computed as someone else's prefix (same page,
"Prefix sharing is where the real win lives"); blocks of 16 or 32 tokens
(same page, "Paging, because contiguous allocation is a disaster").  The real
traffic is not available; these generators stand in for it.

Host-side structure (lengths, tables, slots) is drawn with
``numpy.random.default_rng(seed)``; tensor contents are drawn with a seeded
``torch.Generator`` on the device the tensors are made on.
"""

import math
from dataclasses import dataclass, field
from statistics import NormalDist

import numpy as np
import torch

SUB = 16                      # tokens per sub-block of the cache layout
BF16_NAN = 0x7FC0             # poison for bf16 cache slots nobody may read
FP8_NAN = 0x7F                # poison for e4m3fn cache slots
LOGN_MEDIAN = 2400.0
LOGN_P95 = 18000.0
LOGN_SIGMA = math.log(LOGN_P95 / LOGN_MEDIAN) / NormalDist().inv_cdf(0.95)


class FreeList:
    """FIFO pool of free block ids: allocation pops from the head, a finished
    request returns its blocks to the tail ("KV Cache Engineering for LLM
    Serving", section 10, Paging)."""

    def __init__(self, blocks):
        self.free = [int(b) for b in blocks]

    def alloc(self, n):
        if n > len(self.free):
            raise MemoryError(f"pool exhausted: need {n}, have {len(self.free)}")
        got, self.free = self.free[:n], self.free[n:]
        return got

    def release(self, blocks):
        self.free.extend(int(b) for b in blocks)


class PrefixBlockCache:
    """Full-block prefix sharing: a block is reused only when every token up
    to its end matches an earlier request, so its key is the key of the
    previous block plus this block's tokens (chained keys; "KV Cache
    Engineering for LLM Serving", section 11, Prefix reuse; rajatmohan.com,
    "Prefix sharing is where the real win lives").  Keys are interned
    exactly, so there are no hash collisions.  A partly filled block is never
    shared."""

    def __init__(self, free_list):
        self.free_list = free_list
        self.key_ids = {}         # (prev key id, block tokens) -> key id
        self.block_of_key = {}    # key id -> physical block
        self.hits = 0
        self.misses = 0

    def blocks_for(self, tokens, block_size):
        table = []
        prev = -1
        n_full = len(tokens) // block_size
        for b in range(n_full):
            k = (prev, tuple(tokens[b * block_size:(b + 1) * block_size]))
            kid = self.key_ids.get(k)
            if kid is not None:
                self.hits += 1
                table.append(self.block_of_key[kid])
            else:
                self.misses += 1
                kid = len(self.key_ids)
                self.key_ids[k] = kid
                blk = self.free_list.alloc(1)[0]
                self.block_of_key[kid] = blk
                table.append(blk)
            prev = kid
        if len(tokens) % block_size:
            table.extend(self.free_list.alloc(1))
        return table


@dataclass
class Workload:
    """Host-side description of one paged-decode workload."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seq_lens: np.ndarray          # int32 [S]; includes the token written this step
    block_tables: np.ndarray      # int32 [S, max_blocks]; -1 past each sequence's blocks
    slot_mapping: np.ndarray      # int64 [S]; slot of each sequence's new token
    scale: float
    kv_dtype: str = "bf16"        # "bf16" or "fp8"
    num_layers: int = 1
    seed: int = 0
    k_row_boost: float = 0.0      # fraction of K rows scaled by k_row_factor
    k_row_factor: float = 8.0
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return len(self.seq_lens)

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    @property
    def elem_bytes(self):
        return 2 if self.kv_dtype == "bf16" else 1

    @property
    def cache_elems(self):
        return self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim

    def used_blocks(self):
        """Physical blocks referenced by some block table (unique)."""
        bt = self.block_tables
        return np.unique(bt[bt >= 0])

    def logical_kv_bytes(self):
        """K+V bytes one decode call reads per layer, counting shared blocks
        once per sequence that reads them."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * \
            self.head_dim * self.elem_bytes

    def physical_kv_bytes(self):
        """K+V bytes of distinct cached tokens per layer (shared blocks once)."""
        seen = {}
        for s in range(self.num_seqs):
            L = int(self.seq_lens[s])
            nblk = -(-L // self.block_size)
            for j in range(nblk):
                blk = int(self.block_tables[s, j])
                valid = min(self.block_size, L - j * self.block_size)
                seen[blk] = max(seen.get(blk, 0), valid)
        toks = sum(seen.values())
        return toks * 2 * self.num_kv_heads * self.head_dim * self.elem_bytes

    def summary(self):
        L = self.seq_lens.astype(np.int64)
        ub = len(self.used_blocks())
        logical_blocks = int(sum(-(-int(x) // self.block_size) for x in L))
        return {
            "workload": self.name, "num_seqs": self.num_seqs,
            "num_q_heads": self.num_q_heads, "num_kv_heads": self.num_kv_heads,
            "head_dim": self.head_dim, "block_size": self.block_size,
            "num_blocks": self.num_blocks, "num_layers": self.num_layers,
            "kv_dtype": self.kv_dtype, "tokens": int(L.sum()),
            "len_median": float(np.median(L)), "len_max": int(L.max()),
            "used_blocks": ub, "logical_blocks": logical_blocks,
            "sharing_factor": logical_blocks / max(ub, 1),
            "pool_utilization": int(L.sum()) / max(ub * self.block_size, 1),
            **self.notes,
        }

    # ------------------------------------------------------------------ tensors
    def make_tensors(self, device, layers=None, poison=True):
        """Draw the step's tensors on ``device``.

        Returns a dict with, per layer (leading dimension = len(layers)):
          q        [n, S, Hq, D]  bf16 ~ N(0, 1)
          k_new    [n, S, Hkv, D] bf16 ~ N(0, 1) (the token written this step)
          v_new    [n, S, Hkv, D] bf16 ~ N(0, 1)
          k_cache  [n, cache_elems] bfloat16, or uint8 holding e4m3fn codes
          v_cache  [n, cache_elems]
          k_scale, v_scale  [n] float64 (fp8 only): max |x| / 448 over the
                   layer's drawn K (resp. V) values, new tokens included.
        Every cache element of every block is drawn; with ``poison`` the
        elements no decode may read (unreferenced blocks, token slots at or
        past each sequence's length, and the slot of the new token) are set to
        NaN so that a stray read shows up in the output.
        """
        layers = range(self.num_layers) if layers is None else list(layers)
        n = len(layers)
        dev = torch.device(device)
        S, Hq, Hkv, D = self.num_seqs, self.num_q_heads, self.num_kv_heads, self.head_dim
        cdt = torch.bfloat16 if self.kv_dtype == "bf16" else torch.uint8
        res = {
            "q": torch.empty((n, S, Hq, D), dtype=torch.bfloat16, device=dev),
            "k_new": torch.empty((n, S, Hkv, D), dtype=torch.bfloat16, device=dev),
            "v_new": torch.empty((n, S, Hkv, D), dtype=torch.bfloat16, device=dev),
            "k_cache": torch.empty((n, self.cache_elems), dtype=cdt, device=dev),
            "v_cache": torch.empty((n, self.cache_elems), dtype=cdt, device=dev),
        }
        scales = {"k": [], "v": []}
        poison_idx = self._poison_positions(dev) if poison else None
        free = self._free_blocks() if poison else []
        free_t = torch.tensor(free, dtype=torch.int64, device=dev)
        boost = self._boost_rows(dev) if self.k_row_boost > 0 else None
        nan = BF16_NAN if self.kv_dtype == "bf16" else FP8_NAN
        for li, layer in enumerate(layers):
            g = torch.Generator(device=dev)
            g.manual_seed(self.seed * 1000003 + layer)
            res["q"][li] = _randn_bf16((S, Hq, D), g, dev)
            res["k_new"][li] = _randn_bf16((S, Hkv, D), g, dev)
            res["v_new"][li] = _randn_bf16((S, Hkv, D), g, dev)
            for name in ("k", "v"):
                new = res[name + "_new"][li]
                vals = _randn_bf16((self.cache_elems,), g, dev)
                if name == "k" and boost is not None:
                    vals[boost] = vals[boost] * self.k_row_factor
                cache = res[name + "_cache"][li]
                if self.kv_dtype == "bf16":
                    cache.copy_(vals)
                else:
                    amax = max(float(vals.abs().max()), float(new.abs().max()))
                    sc = float(np.float32(amax / 448.0))
                    # Library cast (torch) of values already inside +-448.
                    codes = (vals.float() / sc).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
                    cache.copy_(codes.view(torch.uint8))
                    del codes
                    scales[name].append(sc)
                del vals
                if poison:
                    bits = cache.view(torch.int16) if self.kv_dtype == "bf16" else cache
                    if len(free):
                        bits.view(self.num_blocks, -1)[free_t] = nan
                    bits[poison_idx[name]] = nan
        if self.kv_dtype == "fp8":
            res["k_scale"] = torch.tensor(scales["k"], dtype=torch.float64)
            res["v_scale"] = torch.tensor(scales["v"], dtype=torch.float64)
        return res

    def _free_blocks(self):
        used = np.zeros(self.num_blocks, dtype=bool)
        used[self.used_blocks()] = True
        return np.nonzero(~used)[0].tolist()

    # Element indices of token rows, from the cache layout (X = 16 / element
    # bytes, R = 4 / element bytes):
    #   K (blk, h, t, d) at [blk][h][t//16][d//X][t%16][d%X]
    #   V (blk, h, t, d) at [blk][h][t//16][d//16R][d%16][(t%16)//4][(d//16)%R][t%4]
    def _row_elems(self, blk, tok, dev):
        """Flat K and V element indices of all (kv head, dim) of the given
        (block, token) rows; blk, tok: int64 tensors of equal length R.
        Returns two [R * Hkv * D] index tensors."""
        Hkv, D, BS = self.num_kv_heads, self.head_dim, self.block_size
        X = 16 // self.elem_bytes
        R = 4 // self.elem_bytes
        sb = BS // SUB
        h = torch.arange(Hkv, device=dev, dtype=torch.int64).view(1, Hkv, 1)
        d = torch.arange(D, device=dev, dtype=torch.int64).view(1, 1, D)
        b = blk.view(-1, 1, 1)
        t = tok.view(-1, 1, 1)
        tile = (b * Hkv + h) * sb + t // SUB
        tt = t % SUB
        k_idx = ((tile * (D // X) + d // X) * SUB + tt) * X + d % X
        v_idx = ((((tile * (D // (16 * R)) + d // (16 * R)) * 16 + d % 16) * 4 + tt // 4) * R
                 + (d // 16) % R) * 4 + tt % 4
        return k_idx.reshape(-1), v_idx.reshape(-1)

    def _poison_positions(self, dev):
        """Token rows inside referenced blocks that no decode may read."""
        BS = self.block_size
        blks, toks = [], []
        # Token slots at or past each sequence's length inside its last block,
        # unless another sequence holds a valid token there (shared blocks).
        valid = {}
        for s in range(self.num_seqs):
            L = int(self.seq_lens[s])
            for j in range(-(-L // BS)):
                blk = int(self.block_tables[s, j])
                valid[blk] = max(valid.get(blk, 0), min(BS, L - j * BS))
        for blk, nv in valid.items():
            for t in range(nv, BS):
                blks.append(blk)
                toks.append(t)
        for slot in self.slot_mapping:
            if slot >= 0:
                blks.append(int(slot) // BS)
                toks.append(int(slot) % BS)
        if not blks:
            e = torch.zeros(0, dtype=torch.int64, device=dev)
            return {"k": e, "v": e}
        k_idx, v_idx = self._row_elems(torch.tensor(blks, dtype=torch.int64, device=dev),
                                       torch.tensor(toks, dtype=torch.int64, device=dev), dev)
        return {"k": k_idx, "v": v_idx}

    def _boost_rows(self, dev):
        """K rows (one token of one KV head) picked, seeded and without
        replacement, among the rows of cached tokens, to be scaled."""
        rng = np.random.default_rng(self.seed + 7919)
        rows = []
        for s in range(self.num_seqs):
            L = int(self.seq_lens[s])
            rows.append((s, L))
        total = sum(L for _, L in rows) * self.num_kv_heads
        n = int(round(self.k_row_boost * total))
        pick = np.sort(rng.choice(total, size=n, replace=False))
        # row r -> (sequence, token, kv head) in (s, t, h) order
        starts = np.cumsum([0] + [L * self.num_kv_heads for _, L in rows])
        s_of = np.searchsorted(starts, pick, side="right") - 1
        rem = pick - starts[s_of]
        t_of = rem // self.num_kv_heads
        h_of = rem % self.num_kv_heads
        blk = self.block_tables[s_of, t_of // self.block_size].astype(np.int64)
        off = t_of % self.block_size
        BS, Hkv, D = self.block_size, self.num_kv_heads, self.head_dim
        X = 16 // self.elem_bytes
        sb = BS // SUB
        tile = (blk * Hkv + h_of) * sb + off // SUB
        d = np.arange(D)
        k_idx = ((tile[:, None] * (D // X) + d[None, :] // X) * SUB + (off % SUB)[:, None]) * X \
            + d[None, :] % X
        return torch.tensor(k_idx.reshape(-1), dtype=torch.int64, device=dev)


def _randn_bf16(shape, g, dev):
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)


def _tables_from_pool(lens, block_size, pool_order):
    """Block tables for sequences of the given lengths, each taking its blocks
    from the head of a FIFO free list in sequence order."""
    fl = FreeList(pool_order)
    nblk = [-(-int(L) // block_size) for L in lens]
    bt = np.full((len(lens), max(max(nblk), 1)), -1, dtype=np.int32)
    for s, n in enumerate(nblk):
        bt[s, :n] = fl.alloc(n)
    return bt


def _slots_for_last_token(lens, bt, block_size):
    slots = np.full(len(lens), -1, dtype=np.int64)
    for s, L in enumerate(lens):
        if L > 0:
            pos = int(L) - 1
            slots[s] = int(bt[s, pos // block_size]) * block_size + pos % block_size
    return slots


def lognormal_lengths(rng, n, lo=16, hi=32768):
    """Prompt lengths with median 2,400 and p95 about 18,000, rounded and
    clipped to [lo, hi]."""
    x = rng.lognormal(mean=math.log(LOGN_MEDIAN), sigma=LOGN_SIGMA, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def _pool_size(needed_blocks, factor=1.25):
    return int(math.ceil(factor * needed_blocks))


def tiny(seed=1, new_token_at_end=True):
    """4 query heads sharing 1 KV head, head_dim 64, block_size 16, 16 blocks;
    3 sequences of lengths 17, 40 and 5 whose block tables come from a seeded
    permutation of the free blocks; scale 1/sqrt(64).

    With ``new_token_at_end`` the lengths include this step's token (written
    at positions 16, 39 and 4); otherwise the cached prefix has those lengths
    and the new token goes after it (positions 17, 40, 5; lengths 18, 41, 6).
    """
    rng = np.random.default_rng(seed)
    base = np.array([17, 40, 5], dtype=np.int32)
    lens = base if new_token_at_end else base + 1
    bt = _tables_from_pool(lens, 16, rng.permutation(16))
    return Workload("tiny_gqa4_d64", 4, 1, 64, 16, 16, lens, bt,
                    _slots_for_last_token(lens, bt, 16), 1.0 / math.sqrt(64), seed=seed)


def llama70b_layer(seed=2, num_seqs=64, block_size=16, kv_dtype="bf16", num_layers=1,
                   name="llama70b_layer_bs64", tp=1):
    """A Llama-70B-shaped layer: 64 query heads, 8 KV heads, head_dim 128;
    lognormal lengths (median 2,400, p95 about 18,000, clipped to
    [16, 32768]); a pool of 1.25x the blocks needed, handed out from a seeded
    shuffle in sequence order.  tp > 1: one GPU's share of the layer split by
    KV head over tp GPUs (64 / tp query heads, 8 / tp KV heads, the same
    sequences and tables)."""
    if tp not in (1, 2, 4, 8):
        raise ValueError("tp must divide the 8 KV heads")
    rng = np.random.default_rng(seed)
    lens = lognormal_lengths(rng, num_seqs)
    need = int(sum(-(-int(L) // block_size) for L in lens))
    nb = _pool_size(need)
    bt = _tables_from_pool(lens, block_size, rng.permutation(nb))
    return Workload(name, 64 // tp, 8 // tp, 128, block_size, nb, lens, bt,
                    _slots_for_last_token(lens, bt, block_size), 1.0 / math.sqrt(128),
                    kv_dtype=kv_dtype, num_layers=num_layers, seed=seed)


def llama70b_tp_shard(tp, seed=2):
    """One GPU's share of the 70B layer bs=64 under tensor parallelism over
    tp GPUs: KV heads 8 / tp, query heads 64 / tp, same lengths and tables."""
    return llama70b_layer(seed=seed, name=f"llama70b_tp{tp}_shard_bs64", tp=tp)


def prefix_shared(seed=3, num_seqs=256, block_size=32, system_tokens=900, num_pools=12,
                  pool_range=(2000, 8000), suffix_median=600.0, pool_share=0.62,
                  max_len=32768, num_q_heads=64, num_kv_heads=8, head_dim=128, kv_dtype="bf16"):
    """Prefix-shared batch on the 70B layer shape, block_size 32.

    Every sequence starts with the same 900-token system prompt; then one of
    12 shared prefix pools (lengths uniform in [2000, 8000], one pool picked
    uniformly per sequence); then a unique suffix.  Suffix lengths are
    lognormal with median 600 at stratified quantiles u = (perm + 0.5) / S;
    their spread sigma is set by bisection so that pool tokens are 62% of all
    non-system tokens.  Blocks are assigned by full-block prefix keys
    (``PrefixBlockCache``), so a block is shared exactly when all tokens up to
    its end are identical; block tables then name shared physical blocks."""
    rng = np.random.default_rng(seed)
    pool_lens = rng.integers(pool_range[0], pool_range[1] + 1, size=num_pools)
    choice = rng.integers(0, num_pools, size=num_seqs)
    u = (rng.permutation(num_seqs) + 0.5) / num_seqs
    z = np.array([NormalDist().inv_cdf(float(x)) for x in u])
    P = pool_lens[choice].astype(np.int64)
    cap = max_len - system_tokens - P

    def suffixes(sigma):
        return np.clip(np.rint(suffix_median * np.exp(sigma * z)), 1, cap).astype(np.int64)

    def share(sigma):
        return P.sum() / (P.sum() + suffixes(sigma).sum())

    lo, hi = 0.0, 6.0
    for _ in range(100):
        mid = 0.5 * (lo + hi)
        if share(mid) > pool_share:
            lo = mid
        else:
            hi = mid
    sigma = 0.5 * (lo + hi)
    suf = suffixes(sigma)
    lens = (system_tokens + P + suf).astype(np.int32)

    # Token ids: shared system prompt, per-pool prompt, per-sequence suffix.
    system = list(range(1, system_tokens + 1))
    pools = [list(range(10_000_000 * (p + 1), 10_000_000 * (p + 1) + int(pool_lens[p])))
             for p in range(num_pools)]
    need_upper = int(sum(-(-int(L) // block_size) for L in lens))
    # Allocate from a big id space first, then shrink to a 1.25x pool.
    fl = FreeList(range(need_upper))
    cache = PrefixBlockCache(fl)
    tables = []
    for s in range(num_seqs):
        toks = system + pools[choice[s]] + \
            list(range(2_000_000_000 + s * 100_000, 2_000_000_000 + s * 100_000 + int(suf[s])))
        tables.append(cache.blocks_for(toks, block_size))
    used = sorted(set(b for t in tables for b in t))
    nb = _pool_size(len(used))
    relabel = dict(zip(used, rng.permutation(nb)[:len(used)].tolist()))
    maxb = max(len(t) for t in tables)
    bt = np.full((num_seqs, maxb), -1, dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = [relabel[b] for b in t]
    w = Workload("prefix_shared_bs256", num_q_heads, num_kv_heads, head_dim, block_size, nb, lens, bt,
                 _slots_for_last_token(lens, bt, block_size), 1.0 / math.sqrt(head_dim), kv_dtype=kv_dtype,
                 seed=seed)
    w.notes = {"suffix_sigma": float(sigma), "pool_share": float(share(sigma)),
               "prefix_hits": cache.hits, "prefix_misses": cache.misses}
    return w


def long_context(seed=4, num_seqs=4, seq_len=131072, block_size=16, boost=0.01):
    """Long-context split-K decode: 4 sequences of 131,072 tokens on the 70B
    layer shape, block_size 16, block tables from a seeded permutation of a
    pool of 1.25x the blocks needed; 1% of K rows scaled by 8."""
    rng = np.random.default_rng(seed)
    lens = np.full(num_seqs, seq_len, dtype=np.int32)
    need = num_seqs * (-(-seq_len // block_size))
    nb = _pool_size(need)
    bt = _tables_from_pool(lens, block_size, rng.permutation(nb))
    return Workload("long_context_128k", 64, 8, 128, block_size, nb, lens, bt,
                    _slots_for_last_token(lens, bt, block_size), 1.0 / math.sqrt(128),
                    seed=seed, k_row_boost=boost)


def fp8_80_layers(seed=5, num_seqs=128, num_layers=80):
    """Full 80-layer fp8 decode step: the 70B layer shape with an e4m3fn KV
    cache and per-layer K and V scales, 128 sequences with lognormal lengths,
    block_size 16, one block table shared by all layers."""
    return llama70b_layer(seed=seed, num_seqs=num_seqs, block_size=16, kv_dtype="fp8",
                          num_layers=num_layers, name="fp8_80layer_bs128")


def random_workload(seed, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    max_len, kv_dtype="bf16", min_len=0, extra_blocks=3, lens=None):
    """Small random workload for parity sweeps: uniform lengths in
    [min_len, max_len] (or the given ones), tables from a seeded shuffle."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(min_len, max_len + 1, size=num_seqs).astype(np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    need = int(sum(-(-int(L) // block_size) for L in lens))
    nb = need + extra_blocks
    bt = _tables_from_pool(lens, block_size, rng.permutation(nb))
    return Workload(f"random_{seed}", num_q_heads, num_kv_heads, head_dim, block_size, nb,
                    lens, bt, _slots_for_last_token(lens, bt, block_size),
                    1.0 / math.sqrt(head_dim), kv_dtype=kv_dtype, seed=seed)


CONFIGS = {
    1: tiny,
    2: llama70b_layer,
    3: prefix_shared,
    4: long_context,
    5: fp8_80_layers,
}


def config(i, **kw):
    """Workload i of the five (1 tiny, 2 70B layer bs=64, 3 prefix-shared
    bs=256, 4 long context, 5 fp8 80 layers), seeded with its number."""
    return CONFIGS[i](**kw)
