"""Query-aware page selection (Quest) over the paged cache (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the method computes, from "KV Cache Engineering for LLM Serving",
section 7 (Query-aware sparse reads), with its four-page example:

* The cache is divided into pages, each a small run of neighbouring tokens.
* Every page keeps, per key dimension, the minimum and the maximum of the keys
  it holds.
* For a new query q, a page's score is sum over d of max(q_d * min_d,
  q_d * max_d): the largest q.k that any key inside the page's min/max box
  could reach, so it bounds every real key of the page from above.
* Only the pages with the highest scores are read; attention runs over their
  tokens.  Nothing is deleted: a page skipped now can be chosen later.

Readings where the page is silent (each is listed in the design notes):

* Q1  A page is one cache block (block_size tokens); the last page of a
      sequence holds its L % block_size trailing tokens (or a full block).
* Q2  Grouped-query heads share a KV head, and its K/V are read once for the
      whole group, so pages are chosen per (sequence, KV head).  A page's
      score for the group is the largest of its query heads' scores: it is
      read if any head of the group ranks it high.
* Q3  The choice of pages is an integer decision taken from a floating-point
      score, so both sides compute the score the same way: float32 products,
      float32 sums in dimension order d = 0, 1, ..., D - 1, then the maximum
      over the group.  A product of two bf16 values is exact in float32
      whenever its magnitude is at least 2^-134, so any float32 evaluation
      that rounds once per added term (a fused multiply-add included) gives
      the same sums.  No scale is applied: a positive softmax scale does not
      change the ranking.
* Q4  The ``budget`` pages with the highest scores are chosen; equal scores
      go to the lower page index.  A budget at least the page count chooses
      every page, which is plain decode.  The selected pages are read in
      ascending order.
* Q5  The summaries hold the values the cache stores: bf16 keys as they are,
      fp8 keys as their e4m3 code values without the per-tensor scale (a
      positive scale does not change min, max or ranking).  Summary values
      are therefore exact in bf16.
* Q6  Summaries are kept current by the cache writes: a token written at
      offset 0 of a block starts that block's summary afresh, and every
      written token's key is merged in.  Blocks filled another way (a copy,
      a swap-in) get their summary recomputed from their first ``count``
      tokens.  NaN keys are ignored by the summaries.
"""

import numpy as np

from . import e4m3, paged


def stored_values(g, stored):
    """Cache elements -> float64 values as stored: bf16 values, or e4m3 code
    values without the scale (Q5)."""
    if g.kv_dtype == "bf16":
        return paged.bf16_bits_to_f64(stored)
    return e4m3.decode(np.asarray(stored, np.uint8))


def empty_summaries(g):
    """Summary state of a pool with nothing written: min +inf, max -inf,
    shape [num_blocks, Hkv, D] each."""
    shape = (g.num_blocks, g.num_kv_heads, g.head_dim)
    return np.full(shape, np.inf), np.full(shape, -np.inf)


def _token_keys(g, k_cache, blk, t):
    """Stored key values [Hkv, D] of token t of block blk."""
    hh, dd = np.meshgrid(np.arange(g.num_kv_heads), np.arange(g.head_dim), indexing="ij")
    return stored_values(g, k_cache[paged.k_offset(g, blk, hh, t, dd)])


def block_summary(g, k_cache, blk, count):
    """(min, max), [Hkv, D] each, over the keys of tokens 0 .. count-1 of
    block blk; +inf / -inf when count is 0.  NaN keys are skipped."""
    mn = np.full((g.num_kv_heads, g.head_dim), np.inf)
    mx = np.full((g.num_kv_heads, g.head_dim), -np.inf)
    for t in range(count):
        k = _token_keys(g, k_cache, blk, t)
        mn = np.fmin(mn, k)
        mx = np.fmax(mx, k)
    return mn, mx


def summarize(g, k_cache, blocks, counts, mn, mx):
    """Recompute, in place, the summaries of blocks[i] from their first
    counts[i] tokens (Q6: blocks filled by a copy or a swap-in)."""
    for b, c in zip(blocks, counts):
        mn[b], mx[b] = block_summary(g, k_cache, int(b), int(c))


def update_summaries(g, k_cache, slot_mapping, mn, mx):
    """The write-maintained summaries (Q6), in place, after a cache write of
    ``slot_mapping`` has landed in ``k_cache``: every block with a token
    written at offset 0 starts empty, then each written token's stored key
    is merged in.  Slots that are negative or past the pool are skipped."""
    nslots = g.num_blocks * g.block_size
    valid = [int(s) for s in slot_mapping if 0 <= int(s) < nslots]
    for s in valid:
        blk, off = paged.slot_to_block(s, g.block_size)
        if off == 0:
            mn[blk] = np.inf
            mx[blk] = -np.inf
    for s in valid:
        blk, off = paged.slot_to_block(s, g.block_size)
        k = _token_keys(g, k_cache, blk, off)
        mn[blk] = np.fmin(mn[blk], k)
        mx[blk] = np.fmax(mx[blk], k)


def sequence_page_summaries(g, k_cache, block_row, L, h):
    """(min, max), [pages, D] each, of KV head h over the pages of one
    sequence of length L: page p covers positions p * block_size up to
    min(L, (p + 1) * block_size).  The same values as ``block_summary`` of
    each block with its count of tokens, taken here from the gathered
    sequence (for long sequences)."""
    K, _ = paged.gather(g, k_cache, k_cache, block_row, L, h, 1.0, 1.0)   # stored values (Q5)
    pages = -(-L // g.block_size)
    pad = pages * g.block_size - L
    lo = np.concatenate([K, np.full((pad, g.head_dim), np.inf)]).reshape(pages, g.block_size, g.head_dim)
    hi = np.concatenate([K, np.full((pad, g.head_dim), -np.inf)]).reshape(pages, g.block_size, g.head_dim)
    return np.fmin.reduce(lo, axis=1), np.fmax.reduce(hi, axis=1)


def page_scores(q_group, mn, mx):
    """Scores of n pages for one group of query heads (Q2, Q3).

    q_group: [G, D] float32 query rows; mn, mx: [n, D] page summaries.
    For each page and head g: s = sum over d, in order, of
    max(q[g, d] * mn[d], q[g, d] * mx[d]) in float32; the page's score is
    the largest s over the group.  Returns float32 [n]."""
    q = np.asarray(q_group, np.float32)
    lo = np.asarray(mn, np.float32)
    hi = np.asarray(mx, np.float32)
    n, D = lo.shape
    G = q.shape[0]
    acc = np.zeros((n, G), np.float32)
    for d in range(D):
        term = np.maximum(lo[:, d:d + 1] * q[None, :, d], hi[:, d:d + 1] * q[None, :, d])
        acc = (acc + term).astype(np.float32)
    return acc.max(axis=1)


def select_pages(scores, budget):
    """Indices of the ``budget`` highest scores, equal scores to the lower
    index, returned in ascending order (Q4); all indices when budget is at
    least their number."""
    n = len(scores)
    if budget >= n:
        return list(range(n))
    order = sorted(range(n), key=lambda i: (-float(scores[i]), i))
    return sorted(order[:budget])


def selection(g, q_bits, mn, mx, block_tables, seq_lens, budget):
    """Chosen page indices per (sequence, KV head): a list of S lists of Hkv
    lists.  mn, mx: the pool's summary state [num_blocks, Hkv, D]."""
    q = paged.bf16_bits_to_f64(q_bits).astype(np.float32)
    S, Hq, _ = q.shape
    G = Hq // g.num_kv_heads
    out = []
    for s in range(S):
        L = max(int(seq_lens[s]), 0)
        pages = -(-L // g.block_size)
        blocks = np.asarray(block_tables[s][:pages], dtype=np.int64)
        row = []
        for h in range(g.num_kv_heads):
            if pages == 0:
                row.append([])
                continue
            sc = page_scores(q[s, h * G:(h + 1) * G], mn[blocks, h], mx[blocks, h])
            row.append(select_pages(sc, budget))
        out.append(row)
    return out


def decode(g, q_bits, k_cache, v_cache, block_tables, seq_lens, mn, mx, budget, scale,
           k_scale=1.0, v_scale=1.0, seqs=None):
    """Quest decode: for each (sequence, KV head), softmax attention of the
    group's query heads over the tokens of the chosen pages only (positions
    below L), in float64.  Returns ([S, Hq, D] float64, the selection);
    rows of sequences outside ``seqs`` are NaN."""
    q = paged.bf16_bits_to_f64(q_bits)
    S, Hq, D = q.shape
    G = Hq // g.num_kv_heads
    chosen = selection(g, q_bits, mn, mx, block_tables, seq_lens, budget)
    out = np.full((S, Hq, D), np.nan)
    for s in (range(S) if seqs is None else seqs):
        L = max(int(seq_lens[s]), 0)
        for h in range(g.num_kv_heads):
            K, V = paged.gather(g, k_cache, v_cache, block_tables[s], L, h, k_scale, v_scale)
            pos = [p * g.block_size + t for p in chosen[s][h] for t in range(g.block_size)
                   if p * g.block_size + t < L]
            out[s, h * G:(h + 1) * G] = paged.softmax_attention(q[s, h * G:(h + 1) * G], K[pos], V[pos],
                                                                scale)
    return out, chosen
