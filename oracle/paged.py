"""Paged KV cache: slot scatter, block-table gather and decode attention
(oracle side, float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the method computes, from the pages:

* A sequence's cache lives in fixed-size physical blocks of ``block_size``
  tokens; a per-sequence block table maps logical block i to a physical block,
  and token i sits at offset i % block_size of block table[i // block_size]
  (rajatmohan.com serving design, "Paging, because contiguous allocation is a
  disaster"; "Taming the token torrent", "The Block Table Logic").  A slot is
  a physical token position, block * block_size + offset.
* Decode runs one query token per sequence and does scaled dot-product
  attention over the sequence's cached keys and values, walking the block
  table ("Taming the token torrent", "The Block Table Logic" and "Custom
  PagedAttention Kernels").  Query head i reads KV head
  i // (query heads / KV heads) ("KV Cache Engineering for LLM Serving",
  section 1).  Several block tables may name the same physical block when the
  sequences share a prefix (same page, section 11; "Taming the token
  torrent", "Implementing Radix Tree Prefix Caching").

This oracle computes the plain definition: it rebuilds each sequence's
logical K and V from the block table and evaluates softmax(scale * q K^T) V
per query head in float64, with no partitioning and no online softmax.

Cache layout (the library's documented layout; the pages leave the inside of
a block open).  A block of ``block_size`` tokens (a multiple of 16) is split
into sub-blocks of 16 tokens.  With X = 16 bytes / element size (8 for bf16,
16 for fp8):

    K element (blk, h, t, d) at
        [blk][h][t // 16][d // X][t % 16][d % X]
    V element (blk, h, t, d) at
        [blk][h][t // 16][d // (16 R)][d % 16][(t % 16) // 4][(d // 16) % R][t % 4]
    with R = 16 bytes / (4 elements) / element size (R = 2 for bf16, 4 for fp8)

Both caches are flat element arrays of num_blocks * kv_heads * block_size *
head_dim elements.  ``k_offset``/``v_offset`` state the layout as index
arithmetic; ``gather`` states it again as a reshape/transpose, and a test
checks that the two agree.
"""

from dataclasses import dataclass

import numpy as np

from . import e4m3

SUB = 16  # tokens per sub-block


@dataclass(frozen=True)
class Geom:
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str = "bf16"  # "bf16" (uint16 bit patterns) or "fp8" (e4m3fn codes)

    @property
    def elem_bytes(self):
        return 2 if self.kv_dtype == "bf16" else 1

    @property
    def x(self):
        return 16 // self.elem_bytes

    @property
    def r(self):
        return 4 // self.elem_bytes

    @property
    def cache_elems(self):
        return self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim

    @property
    def np_dtype(self):
        return np.uint16 if self.kv_dtype == "bf16" else np.uint8


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def k_offset(g, blk, h, t, d):
    """Flat element offset of K element (block, kv head, token-in-block, dim)."""
    sb = g.block_size // SUB
    return (((((blk * g.num_kv_heads + h) * sb + t // SUB) * (g.head_dim // g.x)
              + d // g.x) * SUB + t % SUB) * g.x + d % g.x)


def v_offset(g, blk, h, t, d):
    """Flat element offset of V element (block, kv head, token-in-block, dim)."""
    sb = g.block_size // SUB
    r = g.r
    tile = (blk * g.num_kv_heads + h) * sb + t // SUB
    tt = t % SUB
    return (((((tile * (g.head_dim // (16 * r)) + d // (16 * r)) * 16 + d % 16) * 4 + tt // 4)
             * r + (d // 16) % r) * 4 + tt % 4)


def slot_to_block(slot, block_size):
    """Physical slot -> (physical block, offset in block).  The pages' address
    rule is block start + offset with offset = logical index % block size
    ("Taming the token torrent", "The Block Table Logic"); with block ids in
    block units a slot is block * block_size + offset."""
    return slot // block_size, slot % block_size


def cache_write(g, k_new, v_new, slot_mapping, k_cache, v_cache):
    """Scatter new tokens' K/V (already in the cache's element encoding) into
    the flat caches, in place.  k_new, v_new: [T, Hkv, D]; a negative slot
    means "skip this token"; slots at or past num_blocks * block_size are also
    skipped.  Every other cache element is left as it was."""
    T = len(slot_mapping)
    hh, dd = np.meshgrid(np.arange(g.num_kv_heads), np.arange(g.head_dim), indexing="ij")
    for j in range(T):
        slot = int(slot_mapping[j])
        if slot < 0 or slot >= g.num_blocks * g.block_size:
            continue
        blk, off = slot_to_block(slot, g.block_size)
        k_cache[k_offset(g, blk, hh, off, dd)] = k_new[j]
        v_cache[v_offset(g, blk, hh, off, dd)] = v_new[j]


def cache_write_bf16(g, k_bits, v_bits, slot_mapping, k_cache, v_cache):
    """bf16 cache write: a bit copy of each new token's K and V."""
    cache_write(g, np.asarray(k_bits, np.uint16), np.asarray(v_bits, np.uint16),
                slot_mapping, k_cache, v_cache)


def cache_write_fp8(g, k_bits, v_bits, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """fp8 cache write: each bf16 value x is stored as the e4m3fn code of
    float32(x * float32(1/scale)), rounded to nearest even and saturated
    ("KV Cache Engineering for LLM Serving", section 8: divide by the scale,
    round, clip to the largest code)."""
    kf = bf16_bits_to_f64(k_bits).astype(np.float32)
    vf = bf16_bits_to_f64(v_bits).astype(np.float32)
    cache_write(g, e4m3.quantize(kf, k_scale), e4m3.quantize(vf, v_scale),
                slot_mapping, k_cache, v_cache)


def _values(g, stored, scale):
    if g.kv_dtype == "bf16":
        return bf16_bits_to_f64(stored)
    return e4m3.dequantize(stored, scale)


def gather(g, k_cache, v_cache, block_row, seq_len, h, k_scale=1.0, v_scale=1.0):
    """Logical K and V, [seq_len, D] float64 each, of KV head h for one
    sequence, rebuilt from its block table row.  Token i comes from block
    block_row[i // block_size] at offset i % block_size."""
    nblk = -(-seq_len // g.block_size)
    if nblk == 0:
        return np.zeros((0, g.head_dim)), np.zeros((0, g.head_dim))
    sb = g.block_size // SUB
    blocks = np.asarray(block_row[:nblk], dtype=np.int64)
    r = g.r
    kc = k_cache.reshape(g.num_blocks, g.num_kv_heads, sb, g.head_dim // g.x, SUB, g.x)
    vc = v_cache.reshape(g.num_blocks, g.num_kv_heads, sb, g.head_dim // (16 * r), 16, 4, r, 4)
    kt = kc[blocks, h]                                   # [nblk, sb, D/X, 16, X]
    vt = vc[blocks, h]                                   # [nblk, sb, D/16R, d%16, t/4, (d/16)%R, t%4]
    k_tok = kt.transpose(0, 1, 3, 2, 4).reshape(nblk * g.block_size, g.head_dim)
    # -> [nblk, sb, t/4, t%4, D/16R, (d/16)%R, d%16]
    v_tok = vt.transpose(0, 1, 4, 6, 2, 5, 3).reshape(nblk * g.block_size, g.head_dim)
    return (_values(g, k_tok[:seq_len], k_scale),
            _values(g, v_tok[:seq_len], v_scale))


def softmax_attention(q, K, V, scale):
    """softmax(scale * q K^T) V for a group of query rows sharing one K/V.
    q: [G, D], K, V: [L, D] -> [G, D].  Max-subtracted softmax in float64.
    L == 0 gives zeros."""
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]))
    z = scale * (q @ K.T)                                # [G, L]
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ V


def window_positions(L, window):
    """Positions a local layer with a window of ``window`` tokens keeps (and
    attends to) once L tokens exist: the most recent ``window`` of them, all
    of them when window is 0 ("KV Cache Engineering for LLM Serving",
    section 3: each new entry removes the oldest once the window is full)."""
    if window <= 0 or L <= window:
        return list(range(L))
    return list(range(L - window, L))


def decode(g, q_bits, k_cache, v_cache, block_tables, seq_lens, scale,
           k_scale=1.0, v_scale=1.0, seqs=None, heads=None, window=0, ring=False):
    """Paged decode: out[s, i, :] = softmax(scale * q[s, i] K_s^T) V_s with
    K_s, V_s gathered for KV head i // (Hq / Hkv); with a window, K_s and V_s
    are the rows of ``window_positions(L, window)`` only.

    q_bits: [S, Hq, D] bf16 bit patterns.  Returns float64 [S, Hq, D]; when
    ``seqs`` (and optionally ``heads``, a list of KV heads) restrict the work,
    rows that were not computed are NaN.  Only the blocks holding a kept
    position are looked up.  With ``ring`` each table row is a ring of
    len(row) entries (a local layer that keeps only its window, section 3 of
    "KV Cache Engineering for LLM Serving"): logical block b of the sequence
    is row[b % len(row)]."""
    q = bf16_bits_to_f64(q_bits)
    S, Hq, D = q.shape
    G = Hq // g.num_kv_heads
    bs = g.block_size
    out = np.full((S, Hq, D), np.nan)
    seqs = range(S) if seqs is None else seqs
    heads = range(g.num_kv_heads) if heads is None else heads
    for s in seqs:
        L = max(int(seq_lens[s]), 0)
        keep = np.asarray(window_positions(L, window), dtype=np.int64)
        first_block = int(keep[0]) // bs if keep.size else 0
        row = np.asarray(block_tables[s])
        logical = np.arange(first_block, -(-L // bs))
        span = row[logical % row.size] if ring else row[logical]
        base = first_block * bs
        for h in heads:
            K, V = gather(g, k_cache, v_cache, span, L - base, h, k_scale, v_scale)
            out[s, h * G:(h + 1) * G] = softmax_attention(q[s, h * G:(h + 1) * G], K[keep - base],
                                                          V[keep - base], scale)
    return out


def dense_attention(q, K, V, scale):
    """Textbook attention over a contiguous cache, one query head at a time
    (the contiguous-buffer layout the pages start from), used only to
    cross-check the paged gather.  q: [Hq, D]; K, V: [L, Hkv, D]."""
    Hq = q.shape[0]
    Hkv = K.shape[1]
    out = np.zeros((Hq, V.shape[2]))
    for i in range(Hq):
        h = i * Hkv // Hq
        logits = np.array([scale * np.dot(q[i], K[t, h]) for t in range(K.shape[0])])
        if logits.size == 0:
            continue
        w = np.exp(logits - logits.max())
        out[i] = (w[:, None] * V[:, h]).sum(axis=0) / w.sum()
    return out


def partial_state(q, K, V, scale):
    """Un-normalised softmax state of one token range: (m, l, acc) with
    m = max logit, l = sum exp(logit - m), acc = sum exp(logit - m) V."""
    z = scale * (q @ K.T)
    m = z.max(axis=1)
    w = np.exp(z - m[:, None])
    return m, w.sum(axis=1), w @ V


def lse_merge(states):
    """Merge partial states of disjoint token ranges: with M = max m_p,
    out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p (Milakov and
    Gimelshein's online normaliser).  Used only in an oracle self-test."""
    M = np.max([m for m, _, _ in states], axis=0)
    num = sum(np.exp(m - M)[:, None] * acc for m, _, acc in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den[:, None]
