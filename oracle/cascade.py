"""Shared-prefix (cascade) decomposition of a batch's decode (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sequences whose prompts start alike hold the same physical blocks for that
prefix ("Taming the token torrent", "Implementing Radix Tree Prefix
Caching": a new user's block table points at the existing blocks;
"KV Cache Engineering for LLM Serving", section 11; rajatmohan.com serving
design, "Prefix sharing is where the real win lives").  Attention over a
sequence's tokens can be split at any token boundary into parts whose
partial softmax states are merged by log-sum-exp (Milakov and Gimelshein's
online normaliser), so the tokens of a shared prefix can be attended to for
all of the sequences that hold it in one pass over its blocks.

This module states, plainly:

* ``shared_segments``: the shared parts of a batch.  The full blocks of each
  sequence form a path of block ids; sequences whose tables agree on
  positions 0..j share position j.  A segment is a maximal run of positions
  shared by one and the same set of at least ``min_members`` sequences.
  Each sequence's private part starts after its last shared position.
* ``decode``: attention computed as one partial state per (segment, member)
  and one for each sequence's private part, merged per sequence; the result
  equals plain decode (a test pins it to ``paged.decode``).

Readings: only full blocks are shared (a sequence's partly filled last block
is its own); a segment needs at least two member sequences (a run held by
one sequence is private); block ids are compared as given, so two tables
share a position only if they agree on every position before it too; a
length outside [0, table width * block_size] is invalid and shares nothing.
"""

import numpy as np

from . import paged


def shared_segments(block_tables, seq_lens, block_size, min_members=2):
    """Segments of shared full blocks.

    Returns (segments, prefix_tokens): segments is a list of dicts
    {"first": first logical block, "blocks": [block ids], "members": [seqs]}
    and prefix_tokens[s] is the number of tokens of sequence s covered by
    segments (a multiple of block_size)."""
    S = len(seq_lens)
    full = [int(seq_lens[s]) // block_size if 0 <= int(seq_lens[s]) <= len(block_tables[s]) * block_size
            else 0 for s in range(S)]
    segments = []
    prefix = [0] * S

    def walk(members, j):
        # members agree on positions 0..j-1; split them by their block at j
        groups = {}
        for s in members:
            if j < full[s]:
                groups.setdefault(int(block_tables[s][j]), []).append(s)
        for blk in sorted(groups):
            g = groups[blk]
            if len(g) < min_members:
                continue
            # extend the run while the same members agree
            k = j + 1
            while all(k < full[s] for s in g) and len({int(block_tables[s][k]) for s in g}) == 1:
                k += 1
            segments.append({"first": j, "blocks": [int(block_tables[g[0]][i]) for i in range(j, k)],
                             "members": list(g)})
            for s in g:
                prefix[s] = k * block_size
            walk(g, k)

    walk(list(range(S)), 0)
    return segments, prefix


def decode(g, q_bits, k_cache, v_cache, block_tables, seq_lens, scale, k_scale=1.0, v_scale=1.0,
           min_members=2):
    """Decode by parts: per sequence s and KV head h, the partial softmax
    states (m, l, acc) of the group's query heads over the tokens of each
    segment s belongs to, and over its private tokens, merged by
    log-sum-exp.  Returns [S, Hq, D] float64."""
    q = paged.bf16_bits_to_f64(q_bits)
    S, Hq, D = q.shape
    G = Hq // g.num_kv_heads
    BS = g.block_size
    segments, prefix = shared_segments(block_tables, seq_lens, BS, min_members)
    member_of = [[] for _ in range(S)]
    for seg in segments:
        for s in seg["members"]:
            member_of[s].append(seg)
    out = np.zeros((S, Hq, D))
    for s in range(S):
        L = max(int(seq_lens[s]), 0)
        for h in range(g.num_kv_heads):
            qg = q[s, h * G:(h + 1) * G]
            states = []
            for seg in member_of[s]:
                n = len(seg["blocks"]) * BS
                K, V = paged.gather(g, k_cache, v_cache, seg["blocks"], n, h, k_scale, v_scale)
                states.append(paged.partial_state(qg, K, V, scale))
            K, V = paged.gather(g, k_cache, v_cache, block_tables[s], L, h, k_scale, v_scale)
            if L > prefix[s]:
                states.append(paged.partial_state(qg, K[prefix[s]:L], V[prefix[s]:L], scale))
            if states:
                out[s, h * G:(h + 1) * G] = paged.lse_merge(states)
    return out
