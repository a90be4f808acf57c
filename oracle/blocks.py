"""Block manager model: free list, reference counts, prefix reuse, fork and
copy-on-write (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What a block manager does, from the pages:

* The pool is a list of free block ids.  A request takes blocks from the
  front of the list; a finished request hands its blocks back to the end, in
  the order its block table lists them, and the next request may take them
  at once ("KV Cache Engineering for LLM Serving", section 10, Paging, with
  its six-block example).
* A completed block is stored under a key made of the entire token prefix
  up to the end of that block, so a block is reused only when all preceding
  context is identical (same page, section 11, Prefix reuse; rajatmohan.com
  serving design, "Prefix sharing is where the real win lives").  The key
  also carries the model / adapter identity, since identical tokens give
  different K and V under different weights (rajatmohan.com, same section).
* A local (sliding-window) layer keeps only its most recent positions, so the
  blocks that hold nothing newer can go back to the pool ("KV Cache
  Engineering for LLM Serving", section 3): ``trim``.  Such a layer's window
  works as a ring, each new entry displacing the oldest (same section):
  ``add_ring_sequence`` gives a sequence a table of ceil(W / block_size) + 1
  entries, logical block b at entry b % entries, and a new block reuses the
  block its entry held, which has just left the window.
* Blocks a paused sequence does not need can move to host memory and come
  back when it resumes ("KV Cache Engineering for LLM Serving", section 12,
  Cache Offloading); the blocks of a shared prefix stay on the GPU ("Taming
  the token torrent", "The Swapping Mechanism"): ``swap_out`` / ``swap_in``.
* A reused block gets its reference count incremented instead of new memory;
  when one user writes tokens of its own into a block others still hold, it
  first gets a private copy: copy-on-write ("Taming the token torrent",
  "Implementing Radix Tree Prefix Caching").

This model follows those rules with plain Python containers: the key is the
tuple (model key, all tokens up to the block's end), exactly the page's
readable stand-in for chained hashes, so there are no collisions to reason
about.  Only full blocks are ever stored under a key; a sequence's partly
filled last block is private unless the sequence was forked.
"""

import numpy as np


class OutOfBlocks(Exception):
    pass


class Swapped(Exception):
    """The operation needs a resident sequence (or a swapped one)."""


SWAPPED = -2   # table entry of a block moved to host memory


class BlockManager:
    def __init__(self, num_blocks, block_size):
        self.block_size = block_size
        self.free = list(range(num_blocks))   # front = next to hand out
        self.ref = [0] * num_blocks
        self.key_block = {}                   # prefix key -> block
        self.block_key = {}                   # block -> prefix key it is stored under
        self.seqs = {}                        # seq id -> {"tokens", "table", "model", "swapped", "ring"}
        self.hits = 0
        self.misses = 0

    # -- allocation -------------------------------------------------------
    def _take(self):
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.pop(0)
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            k = self.block_key.pop(b, None)
            if k is not None and self.key_block.get(k) == b:
                del self.key_block[k]
            self.free.append(b)

    def _key(self, model, tokens, end):
        return (model, tuple(tokens[:end]))

    def _store(self, b, key):
        """Record a just-completed block under its prefix key, unless an
        equal block is already stored."""
        if key not in self.key_block:
            self.key_block[key] = b
            self.block_key[b] = key

    # -- operations ---------------------------------------------------------
    def add_sequence(self, seq, tokens, model=0):
        """A new request with prompt ``tokens``: every full block whose key
        is stored is reused, every other block is taken from the free list.
        Returns the number of reused blocks.  When the pool cannot supply
        the new blocks nothing changes and OutOfBlocks is raised."""
        if seq in self.seqs:
            raise KeyError(seq)
        bs = self.block_size
        full = len(tokens) // bs
        keys = [self._key(model, tokens, (i + 1) * bs) for i in range(full)]
        need = sum(k not in self.key_block for k in keys) + (1 if len(tokens) % bs else 0)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        table, reused = [], 0
        for key in keys:
            b = self.key_block.get(key)
            if b is not None:
                self.ref[b] += 1
                reused += 1
            else:
                b = self._take()
                self._store(b, key)
            table.append(b)
        if len(tokens) % bs:
            table.append(self._take())
        self.hits += reused
        self.misses += len(table) - reused
        self.seqs[seq] = {"tokens": list(tokens), "table": table, "model": model, "swapped": False, "ring": 0}
        return reused

    def add_ring_sequence(self, seq, n, window):
        """A local layer's sequence of n tokens whose table is a ring of
        E = ceil(window / block_size) + 1 entries: logical block b lives at
        entry b % E, so the blocks of any ``window`` consecutive positions
        have distinct entries.  Blocks are taken for the last min(blocks, E)
        logical blocks of the n tokens; other entries are -1.  No prefix
        keys: a ring block is rewritten as the window moves.  Returns E."""
        if seq in self.seqs:
            raise KeyError(seq)
        if window < 1:
            raise ValueError("window must be >= 1")
        bs = self.block_size
        E = -(-window // bs) + 1
        nb = -(-n // bs)
        held = min(nb, E)
        if held > len(self.free):
            raise OutOfBlocks(f"need {held} blocks, {len(self.free)} free")
        table = [-1] * E
        for b in range(nb - held, nb):
            table[b % E] = self._take()
        self.misses += held
        self.seqs[seq] = {"tokens": [0] * n, "table": table, "model": None, "swapped": False, "ring": E}
        return E

    def fork(self, parent, child):
        """``child`` shares every block of ``parent``, partial last block
        included."""
        if child in self.seqs:
            raise KeyError(child)
        p = self.seqs[parent]
        if p["swapped"]:
            raise Swapped(parent)
        for b in p["table"]:
            if b >= 0:
                self.ref[b] += 1
        self.seqs[child] = {"tokens": list(p["tokens"]), "table": list(p["table"]),
                            "model": p["model"], "swapped": False, "ring": p["ring"]}

    def append_token(self, seq, token):
        """One generated token.  Returns (slot, copy_src, copy_dst): the slot
        the token's K/V go to, and the block copy that must happen first
        (-1, -1 when none)."""
        s = self.seqs[seq]
        if s["swapped"]:
            raise Swapped(seq)
        bs = self.block_size
        pos = len(s["tokens"])
        src = dst = -1
        if s["ring"]:
            return self._append_ring(s, pos, token)
        if (pos % bs == 0 or self.ref[s["table"][-1]] > 1) and not self.free:
            raise OutOfBlocks("no free block")
        if pos % bs == 0:
            s["table"].append(self._take())
        else:
            last = s["table"][-1]
            if self.ref[last] > 1:
                dst = self._take()
                src = last
                self.ref[last] -= 1
                s["table"][-1] = dst
        s["tokens"].append(token)
        blk = s["table"][pos // bs]
        if (pos + 1) % bs == 0:
            self._store(blk, self._key(s["model"], s["tokens"], pos + 1))
        return blk * bs + pos % bs, src, dst

    def _append_ring(self, s, pos, token):
        """append_token on a ring table.  The new position's entry is
        e = (pos // block_size) % E.  Starting a block: the entry's old block
        has left the window, so it is written over in place if this
        sequence alone holds it; if a fork still shares it, or the entry is
        empty, a fresh block is taken (the shared one loses a reference).
        Inside a block: a shared block is copied first (copy-on-write)."""
        bs = self.block_size
        e = (pos // bs) % s["ring"]
        old = s["table"][e]
        fresh = old < 0 or (pos % bs == 0 and self.ref[old] > 1)
        copy = not fresh and pos % bs != 0 and self.ref[old] > 1
        if (fresh or copy) and not self.free:
            raise OutOfBlocks("no free block")
        src = dst = -1
        if fresh:
            if old >= 0:
                self._release(old)
            s["table"][e] = self._take()
        elif copy:
            src, dst = old, self._take()
            self.ref[old] -= 1
            s["table"][e] = dst
        s["tokens"].append(token)
        return s["table"][e] * bs + pos % bs, src, dst

    def slots(self, seq, first, count):
        """Slots of positions first .. first + count - 1 (block * block_size
        + offset), -1 where no table entry holds the position's block any
        more (released by a trim, or a ring entry that has moved on)."""
        s = self.seqs[seq]
        if s["swapped"]:
            raise Swapped(seq)
        n = len(s["tokens"])
        if first < 0 or count < 0 or first + count > n:
            raise ValueError("positions outside the sequence")
        bs = self.block_size
        nb = -(-n // bs)
        out = []
        for pos in range(first, first + count):
            b = pos // bs
            if s["ring"]:
                blk = s["table"][b % s["ring"]] if b >= nb - s["ring"] else -1
            else:
                blk = s["table"][b]
            out.append(blk * bs + pos % bs if blk >= 0 else -1)
        return out

    def trim(self, seq, keep):
        """Sliding window: release the blocks of ``seq`` that hold only
        positions before its last ``keep`` tokens (keep >= 1); their table
        entries become -1 and later positions keep their logical blocks.
        Returns the number of entries released."""
        if keep < 1:
            raise ValueError("keep must be >= 1")
        s = self.seqs[seq]
        if s["swapped"]:
            raise Swapped(seq)
        bs = self.block_size
        first = max(len(s["tokens"]) - keep, 0) // bs   # first block with a kept position
        E = s["ring"]
        start = max(-(-len(s["tokens"]) // bs) - E, 0) if E else 0   # oldest block a ring still lists
        n = 0
        for b in range(start, first):
            i = b % E if E else b
            if s["table"][i] >= 0:
                self._release(s["table"][i])
                s["table"][i] = -1
                n += 1
        return n

    def swap_out(self, seq):
        """Release the blocks only ``seq`` holds, in table order, marking
        their entries SWAPPED; returns those blocks (the ones to copy out)."""
        s = self.seqs[seq]
        if s["swapped"]:
            raise Swapped(seq)
        out = []
        for i, b in enumerate(s["table"]):
            if b >= 0 and self.ref[b] == 1:
                out.append(b)
                self._release(b)
                s["table"][i] = SWAPPED
        s["swapped"] = True
        return out

    def swap_in(self, seq):
        """Give every SWAPPED entry a block from the free list, in table
        order; a full block goes back under its prefix key unless an equal
        block is stored.  Returns the new blocks in that order."""
        s = self.seqs[seq]
        if not s["swapped"]:
            raise Swapped(seq)
        idx = [i for i, b in enumerate(s["table"]) if b == SWAPPED]
        if len(idx) > len(self.free):
            raise OutOfBlocks(f"need {len(idx)} blocks, {len(self.free)} free")
        bs = self.block_size
        out = []
        for i in idx:
            b = self._take()
            s["table"][i] = b
            out.append(b)
            if not s["ring"] and (i + 1) * bs <= len(s["tokens"]):
                self._store(b, self._key(s["model"], s["tokens"], (i + 1) * bs))
        s["swapped"] = False
        return out

    def free_sequence(self, seq):
        s = self.seqs.pop(seq)
        for b in s["table"]:
            if b >= 0:
                self._release(b)

    # -- queries ----------------------------------------------------------
    def table(self, seq):
        return list(self.seqs[seq]["table"])

    def length(self, seq):
        return len(self.seqs[seq]["tokens"])

    def num_free(self):
        return len(self.free)


def copy_blocks(k_cache, v_cache, pairs, block_elems):
    """Copy whole blocks (every KV head, K and V) from src to dst for each
    (src, dst) pair, in order, on flat caches whose blocks are contiguous
    runs of ``block_elems`` elements."""
    for src, dst in pairs:
        for c in (k_cache, v_cache):
            c[dst * block_elems:(dst + 1) * block_elems] = c[src * block_elems:(src + 1) * block_elems]


def swap_image(k_cache, v_cache, blocks, block_elems):
    """The host copy of a swap-out: the K blocks named by ``blocks``, in list
    order, followed by the V blocks in the same order."""
    return np.concatenate([c[b * block_elems:(b + 1) * block_elems] for c in (k_cache, v_cache)
                           for b in blocks] or [k_cache[:0]])


def swap_restore(k_cache, v_cache, blocks, image, block_elems):
    """The swap-in of a host copy: its i-th K and V blocks become block
    blocks[i] of each cache."""
    n = len(blocks)
    for i, b in enumerate(blocks):
        k_cache[b * block_elems:(b + 1) * block_elems] = image[i * block_elems:(i + 1) * block_elems]
        v_cache[b * block_elems:(b + 1) * block_elems] = image[(n + i) * block_elems:(n + i + 1) * block_elems]
