"""A whole decode step over a stack of layers, eager or as one HIP graph.

Per layer the step writes this step's new K/V into the layer's cache
(``pa_cache_write`` or ``pa_cache_write_fp8``) and then decodes every
sequence against it (``pa_decode`` or ``pa_decode_fp8``), so a step over n
layers is 2n kernel launches; with ``fused=True`` each layer is one
``pa_decode_append`` (or ``_fp8``) launch that does both, n launches in all,
with the same caches and outputs.  The write and decode of one layer are
latency bound at small batches, so ``capture()`` records the launches once
into a HIP graph (torch's ``CUDAGraph``, which is hipGraph on ROCm) and
``replay()`` submits them with one call.  The library's kernels allocate
nothing and issue no memset, and the decode returns its workspace counters
to zero itself, so replaying the graph needs no host-side work between
steps.

All layers share one block table, one set of sequence lengths and one slot
mapping (the pages' block table maps a sequence's logical blocks to physical
blocks of the pool; every layer's cache uses the same mapping).
"""

import torch

from . import (alloc_workspace, pa_cache_write, pa_cache_write_fp8, pa_decode,
               pa_decode_append, pa_decode_append_fp8, pa_decode_fp8)


class DecodeStep:
    """Cache write + decode for layers 0..n-1 of stacked per-layer tensors.

    q        [n, S, Hq, D] bf16          k_new, v_new  [n, S, Hkv, D] bf16
    k_cache, v_cache  [n, elems] bf16 (or uint8 e4m3fn codes with ``k_scale``
             and ``v_scale``: n per-layer float scales)
    out      [n, S, Hq, D] float32
    block_tables [S, max_blocks] int32, seq_lens [S] int32, slot_mapping [S] int64
    (the slot of each sequence's new token, position seq_lens[s] - 1; the
    fused step derives it from the tables and does not read slot_mapping)
    """

    def __init__(self, *, q, k_new, v_new, k_cache, v_cache, out, block_tables, seq_lens,
                 slot_mapping, scale, num_kv_heads, block_size, k_scale=None, v_scale=None,
                 partition_tokens=0, workspace=None, fused=False):
        self.n = q.shape[0]
        self.fused = bool(fused)
        self.fp8 = k_cache.dtype == torch.uint8
        if self.fp8 and (k_scale is None or v_scale is None):
            raise ValueError("an fp8 cache needs per-layer k_scale and v_scale")
        for name, x in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                        ("v_cache", v_cache), ("out", out)):
            if x.shape[0] != self.n:
                raise ValueError(f"{name} has {x.shape[0]} layers, q has {self.n}")
        self.q, self.k_new, self.v_new = q, k_new, v_new
        self.k_cache, self.v_cache, self.out = k_cache, v_cache, out
        self.block_tables, self.seq_lens, self.slot_mapping = block_tables, seq_lens, slot_mapping
        self.scale = float(scale)
        self.num_kv_heads, self.block_size = num_kv_heads, block_size
        self.k_scale = [float(x) for x in k_scale] if self.fp8 else None
        self.v_scale = [float(x) for x in v_scale] if self.fp8 else None
        self.partition_tokens = partition_tokens
        S, Hq, D = q.shape[1:]
        if workspace is None:
            elems = k_cache.shape[1]
            nb = elems // (num_kv_heads * block_size * D)
            workspace = alloc_workspace(nb, block_size, num_kv_heads, D, S, Hq,
                                        block_tables.shape[1], partition_tokens, q.device)
        self.workspace = workspace
        self.graph = None

    def write(self, i):
        if self.fp8:
            pa_cache_write_fp8(self.k_new[i], self.v_new[i], self.slot_mapping, self.k_cache[i],
                               self.v_cache[i], self.k_scale[i], self.v_scale[i],
                               block_size=self.block_size)
        else:
            pa_cache_write(self.k_new[i], self.v_new[i], self.slot_mapping, self.k_cache[i],
                           self.v_cache[i], block_size=self.block_size)

    def decode(self, i):
        if self.fp8:
            pa_decode_fp8(self.q[i], self.k_cache[i], self.v_cache[i], self.block_tables,
                          self.seq_lens, self.scale, self.k_scale[i], self.v_scale[i], self.out[i],
                          num_kv_heads=self.num_kv_heads, block_size=self.block_size,
                          partition_tokens=self.partition_tokens, workspace=self.workspace)
        else:
            pa_decode(self.q[i], self.k_cache[i], self.v_cache[i], self.block_tables,
                      self.seq_lens, self.scale, self.out[i], num_kv_heads=self.num_kv_heads,
                      block_size=self.block_size, partition_tokens=self.partition_tokens,
                      workspace=self.workspace)

    def append_decode(self, i):
        """Layer i's write and decode as one fused launch."""
        args = (self.q[i], self.k_new[i], self.v_new[i], self.k_cache[i], self.v_cache[i],
                self.block_tables, self.seq_lens, self.scale)
        kw = dict(num_kv_heads=self.num_kv_heads, block_size=self.block_size,
                  partition_tokens=self.partition_tokens, workspace=self.workspace)
        if self.fp8:
            pa_decode_append_fp8(*args, self.k_scale[i], self.v_scale[i], self.out[i], **kw)
        else:
            pa_decode_append(*args, self.out[i], **kw)

    def run(self, events=None):
        """Enqueue the step eagerly on the current stream.  With ``events``
        (a list of n + 1 timing events) an event is recorded before layer 0
        and after each layer."""
        stream = torch.cuda.current_stream(self.q.device)
        for i in range(self.n):
            if events is not None and i == 0:
                events[0].record(stream)
            if self.fused:
                self.append_decode(i)
            else:
                self.write(i)
                self.decode(i)
            if events is not None:
                events[i + 1].record(stream)

    def capture(self):
        """Record the step into a HIP graph.  Runs the step once eagerly first
        (device queries the library caches on first use must not happen
        during capture)."""
        self.run()
        torch.cuda.synchronize(self.q.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize(self.q.device)
        self.graph = g
        return g

    def replay(self):
        if self.graph is None:
            raise RuntimeError("capture() first")
        self.graph.replay()
