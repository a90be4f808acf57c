"""CPU oracle for paged-attention decode over a block-table KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP kernels, their headers or the Python binding, and it imports neither.

Everything here is plain numpy in float64 (the fp8 codec works on exact bit
patterns), written so that each function can be checked against the pages by
eye:

* ``oracle.pages``  - the pages' own arithmetic (per-token bytes, GQA head
  mapping, pool capacity, the symmetric max-abs quantizer).
* ``oracle.e4m3``   - OCP fp8 e4m3fn encode (round-to-nearest-even,
  saturating) and decode.
* ``oracle.paged``  - the cache layout, slot scatter, block-table gather and
  softmax attention per query head, plus a textbook contiguous attention used
  only to cross-check the gather, and a log-sum-exp merge used only in a
  self-test.
* ``oracle.blocks`` - the block manager's rules (FIFO free list, reference
  counts, full-prefix keys with a model key, fork, copy-on-write) and the
  whole-block copy, and swaps to host memory and back.
* ``oracle.cascade`` - the shared-prefix segments of a batch (maximal runs of
  full blocks held by the same set of sequences) and decode by parts merged
  by log-sum-exp.
* ``oracle.quest``  - query-aware page selection: per-block min/max key
  summaries (recomputed, or kept by the cache writes), page scores, the
  top-budget choice, and attention over the chosen pages.

Every function is pinned by a ``-m "not gpu"`` test in ``tests/`` against a
value the pages print, a closed form, an invariant or brute force; none is
"parity unpinned".
"""

from . import blocks, cascade, e4m3, pages, paged, quest  # noqa: F401
