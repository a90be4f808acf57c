"""Benchmark: paged-attention decode on a Llama-70B-shaped layer, batch 64.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-scrub] [--skip-cpu] [--partition-tokens P]

Default workload (llama70b_layer_bs64).  One step = the whole hot path over
one batch: pa_cache_write of the 64 new tokens (one per sequence) into their
slots, then pa_decode of the 64 sequences (64 query heads, 8 KV heads,
head_dim 128, bf16 KV cache, block size 16, lognormal lengths with median
2,400 and p95 about 18,000 clipped to [16, 32768]).  Inputs are synthetic and
already resident in HBM.

Before every timed step a 512 MiB buffer is read (a reduction) so the KV
blocks of the previous step are not served from the 256 MiB Infinity Cache
(a read leaves clean lines, so the decode pays no write-back for the scrub);
the write and the decode are each bracketed by HIP events recorded on the
stream they run on, so the scrub is not timed.  `value` is KV bytes read per
decode call (sum of sequence lengths x 2 x 8 heads x 128 x 2 B) divided by
the mean event-timed duration of pa_decode, in GB/s (1e9 B/s).  `ceilings`
gives two practical read ceilings measured in the same run with the probes
of include/pa_probe.h: a plain streaming read of the 512 MiB scrub buffer,
and a read of exactly the decode's K/V tiles with no arithmetic.
`fused_append_decode` times the same step as one pa_decode_append launch (the
write folded into the decode), after the same scrub, beside the two launches.

Other workloads (--workload), each on the same 70B layer shape:
  prefix_shared_bs256  256 sequences, block 32, a shared 900-token system
                       prompt and 12 shared prefix pools; `value` counts the
                       distinct (physical) KV bytes, logical bytes reported too
  long_context_128k    4 sequences of 131,072 tokens, 1% of K rows x8
  fp8_80layer_bs128    a full 80-layer step with an e4m3fn cache: per layer
                       pa_cache_write_fp8 then pa_decode_fp8, 160 launches
                       replayed as one HIP graph; `value` is KV GB/s over the
                       whole step, decode tok/s = 128 / step time
  sliding_window_llama70b  the default batch decoded by a local layer with a
                       1,024-token window from ring tables of 65 entries
                       (pa_decode_ring; the fused step is pa_decode_ring with
                       the new tokens): `value` counts the K/V of the last
                       min(L, 1024) tokens of each sequence; the linear-table
                       pa_decode_window of the same batch is timed beside it
  llama70b_tp2_shard_bs64, llama70b_tp8_shard_bs64  one GPU's share of the
                       default layer split by KV head over 2 or 8 GPUs (4 or 1
                       KV heads, 32 or 8 query heads; the same sequences), as
                       the default step
  bulk_write_llama70b  pa_cache_write of 64 prompts of 2,000 to 2,800 tokens
                       (153,600 tokens) into fresh blocks of the 70B layer's
                       pool, as a prefill writes them: `value` is the bytes
                       read (new K/V rows, slots) plus written (cache tiles)
                       per call / time; the fp8 write is timed beside it
  copy_blocks_llama70b pa_copy_blocks of 4,096 independent block pairs on the
                       70B layer's bf16 pool (block 16): `value` is bytes read
                       plus written per call / time; also the host block
                       manager's add_sequence / append_token rates
  quest_long_context_128k  the long-context batch (4 x 131,072 tokens) decoded
                       with query-aware page selection, 256 pages (4,096
                       tokens) per (sequence, KV head): a step is
                       pa_quest_cache_write (the cache write keeping the page
                       summaries in the same launch), pa_quest_select and
                       pa_decode_quest; `value` counts the bytes the step
                       must read (page summaries, chosen K/V, q, out,
                       tables); the plain decode of the same batch is timed
                       beside it.  The write is pa_quest_cache_write: the
                       summary update in the write's own launch
  quest_llama70b_bs64  the same on the 70B layer bs=64 batch, 64 pages
                       (1,024 tokens) per (sequence, KV head)
  cascade_prefix_shared_bs256  the prefix-shared batch decoded with
                       pa_decode_cascade: its shared segments (the system
                       prompt, the 12 pools) attended to once for all their
                       sequences, each sequence's private tokens by the paged
                       decode, then the merge; `value` counts distinct
                       (physical) KV bytes like prefix_shared_bs256, and the
                       plain decode of the same batch is timed beside it
  swap_blocks_llama70b pa_swap_out then pa_swap_in of 1,024 blocks (64 MiB of
                       K+V) through pinned host memory: `value` is bytes moved
                       per direction / time (bound by the host link, PCIe 5.0
                       x16, 64 GB/s per direction); also the default batch's
                       decode timed alone and with a swap in flight on a
                       second stream

Prints exactly one JSON line on stdout; everything else goes to stderr.
"""

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import paged_kv_cache_32_amd as pa  # noqa: E402
from paged_kv_cache_32_amd import workloads as W  # noqa: E402
from paged_kv_cache_32_amd.step import DecodeStep  # noqa: E402

METRIC = "paged-decode KV GB/s (% of HBM peak) + decode tok/s, 70B-shaped layer, bs=64"
HBM_PEAK_GBS = 8000.0
MODEL_LAYERS = 80
SCRUB_BYTES = 512 << 20
WORKLOADS = {"llama70b_layer_bs64": 2, "prefix_shared_bs256": 3, "long_context_128k": 4,
             "fp8_80layer_bs128": 5, "copy_blocks_llama70b": 2, "sliding_window_llama70b": 2,
             "swap_blocks_llama70b": 2, "quest_long_context_128k": 4, "quest_llama70b_bs64": 2,
             "cascade_prefix_shared_bs256": 3, "bulk_write_llama70b": 2,
             "llama70b_tp2_shard_bs64": 2, "llama70b_tp8_shard_bs64": 2}
CASCADE_CHUNK_TOKENS = 1024
QUEST_BUDGET = {"quest_long_context_128k": 256, "quest_llama70b_bs64": 64}   # pages per (seq, KV head)
HOST_LINK_GBS = 64.0  # PCIe 5.0 x16, per direction: 32 GT/s x 16 lanes / 8 bits
LOCAL_WINDOW = 1024   # a local layer's window ("KV Cache Engineering for LLM Serving", section 3)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, physical=False, window=0):
    """Bytes one decode call must move at minimum: K and V of every cached
    token (each distinct token once when ``physical``; only the last
    ``window`` tokens of each sequence with a window), the queries, the
    outputs, the block-table entries and lengths."""
    S, Hq, D = w.num_seqs, w.num_q_heads, w.head_dim
    if window:
        toks = [min(int(L), window) for L in w.seq_lens]
        kv = sum(toks) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
        blocks = sum(-(-int(L) // w.block_size) - max(int(L) - window, 0) // w.block_size for L in w.seq_lens)
        tables = blocks * 4
        return kv, kv + S * Hq * D * 2 + S * Hq * D * 4 + tables + 4 * S
    kv = w.physical_kv_bytes() if physical else w.logical_kv_bytes()
    tables = int(sum(-(-int(L) // w.block_size) for L in w.seq_lens)) * 4
    other = S * Hq * D * 2 + S * Hq * D * 4 + tables + 4 * S
    return kv, kv + other


KERNEL_SOURCES = ("paged_kv_cache_32_amd/csrc/decode.hip", "paged_kv_cache_32_amd/csrc/pa_internal.h",
                  "paged_kv_cache_32_amd/csrc/api.hip")
CACHE_WRITE_SOURCES = ("paged_kv_cache_32_amd/csrc/cache_write.hip", "paged_kv_cache_32_amd/csrc/pa_internal.h",
                       "paged_kv_cache_32_amd/csrc/api.hip")
TRAFFIC_PROFILES = {"llama70b_layer_bs64": "profiles/decode_kernel_llama70b_bs64_traffic.md",
                    "prefix_shared_bs256": "profiles/decode_kernel_prefix_shared_bs256_traffic.md",
                    "long_context_128k": "profiles/decode_kernel_long_context_128k_traffic.md",
                    "fp8_80layer_bs128": "profiles/decode_kernel_fp8_80layer_bs128_traffic.md",
                    "bulk_write_llama70b": "profiles/cache_write_tiles_kernel_bulk_write_llama70b_traffic.md",
                    "sliding_window_llama70b": "profiles/decode_kernel_sliding_window_llama70b_traffic.md",
                    "llama70b_tp2_shard_bs64": "profiles/decode_kernel_llama70b_tp2_shard_bs64_traffic.md",
                    "llama70b_tp8_shard_bs64": "profiles/decode_kernel_llama70b_tp8_shard_bs64_traffic.md",
                    "quest_llama70b_bs64": "profiles/quest_llama70b_bs64_traffic.md",
                    "quest_long_context_128k": "profiles/quest_long_context_128k_traffic.md",
                    "cascade_prefix_shared_bs256": "profiles/cascade_prefix_shared_bs256_traffic.md",
                    "copy_blocks_llama70b": "profiles/move_blocks_kernel_copy_llama70b_pool_traffic.md"}


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload="llama70b_layer_bs64", part=None):
    """HBM bytes per launch of the workload's dominant kernel (or, with
    ``part``, of that named part of the step) from the committed rocprofv3
    counter summary, or None when there is none or the sources it names
    changed since it was taken."""
    if workload not in TRAFFIC_PROFILES:
        return None
    path = os.path.join(ROOT, TRAFFIC_PROFILES[workload])
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    sources = rec.get("kernel_sources") or (CACHE_WRITE_SOURCES if workload == "bulk_write_llama70b"
                                            else KERNEL_SOURCES)
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    if part is not None:
        return rec.get("parts", {}).get(part, {}).get("traffic_bytes_per_launch")
    return rec.get("traffic_bytes_per_launch")


def host_cores():
    """Host cores this process may run on, with the BLAS pool set to that
    many threads for the oracle's matrix products."""
    from threadpoolctl import threadpool_limits
    n = len(os.sched_getaffinity(0))
    threadpool_limits(limits=n, user_api="blas")
    return n


def cpu_baseline(w, t, out_gpu, layer=0, min_seconds=10.0, max_seconds=30.0, window=0):
    """Time the CPU oracle (float64 numpy) on a bounded sample of the same
    workload: one sequence at a time, in order and wrapping around, until
    about 10 s have elapsed (a whole pass when the batch fits in that time).
    Reports logical KV GB/s of the oracle and its agreement with the GPU on
    the sequences it computed."""
    from oracle import paged
    g = paged.Geom(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)

    def bits(x):
        x = x.detach().cpu()
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()

    kc, vc, q = bits(t["k_cache"][layer]), bits(t["v_cache"][layer]), bits(t["q"][layer])
    kn, vn = bits(t["k_new"][layer]), bits(t["v_new"][layer])
    # The oracle's own write of this step's tokens: every slot the kernels
    # wrote is overwritten with the oracle's encoding; all other slots still
    # hold the generator's values.
    if w.kv_dtype == "bf16":
        ks = vs = 1.0
        paged.cache_write_bf16(g, kn, vn, w.slot_mapping, kc, vc)
    else:
        ks, vs = float(t["k_scale"][layer]), float(t["v_scale"][layer])
        paged.cache_write_fp8(g, kn, vn, w.slot_mapping, kc, vc, np.float32(ks), np.float32(vs))
    threads = host_cores()
    per_token = 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    read = (lambda L: min(L, window)) if window else (lambda L: L)
    ref = np.full((w.num_seqs, w.num_q_heads, w.head_dim), np.nan)
    done = set()
    calls, elapsed, nbytes, s = 0, 0.0, 0, 0
    while elapsed < min_seconds and elapsed < max_seconds:
        t0 = time.perf_counter()
        r = paged.decode(g, q, kc, vc, w.block_tables, w.seq_lens, w.scale, k_scale=ks,
                         v_scale=vs, seqs=[s], window=window)
        elapsed += time.perf_counter() - t0
        nbytes += read(int(w.seq_lens[s])) * per_token
        calls += 1
        if s not in done:
            ref[s] = r[s]
            done.add(s)
        s = (s + 1) % w.num_seqs
    got = out_gpu.detach().cpu().double().numpy()
    idx = sorted(done)
    err = np.abs(got[idx] - ref[idx])
    whole = len(done) == w.num_seqs
    what = (f"{calls // w.num_seqs} whole pass(es) over the {w.num_seqs}-sequence batch"
            if whole and calls % w.num_seqs == 0 else
            f"{calls} single-sequence decodes covering {len(done)} of the {w.num_seqs} sequences")
    return {
        "value": nbytes / elapsed / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"{what} of the same workload (layer {layer}), float64 numpy oracle, "
                   f"{elapsed:.1f} s, {nbytes / 1e9:.2f} GB of logical KV"),
        "seconds": elapsed,
        "gpu_vs_oracle_max_abs": float(err.max()), "gpu_vs_oracle_mean_abs": float(err.mean()),
    }


def base_record(args, w, K):
    return {
        "metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8" if w.kv_dtype == "fp8" else "bf16",
        "data": "synthetic (seeded lognormal lengths, N(0,1) bf16 q/k/v, shuffled block pool)",
        "config": {"workload": args.workload, "num_seqs": w.num_seqs,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "kv_dtype": w.kv_dtype,
                   "num_layers": w.num_layers, "tokens": int(w.seq_lens.sum()),
                   "partition_tokens": args.partition_tokens},
    }


def probe_ceilings(w, kc, vc, bt, sl, scrub, sink, stream, no_scrub, reps=10, tiles=True, window=0):
    """Practical read ceilings (include/pa_probe.h): a plain streaming read of
    the 512 MiB scrub buffer (larger than the Infinity Cache, so every pass
    reads HBM), and the decode's own tile loads with no arithmetic, each
    timed with HIP events on the stream it runs on (the tile read after a
    scrub, like the decode)."""
    dev = kc.device
    psink = torch.zeros(1, dtype=torch.int32, device=dev)

    def tile_read():
        pa.pa_probe_tile_read(kc, vc, bt, sl, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                              block_size=w.block_size, window=window, sink=psink)
    pa.pa_probe_stream_read(scrub, psink)              # warm-up: first launches load the code
    if tiles:
        tile_read()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        pa.pa_probe_stream_read(scrub, psink)
        e[1].record(stream)
    torch.cuda.synchronize()
    stream_s = float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3
    res = {"stream_read_gbs": round(scrub.numel() * 4 / stream_s / 1e9, 1)}
    if tiles:
        eb = 1 if w.kv_dtype == "fp8" else 2
        ok = (w.seq_lens >= 1) & (w.seq_lens <= w.max_blocks_per_seq * w.block_size)
        first = [(int(L) - window) // 16 if 0 < window < int(L) else 0 for L in w.seq_lens[ok]]
        tiles_n = sum(-(-int(L) // 16) - c0 for L, c0 in zip(w.seq_lens[ok], first))
        tile_bytes = int(tiles_n) * 16 * w.num_kv_heads * w.head_dim * eb * 2
        for e in ev:
            if not no_scrub:
                torch.sum(scrub, dim=0, out=sink)
            e[0].record(stream)
            tile_read()
            e[1].record(stream)
        torch.cuda.synchronize()
        tile_s = float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3
        res.update({"tile_read_gbs": round(tile_bytes / tile_s / 1e9, 1), "tile_read_us": round(tile_s * 1e6, 2),
                    "tile_read_bytes": tile_bytes})
    return res


def new_token_blocks_private(w):
    """Whether every sequence's new token (position L - 1) sits in a block no
    other sequence's table names, as the fused append requires."""
    bt, BS = w.block_tables, w.block_size
    used = bt[bt >= 0]
    ids, counts = np.unique(used, return_counts=True)
    refs = dict(zip(ids.tolist(), counts.tolist()))
    for s, L in enumerate(w.seq_lens):
        if L > 0 and refs.get(int(bt[s, (int(L) - 1) // BS]), 0) > 1:
            return False
    return True


def bench_layer(args, dev):
    """One-layer workloads: the cache write and the decode of one batch."""
    m = re.match(r"llama70b_tp(\d)_shard_bs64$", args.workload)
    w = W.llama70b_tp_shard(int(m.group(1))) if m else W.config(WORKLOADS[args.workload])
    shared = args.workload == "prefix_shared_bs256"
    window = LOCAL_WINDOW if args.workload == "sliding_window_llama70b" else 0
    log("workload:", json.dumps(w.summary()))
    t = w.make_tensors(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    sm = torch.from_numpy(w.slot_mapping).to(dev)
    q, kn, vn, kc, vc = t["q"][0], t["k_new"][0], t["v_new"][0], t["k_cache"][0], t["v_cache"][0]
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws_bytes = pa.pa_decode_workspace_size(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                           w.num_seqs, w.num_q_heads, w.max_blocks_per_seq,
                                           args.partition_tokens)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)  # zero-filled once, as required
    # float32 so the reduction reads the buffer directly (an int32 sum would
    # first widen it to int64, writing 1 GiB).
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def write():
        pa.pa_cache_write(kn, vn, sm, kc, vc, block_size=w.block_size)

    ring = None
    if window:
        # A local layer's ring rows: logical block b of the window's span
        # at entry b % (ceil(window / block_size) + 1).
        E = -(-window // w.block_size) + 1
        rt = np.full((w.num_seqs, E), -1, dtype=np.int32)
        for s, L in enumerate(w.seq_lens):
            for b in range(max(0, int(L) - window) // w.block_size, -(-int(L) // w.block_size)):
                rt[s, b % E] = w.block_tables[s, b]
        ring = torch.from_numpy(rt).to(dev)

    def decode():
        if window:
            pa.pa_decode_ring(q, kc, vc, ring, sl, window, w.scale, out, num_kv_heads=w.num_kv_heads,
                              block_size=w.block_size, partition_tokens=args.partition_tokens,
                              workspace=ws)
        else:
            pa.pa_decode(q, kc, vc, bt, sl, w.scale, out, num_kv_heads=w.num_kv_heads,
                         block_size=w.block_size, partition_tokens=args.partition_tokens, workspace=ws)

    for i in range(args.warmup):
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=sink)
        write()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=sink)
        ev[i][0].record(stream)
        write()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])

    # Hot-cache reference: the same decode back to back with no scrub.
    hot = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    hot[0].record(stream)
    for _ in range(K):
        decode()
    hot[1].record(stream)
    torch.cuda.synchronize()
    hot_ms = hot[0].elapsed_time(hot[1]) / K

    # The local layer's decode from its linear table, timed the same way.
    linear = None
    if window:
        lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            if not args.no_scrub:
                torch.sum(scrub, dim=0, out=sink)
            lev[i][0].record(stream)
            pa.pa_decode_window(q, kc, vc, bt, sl, window, w.scale, out, num_kv_heads=w.num_kv_heads,
                                block_size=w.block_size, partition_tokens=args.partition_tokens, workspace=ws)
            lev[i][1].record(stream)
        torch.cuda.synchronize()
        linear = np.array([e[0].elapsed_time(e[1]) for e in lev])

    # The same step as one fused launch (pa_decode_append, or pa_decode_ring
    # with the new tokens: the write folded into the decode), timed the same
    # way.
    fused = None
    if new_token_blocks_private(w):
        def fused_step():
            if window:
                pa.pa_decode_ring(q, kc, vc, ring, sl, window, w.scale, out, num_kv_heads=w.num_kv_heads,
                                  block_size=w.block_size, k_new=kn, v_new=vn,
                                  partition_tokens=args.partition_tokens, workspace=ws)
            else:
                pa.pa_decode_append(q, kn, vn, kc, vc, bt, sl, w.scale, out, num_kv_heads=w.num_kv_heads,
                                    block_size=w.block_size, partition_tokens=args.partition_tokens,
                                    workspace=ws)
        for _ in range(args.warmup):
            if not args.no_scrub:
                torch.sum(scrub, dim=0, out=sink)
            fused_step()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            if not args.no_scrub:
                torch.sum(scrub, dim=0, out=sink)
            fev[i][0].record(stream)
            fused_step()
            fev[i][1].record(stream)
        torch.cuda.synchronize()
        fused = np.array([e[0].elapsed_time(e[1]) for e in fev])

    # The tile-read probe splits the tiles evenly over 4 waves per SIMD with
    # one batch in flight each: a faithful bound for the long reads, but on
    # the short windowed read (247 MB) it is slower than the decode itself,
    # so that workload reports the streaming-read ceiling only.
    ceilings = probe_ceilings(w, kc, vc, bt, sl, scrub, sink, stream, args.no_scrub, tiles=not window)

    kv_bytes, alg_bytes = algorithmic_bytes(w, physical=shared, window=window)
    logical_kv = w.logical_kv_bytes()
    dec_s = float(dec_ms.mean()) / 1e3
    step_ms = float((write_ms + dec_ms).mean())
    kv_gbs = kv_bytes / dec_s / 1e9
    alg_gbs = alg_bytes / dec_s / 1e9
    res = base_record(args, w, K)
    if args.workload != "llama70b_layer_bs64":
        res["metric"] = f"paged-decode KV GB/s (% of HBM peak) + decode tok/s, {args.workload}"
    res.update({"value": round(kv_gbs, 1), "ms_per_step": round(step_ms, 4)})
    res["config"].update({"kv_bytes_per_call": kv_bytes, "kv_bytes_basis":
                          "distinct (physical) tokens" if shared else
                          (f"last {window} tokens of each sequence" if window else "every cached token"),
                          "window": window,
                          "scrub_mib_between_steps": 0 if args.no_scrub else SCRUB_BYTES >> 20})
    res.update({
        "hbm_peak_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "decode_us": {"mean": round(dec_s * 1e6, 2), "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.median(dec_ms)) * 1e3, 2),
                      "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2)},
        "cache_write_us": round(float(write_ms.mean()) * 1e3, 2),
        "decode_hot_cache_us": round(hot_ms * 1e3, 2),
        "layer_tok_s": round(w.num_seqs / (step_ms / 1e3), 1),
        "decode_tok_s_80layer_equiv": round(w.num_seqs / (MODEL_LAYERS * step_ms / 1e3), 1),
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(alg_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(alg_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload),
                     "kernel": "decode_kernel (pa_decode is one launch)",
                     "bytes_per_launch": alg_bytes},
    })
    if window:
        res["config"]["ring_entries"] = int(ring.shape[1])
        res["config"]["linear_table_entries"] = int(w.max_blocks_per_seq)
        res["linear_table_window_decode_us"] = {"mean": round(float(linear.mean()) * 1e3, 2),
                                                "p50": round(float(np.median(linear)) * 1e3, 2)}
    ceilings["decode_frac_of_stream_read"] = round(kv_gbs / ceilings["stream_read_gbs"], 4)
    if "tile_read_us" in ceilings:
        # Both read the same tiles: the ratio of times is the fraction of the
        # access pattern's own ceiling that the decode reaches.
        ceilings["decode_frac_of_tile_read"] = round(ceilings["tile_read_us"] / float(np.median(dec_ms) * 1e3), 4)
    res["ceilings"] = ceilings
    if fused is not None:
        f_ms = float(fused.mean())
        res["fused_append_decode"] = {
            "entry_point": "pa_decode_ring" if window else "pa_decode_append", "us_mean": round(f_ms * 1e3, 2),
            "us_p50": round(float(np.median(fused)) * 1e3, 2),
            "layer_tok_s": round(w.num_seqs / (f_ms / 1e3), 1),
            "step_saving_us": round((step_ms - f_ms) * 1e3, 2)}
    else:
        res["fused_append_decode"] = "not timed: a new token's block is read by another sequence"
    if shared:
        res["logical_kv_gbs"] = round(logical_kv / dec_s / 1e9, 1)
        res["logical_kv_bytes_per_call"] = logical_kv
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_baseline(w, t, out, window=window)
    return res


def bench_model_step(args, dev):
    """The 80-layer fp8 step: per layer the fp8 write and the fp8 decode, all
    160 launches captured once in a HIP graph and replayed per step."""
    w = W.config(WORKLOADS[args.workload])
    log("workload:", json.dumps(w.summary()))
    t0 = time.perf_counter()
    t = w.make_tensors(dev)
    log(f"tensors for {w.num_layers} layers drawn in {time.perf_counter() - t0:.1f} s")
    n = w.num_layers
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    sm = torch.from_numpy(w.slot_mapping).to(dev)
    out = torch.empty((n, w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    step = DecodeStep(q=t["q"], k_new=t["k_new"], v_new=t["v_new"], k_cache=t["k_cache"],
                      v_cache=t["v_cache"], out=out, block_tables=bt, seq_lens=sl, slot_mapping=sm,
                      scale=w.scale, num_kv_heads=w.num_kv_heads, block_size=w.block_size,
                      k_scale=t["k_scale"].tolist(), v_scale=t["v_scale"].tolist(),
                      partition_tokens=args.partition_tokens)
    stream = torch.cuda.current_stream(dev)

    # Eager, with an event after every layer: per-layer times.
    K = args.steps
    for _ in range(max(args.warmup, 1)):
        step.run()
    torch.cuda.synchronize()
    lay_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    eager_ms = []
    per_layer = np.zeros(n)
    eager_steps = min(K, 5)
    for _ in range(eager_steps):
        step.run(events=lay_ev)
        torch.cuda.synchronize()
        eager_ms.append(lay_ev[0].elapsed_time(lay_ev[n]))
        per_layer += np.array([lay_ev[i].elapsed_time(lay_ev[i + 1]) for i in range(n)])
    per_layer /= eager_steps

    # One write + one decode of a middle layer, each between events, for the
    # decode kernel's own time (the roofline's unit).
    mid = n // 2
    kd = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        kd[i][0].record(stream)
        step.write(mid)
        kd[i][1].record(stream)
        step.decode(mid)
        kd[i][2].record(stream)
    torch.cuda.synchronize()
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in kd])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in kd])

    # Graph: the whole step as one replay.
    step.capture()
    for _ in range(args.warmup):
        step.replay()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    tw = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        step.replay()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw
    graph_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])

    # The same step with each layer's write and decode as one fused launch
    # (pa_decode_append_fp8): 80 launches in its graph instead of 160.
    fused_ms = None
    if new_token_blocks_private(w):
        fstep = DecodeStep(q=t["q"], k_new=t["k_new"], v_new=t["v_new"], k_cache=t["k_cache"],
                           v_cache=t["v_cache"], out=out, block_tables=bt, seq_lens=sl, slot_mapping=sm,
                           scale=w.scale, num_kv_heads=w.num_kv_heads, block_size=w.block_size,
                           k_scale=t["k_scale"].tolist(), v_scale=t["v_scale"].tolist(),
                           partition_tokens=args.partition_tokens, workspace=step.workspace, fused=True)
        fstep.capture()
        for _ in range(args.warmup):
            fstep.replay()
        torch.cuda.synchronize()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            fev[i][0].record(stream)
            fstep.replay()
            fev[i][1].record(stream)
        torch.cuda.synchronize()
        fused_ms = np.array([e[0].elapsed_time(e[1]) for e in fev])

    kv_layer, alg_layer = algorithmic_bytes(w)
    step_s = float(graph_ms.mean()) / 1e3
    dec_s = float(dec_ms.mean()) / 1e3
    kv_gbs = n * kv_layer / step_s / 1e9
    res = base_record(args, w, K)
    res["metric"] = f"paged-decode KV GB/s (% of HBM peak) + decode tok/s, {args.workload}"
    res.update({"value": round(kv_gbs, 1), "ms_per_step": round(float(graph_ms.mean()), 4)})
    res["config"].update({"kv_bytes_per_step": n * kv_layer, "kv_bytes_per_layer": kv_layer,
                          "step": "per layer pa_cache_write_fp8 + pa_decode_fp8, one HIP graph"})
    res.update({
        "hbm_peak_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "decode_tok_s": round(w.num_seqs / step_s, 1),
        "step_ms": {"graph_mean": round(float(graph_ms.mean()), 4),
                    "graph_p10": round(float(np.percentile(graph_ms, 10)), 4),
                    "graph_p90": round(float(np.percentile(graph_ms, 90)), 4),
                    "eager_mean": round(float(np.mean(eager_ms)), 4)},
        "layer_ms_eager": {"mean": round(float(per_layer.mean()), 4),
                           "min": round(float(per_layer.min()), 4),
                           "max": round(float(per_layer.max()), 4)},
        "decode_us_one_layer": round(dec_s * 1e6, 2),
        "cache_write_us_one_layer": round(float(write_ms.mean()) * 1e3, 2),
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(alg_layer / dec_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg_layer / dec_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload),
                     "kernel": "decode_kernel fp8 (one layer's pa_decode_fp8)",
                     "bytes_per_launch": alg_layer},
    })
    if fused_ms is not None:
        f_s = float(fused_ms.mean()) / 1e3
        res["fused_append_decode"] = {
            "entry_point": "pa_decode_append_fp8, one launch per layer, one HIP graph",
            "step_ms_mean": round(f_s * 1e3, 4), "step_ms_p10": round(float(np.percentile(fused_ms, 10)), 4),
            "step_ms_p90": round(float(np.percentile(fused_ms, 90)), 4),
            "decode_tok_s": round(w.num_seqs / f_s, 1), "kv_gbs": round(n * kv_layer / f_s / 1e9, 1)}
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_baseline(w, t, out[0], layer=0)
    return res


def bench_copy_blocks(args, dev):
    """pa_copy_blocks on the 70B layer's pool, and the host block manager."""
    w = W.config(2)
    Hkv, D, BS = w.num_kv_heads, w.head_dim, w.block_size
    n_pairs = 4096
    elems = w.num_blocks * Hkv * BS * D
    kc = torch.empty(elems, dtype=torch.bfloat16, device=dev).normal_()
    vc = torch.empty(elems, dtype=torch.bfloat16, device=dev).normal_()
    rng = np.random.default_rng(2)
    perm = rng.permutation(w.num_blocks)
    pairs = torch.from_numpy(np.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], 1).astype(np.int32)).to(dev)
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def copy():
        pa.pa_copy_blocks(kc, vc, pairs, num_kv_heads=Hkv, head_dim=D, block_size=BS)

    for _ in range(args.warmup):
        copy()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=sink)
        ev[i][0].record(stream)
        copy()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    block_bytes = Hkv * BS * D * 2
    moved = n_pairs * 2 * block_bytes * 2             # K and V, read and write
    gbs = moved / (ms.mean() / 1e3) / 1e9

    # Host block manager: the batch's prompts (a shared 900-token system
    # prompt, then private tokens) added, then one append per sequence per
    # step for 256 steps.
    bm = pa.BlockManager(w.num_blocks, BS)
    system = list(range(900))
    t0 = time.perf_counter()
    for s, L in enumerate(w.seq_lens):
        L = int(L)
        bm.add_sequence(s, (system + list(range(10_000 + s * 40_000, 10_000 + s * 40_000 + L)))[:L])
    t_add = time.perf_counter() - t0
    t0 = time.perf_counter()
    n_app = 0
    for step in range(256):
        for s in range(w.num_seqs):
            bm.append_token(s, step)
            n_app += 1
    t_app = time.perf_counter() - t0
    hits, misses = bm.stats()
    res = base_record(args, w, K)
    res["metric"] = "pa_copy_blocks GB/s (read + write) on the 70B layer pool, and block manager op rates"
    res.update({"value": round(gbs, 1), "ms_per_step": round(float(ms.mean()), 4)})
    res["config"].update({"workload": args.workload, "pairs": n_pairs, "block_bytes_per_cache": block_bytes,
                          "bytes_moved_per_call": moved})
    res.update({
        "copy_us": {"mean": round(float(ms.mean()) * 1e3, 2), "p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                    "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                     "kernel": "move_blocks_kernel (pa_copy_blocks is one launch)", "bytes_per_launch": moved},
        "block_manager": {"add_sequence_tokens_per_s": round(float(w.seq_lens.sum()) / t_add, 1),
                          "append_token_per_s": round(n_app / t_app, 1),
                          "prefix_hits": hits, "blocks_taken": misses},
    })
    return res


BULK_PROMPTS, BULK_MEAN_TOKENS = 64, 2400


def bulk_write_inputs(w, rng):
    """Slots of 64 prompts of 2,000 to 2,800 tokens (153,600 in all), each
    written from position 0 into blocks drawn at random from the pool."""
    d = rng.integers(-400, 401, BULK_PROMPTS // 2)
    lens = BULK_MEAN_TOKENS + rng.permutation(np.concatenate([d, -d]))
    perm = rng.permutation(w.num_blocks)
    slots, used = [], 0
    for L in lens:
        nb = -(-int(L) // w.block_size)
        blocks = perm[used:used + nb].astype(np.int64)
        used += nb
        pos = np.arange(int(L))
        slots.append(blocks[pos // w.block_size] * w.block_size + pos % w.block_size)
    assert used <= w.num_blocks
    return lens, np.concatenate(slots)


def bench_bulk_write(args, dev):
    """pa_cache_write of a prefill-sized batch of prompt rows."""
    w = W.config(2)
    Hkv, D, BS = w.num_kv_heads, w.head_dim, w.block_size
    rng = np.random.default_rng(8)
    lens, slots = bulk_write_inputs(w, rng)
    T = int(slots.size)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    k = torch.randn((T, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((T, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    sm = torch.from_numpy(slots).to(dev)
    elems = w.num_blocks * Hkv * BS * D
    kc = torch.zeros(elems, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(elems, dtype=torch.bfloat16, device=dev)
    kc8 = torch.zeros(elems, dtype=torch.uint8, device=dev)
    vc8 = torch.zeros(elems, dtype=torch.uint8, device=dev)
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ks, vs = 0.02, 0.02

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            if not args.no_scrub:
                torch.sum(scrub, dim=0, out=sink)
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in ev])

    t0 = time.perf_counter()
    ms = timed(lambda: pa.pa_cache_write(k, v, sm, kc, vc, block_size=BS))
    wall = time.perf_counter() - t0
    ms8 = timed(lambda: pa.pa_cache_write_fp8(k, v, sm, kc8, vc8, ks, vs, block_size=BS))
    row = Hkv * D
    read = T * row * 2 * 2 + T * 8                  # new K and V rows (bf16), slots
    wrote, wrote8 = T * row * 2 * 2, T * row * 2    # K and V tiles
    gbs = (read + wrote) / (ms.mean() / 1e3) / 1e9
    gbs8 = (read + wrote8) / (ms8.mean() / 1e3) / 1e9
    whole = sum(int(L) // 16 for L in lens)
    res = base_record(args, w, args.steps)
    res["metric"] = "pa_cache_write GB/s (bytes read + written) of a prefill-sized batch, 70B layer"
    res.update({"value": round(gbs, 1), "ms_per_step": round(float(ms.mean()), 4),
                "data": "synthetic (seeded N(0,1) bf16 K/V rows, prompt lengths uniform in [2000, 2800], "
                        "shuffled block pool)"})
    res["config"].update({"workload": args.workload, "num_seqs": BULK_PROMPTS, "tokens": T,
                          "prompt_tokens_min_max": [int(lens.min()), int(lens.max())],
                          "whole_16_token_sub_blocks": whole, "bytes_read_per_call": read,
                          "bytes_written_per_call": wrote})
    res.update({
        "write_us": {"mean": round(float(ms.mean()) * 1e3, 2), "p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                     "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)},
        "tokens_per_s": round(T / (ms.mean() / 1e3), 1),
        "wall_s_timed_region": round(wall, 4),
        "fp8_write": {"us_mean": round(float(ms8.mean()) * 1e3, 2), "gbs": round(gbs8, 1),
                      "bytes_written_per_call": wrote8, "hbm_peak_frac": round(gbs8 / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                     "kernel": "cache_write_tiles_kernel (pa_cache_write is one launch)",
                     "bytes_per_launch": read + wrote},
    })
    if not args.skip_cpu:
        res["cpu_baseline"] = bulk_write_cpu_baseline(w, lens, slots, k, v, kc)
    return res


def bulk_write_cpu_baseline(w, lens, slots, k, v, kc_gpu, min_seconds=10.0):
    """The oracle's scatter (numpy) on whole prompts of the same batch, in
    order until about 10 s have elapsed; the written slots are compared with
    the GPU's cache."""
    from oracle import paged
    g = paged.Geom(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, "bf16")
    cores = host_cores()

    def bits(x):
        return x.detach().cpu().view(torch.int16).numpy().view(np.uint16)

    kb, vb = bits(k), bits(v)
    kc = np.zeros(g.cache_elems, dtype=np.uint16)
    vc = kc.copy()
    starts = np.concatenate([[0], np.cumsum(lens)])
    elapsed, done = 0.0, 0
    while elapsed < min_seconds and done < len(lens):
        a, b = int(starts[done]), int(starts[done + 1])
        t0 = time.perf_counter()
        paged.cache_write_bf16(g, kb[a:b], vb[a:b], slots[a:b], kc, vc)
        elapsed += time.perf_counter() - t0
        done += 1
    n = int(starts[done])
    got = bits(kc_gpu)
    hh, dd = np.meshgrid(np.arange(w.num_kv_heads), np.arange(w.head_dim), indexing="ij")
    blk, off = np.divmod(slots[:n:97], w.block_size)
    idx = np.stack([paged.k_offset(g, b, hh, o, dd) for b, o in zip(blk, off)]).ravel()
    row = w.num_kv_heads * w.head_dim
    moved = n * row * 2 * 4 + n * 8
    return {"value": moved / elapsed / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"{done} of the {len(lens)} prompts ({n} tokens) of the same batch, numpy oracle "
                       f"scatter, {elapsed:.1f} s"),
            "seconds": elapsed, "gpu_vs_oracle_k_mismatches_sampled": int((got[idx] != kc[idx]).sum())}


def quest_bytes(w, budget):
    """Algorithmic bytes of one query-aware step, per call: the update reads
    the new keys and rewrites their blocks' summary words; the selection
    reads every page's summary words, the queries and the table entries and
    writes the chosen tables; the decode reads the chosen pages' K and V
    (the tokens each (sequence, KV head) keeps), the queries and the chosen
    tables, and writes the outputs."""
    S, Hq, Hkv, D, BS, eb = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.elem_bytes
    pages = [-(-int(L) // BS) for L in w.seq_lens]
    update = S * Hkv * D * eb + 2 * S * Hkv * D * 4
    select = sum(pages) * Hkv * D * 4 + S * Hq * D * 2 + sum(pages) * 4 + 4 * S + S * Hkv * (budget + 1) * 4
    kept = 0
    for L, n in zip(w.seq_lens, pages):
        L = int(L)
        kept += Hkv * (L if n <= budget else budget * BS)      # the last page may be short: upper bound
    decode = kept * 2 * D * eb + S * Hq * D * 2 + S * Hq * D * 4 + S * Hkv * (min(budget, max(pages)) + 1) * 4
    return {"update": update, "select": select, "decode": decode, "kept_tokens_upper": kept}


def quest_cpu_baseline(w, t, out_gpu, budget, min_seconds=10.0):
    """The Quest oracle on a bounded sample of the same batch: (sequence, KV
    head) units in order until about 10 s have elapsed; bytes as the GPU's
    algorithmic bytes for those units (summaries of every page, K/V of the
    kept tokens)."""
    from oracle import paged, quest
    g = paged.Geom(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)

    def bits(x):
        x = x.detach().cpu()
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()

    kc, vc = bits(t["k_cache"][0]), bits(t["v_cache"][0])
    paged.cache_write_bf16(g, bits(t["k_new"][0]), bits(t["v_new"][0]), w.slot_mapping, kc, vc)
    qf = paged.bf16_bits_to_f64(bits(t["q"][0]))
    G, BS, D = w.num_q_heads // w.num_kv_heads, w.block_size, w.head_dim
    got = out_gpu.detach().cpu().double().numpy()
    threads = host_cores()
    elapsed, nbytes, units, errs = 0.0, 0, 0, []
    u = 0
    while elapsed < min_seconds and units < w.num_seqs * w.num_kv_heads:
        s, h = divmod(u, w.num_kv_heads)
        L = int(w.seq_lens[s])
        t0 = time.perf_counter()
        mn, mx = quest.sequence_page_summaries(g, kc, w.block_tables[s], L, h)
        chosen = quest.select_pages(quest.page_scores(qf[s, h * G:(h + 1) * G].astype(np.float32), mn, mx),
                                    budget)
        K, V = paged.gather(g, kc, vc, w.block_tables[s], L, h)
        pos = [p * BS + i for p in chosen for i in range(BS) if p * BS + i < L]
        ref = paged.softmax_attention(qf[s, h * G:(h + 1) * G], K[pos], V[pos], w.scale)
        elapsed += time.perf_counter() - t0
        nbytes += len(mn) * D * 4 + len(pos) * 2 * D * w.elem_bytes
        errs.append(float(np.abs(got[s, h * G:(h + 1) * G] - ref).max()))
        units += 1
        u += 1
    return {"value": nbytes / elapsed / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{units} of the {w.num_seqs * w.num_kv_heads} (sequence, KV head) units of the same "
                       f"batch, float64 numpy Quest oracle (summaries from the gathered sequence, float32 "
                       f"scores, choice, attention over the kept tokens), {elapsed:.1f} s"),
            "seconds": elapsed, "gpu_vs_oracle_max_abs": max(errs)}


def bench_quest(args, dev):
    """Query-aware step (write, summary update, page choice, decode over the
    chosen pages) against the plain decode of the same batch."""
    w = W.config(WORKLOADS[args.workload])
    budget = QUEST_BUDGET[args.workload]
    Hkv, D, BS = w.num_kv_heads, w.head_dim, w.block_size
    kw = dict(num_kv_heads=Hkv, block_size=BS)
    log("workload:", json.dumps(w.summary()), "budget pages:", budget)
    t = w.make_tensors(dev, poison=False)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    sm = torch.from_numpy(w.slot_mapping).to(dev)
    q, kn, vn, kc, vc = t["q"][0], t["k_new"][0], t["v_new"][0], t["k_cache"][0], t["v_cache"][0]
    S = w.num_seqs
    out = torch.empty((S, w.num_q_heads, D), dtype=torch.float32, device=dev)
    full_out = torch.empty_like(out)
    # The step's write once, then summaries of every block the batch holds
    # (set-up, not timed): the summaries then cover the written tokens.
    pa.pa_cache_write(kn, vn, sm, kc, vc, block_size=BS)
    items = {}
    for s, L in enumerate(w.seq_lens):
        L = int(L)
        for p in range(-(-L // BS)):
            items[int(w.block_tables[s, p])] = min(BS, L - p * BS)
    summ = pa.quest_summaries(kc, num_kv_heads=Hkv, head_dim=D, block_size=BS)
    pa.pa_quest_summarize(kc, torch.tensor(list(items), dtype=torch.int32, device=dev),
                          torch.tensor(list(items.values()), dtype=torch.int32, device=dev), summ,
                          num_kv_heads=Hkv, head_dim=D, block_size=BS)
    sel_t = torch.empty((S * Hkv, budget), dtype=torch.int32, device=dev)
    sel_l = torch.empty((S * Hkv,), dtype=torch.int32, device=dev)
    sel_ws = torch.empty(max(pa.lib().pa_quest_select_workspace_size(S, Hkv, w.max_blocks_per_seq), 1),
                         dtype=torch.uint8, device=dev)
    desc = pa.make_desc(kc, Hkv, D, BS)
    dws = torch.zeros(pa.lib().pa_decode_quest_workspace_size(ctypes.byref(desc), S, w.num_q_heads, budget, 0),
                      dtype=torch.uint8, device=dev)
    fws = torch.zeros(pa.pa_decode_workspace_size(w.num_blocks, BS, Hkv, D, S, w.num_q_heads,
                                                  w.max_blocks_per_seq, 0), dtype=torch.uint8, device=dev)
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def phases():
        # The step's write keeps the summaries in the same launch (one new
        # token per sequence, each in a block of its own).
        pa.pa_quest_cache_write(kn, vn, sm, kc, vc, summ, block_size=BS)
        yield
        pa.pa_quest_select(q, summ, bt, sl, budget, sel_tables=sel_t, sel_lens=sel_l, workspace=sel_ws, **kw)
        yield
        pa.pa_decode_quest(q, kc, vc, sel_t, sel_l, w.scale, out, workspace=dws, **kw)
        yield

    def full():
        pa.pa_decode(q, kc, vc, bt, sl, w.scale, full_out, workspace=fws, **kw)

    for _ in range(args.warmup):
        for _ in phases():
            pass
        full()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=sink)
        ev[i][0].record(stream)
        for j, _ in enumerate(phases()):
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(K):
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=sink)
        fev[i][0].record(stream)
        full()
        fev[i][1].record(stream)
    torch.cuda.synchronize()
    ph = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev])   # ms
    full_ms = np.array([e[0].elapsed_time(e[1]) for e in fev])
    step_ms = float(ph.sum(axis=1).mean())
    qb = quest_bytes(w, budget)
    kept = int(sel_l.clamp(min=0).sum().item())
    qb["decode"] -= (qb["kept_tokens_upper"] - kept) * 2 * D * w.elem_bytes     # the exact kept tokens
    total = qb["update"] + qb["select"] + qb["decode"] + S * Hkv * D * 2 * w.elem_bytes
    names = ["quest_cache_write", "quest_select", "decode_quest"]
    means = {n: float(ph[:, j].mean()) for j, n in enumerate(names)}
    dom = max(("quest_select", "decode_quest"), key=lambda n: means[n])
    dom_bytes = qb["select"] if dom == "quest_select" else qb["decode"]
    dom_gbs = dom_bytes / (means[dom] / 1e3) / 1e9
    full_kv, _ = algorithmic_bytes(w)
    res = base_record(args, w, K)
    res["metric"] = f"query-aware (Quest) decode step: algorithmic GB/s and speed-up over plain decode, {args.workload}"
    res.update({"value": round(total / (step_ms / 1e3) / 1e9, 1), "ms_per_step": round(step_ms, 4)})
    res["config"].update({"workload": args.workload, "budget_pages": budget, "budget_tokens": budget * BS,
                          "kept_tokens": kept, "bytes_per_step": total,
                          "scrub_mib_between_steps": 0 if args.no_scrub else SCRUB_BYTES >> 20})
    res.update({
        "phase_us": {n: round(v * 1e3, 2) for n, v in means.items()},
        "full_decode_us": round(float(full_ms.mean()) * 1e3, 2),
        "speedup_vs_full_decode": round(float(full_ms.mean()) / step_ms, 3),
        "full_kv_bytes": full_kv, "kept_kv_bytes": kept * 2 * D * w.elem_bytes,
        "layer_tok_s": round(S / (step_ms / 1e3), 1),
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload, dom),
                     "kernel": {"quest_select": "page_score_kernel + page_select_kernel (pa_quest_select)",
                                "decode_quest": "decode_kernel (pa_decode_quest is one launch)"}[dom],
                     "bytes_per_launch": dom_bytes},
    })
    if not args.skip_cpu:
        res["cpu_baseline"] = quest_cpu_baseline(w, t, out, budget)
    return res


def bench_cascade(args, dev):
    """Shared-prefix decode of the prefix-shared batch against its plain
    decode (the write of the step's tokens is the same for both and timed
    separately)."""
    w = W.config(3)
    log("workload:", json.dumps(w.summary()))
    Hkv, D, BS, S = w.num_kv_heads, w.head_dim, w.block_size, w.num_seqs
    t = w.make_tensors(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    sm = torch.from_numpy(w.slot_mapping).to(dev)
    q, kn, vn, kc, vc = t["q"][0], t["k_new"][0], t["v_new"][0], t["k_cache"][0], t["v_cache"][0]
    t0 = time.perf_counter()
    plan = pa.CascadePlan(w.block_tables, w.seq_lens, block_size=BS, num_kv_heads=Hkv, num_q_heads=w.num_q_heads,
                          chunk_tokens=CASCADE_CHUNK_TOKENS, device=dev)
    plan_ms = (time.perf_counter() - t0) * 1e3
    out = torch.empty((S, w.num_q_heads, D), dtype=torch.float32, device=dev)
    full_out = torch.empty_like(out)
    desc = pa.make_desc(kc, Hkv, D, BS)
    cws = torch.zeros(pa.lib().pa_decode_cascade_workspace_size(ctypes.byref(desc), S, w.num_q_heads,
                                                                w.max_blocks_per_seq, plan.info["num_slots"], 0),
                      dtype=torch.uint8, device=dev)
    fws = torch.zeros(pa.pa_decode_workspace_size(w.num_blocks, BS, Hkv, D, S, w.num_q_heads,
                                                  w.max_blocks_per_seq, 0), dtype=torch.uint8, device=dev)
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    kw = dict(num_kv_heads=Hkv, block_size=BS)

    def write():
        pa.pa_cache_write(kn, vn, sm, kc, vc, block_size=BS)

    def cascade():
        pa.pa_decode_cascade(q, kc, vc, plan, w.scale, out, workspace=cws, **kw)

    def full():
        pa.pa_decode(q, kc, vc, bt, sl, w.scale, full_out, workspace=fws, **kw)

    for _ in range(args.warmup):
        write()
        cascade()
        full()
    torch.cuda.synchronize()
    K = args.steps

    def timed(fn):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for e in ev:
            if not args.no_scrub:
                torch.sum(scrub, dim=0, out=sink)
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    write_ms = timed(write)
    cas_ms = timed(cascade)
    full_ms = timed(full)
    err = float((out - full_out).abs().max().item())
    kv_phys, alg_phys = algorithmic_bytes(w, physical=True)
    kv_log = w.logical_kv_bytes()
    dec_s = float(cas_ms.mean()) / 1e3
    step_ms = float((write_ms + cas_ms).mean())
    gbs = kv_phys / dec_s / 1e9
    alg_gbs = alg_phys / dec_s / 1e9
    res = base_record(args, w, K)
    res["metric"] = "shared-prefix (cascade) decode: distinct KV GB/s and speed-up over plain decode, prefix_shared_bs256"
    res.update({"value": round(gbs, 1), "ms_per_step": round(step_ms, 4)})
    res["config"].update({"workload": args.workload, "kv_bytes_per_call": kv_phys,
                          "kv_bytes_basis": "distinct (physical) tokens", "chunk_tokens": CASCADE_CHUNK_TOKENS,
                          "scrub_mib_between_steps": 0 if args.no_scrub else SCRUB_BYTES >> 20})
    res.update({
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "decode_us": {"mean": round(dec_s * 1e6, 2), "p10": round(float(np.percentile(cas_ms, 10)) * 1e3, 2),
                      "p90": round(float(np.percentile(cas_ms, 90)) * 1e3, 2)},
        "plain_decode_us": round(float(full_ms.mean()) * 1e3, 2),
        "speedup_vs_plain_decode": round(float(full_ms.mean()) / float(cas_ms.mean()), 3),
        "cascade_vs_plain_max_abs": err,
        "cache_write_us": round(float(write_ms.mean()) * 1e3, 2),
        "logical_kv_gbs": round(kv_log / dec_s / 1e9, 1),
        "plan": {k: plan.info[k] for k in ("num_segments", "num_items", "num_slots", "shared_tokens",
                                           "segment_tokens")},
        "plan_build_host_ms": round(plan_ms, 2),
        "layer_tok_s": round(S / (step_ms / 1e3), 1),
        "roofline": {"bound": "hbm", "achieved": round(alg_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                     "kernel": "segment_kernel + decode_kernel + combine_kernel (pa_decode_cascade)",
                     "bytes_per_launch": alg_phys},
    })
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_baseline(w, t, out)
    return res


def bench_swap(args, dev):
    """pa_swap_out / pa_swap_in of 1,024 blocks of the 70B layer's pool, and
    the default batch's decode with a swap running beside it on a second
    stream (the overlap the swapping design relies on)."""
    w = W.config(2)
    Hkv, D, BS = w.num_kv_heads, w.head_dim, w.block_size
    n = 1024
    block_bytes = Hkv * BS * D * 2
    # The pool has n spare blocks past the ones the batch's tables use: the
    # swap-in lands there, so the concurrent decode never reads a block that
    # is being written.
    t = w.make_tensors(dev, poison=False)
    extra = n * Hkv * BS * D
    kc = torch.cat([t["k_cache"][0].reshape(-1), torch.zeros(extra, dtype=torch.bfloat16, device=dev)])
    vc = torch.cat([t["v_cache"][0].reshape(-1), torch.zeros(extra, dtype=torch.bfloat16, device=dev)])
    del t["k_cache"], t["v_cache"]
    rng = np.random.default_rng(3)
    out_ids = torch.from_numpy(rng.permutation(w.num_blocks)[:n].astype(np.int32)).to(dev)
    in_ids = torch.from_numpy((w.num_blocks + rng.permutation(n)).astype(np.int32)).to(dev)
    nbytes = 2 * n * block_bytes
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    kw = dict(num_kv_heads=Hkv, head_dim=D, block_size=BS)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    q = t["q"][0]
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.zeros(pa.pa_decode_workspace_size(w.num_blocks + n, BS, Hkv, D, w.num_seqs, w.num_q_heads,
                                                 w.max_blocks_per_seq, 0), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)

    def swap_out():
        pa.pa_swap_out(kc, vc, out_ids, host, **kw)

    def swap_in():
        pa.pa_swap_in(kc, vc, in_ids, host, **kw)

    def decode():
        pa.pa_decode(q, kc, vc, bt, sl, w.scale, out, num_kv_heads=Hkv, block_size=BS, workspace=ws)

    for _ in range(args.warmup):
        swap_out()
        swap_in()
        decode()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        swap_out()
        ev[i][1].record(stream)
        swap_in()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    out_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    in_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])

    # Decode alone, then decode with a swap-out + swap-in on the side stream.
    def timed_decodes(with_swap):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        side_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            if not args.no_scrub:
                torch.sum(scrub, dim=0, out=sink)
            side.wait_stream(stream)
            evs[i][0].record(stream)
            if with_swap:
                with torch.cuda.stream(side):
                    side_ev[i][0].record(side)
                    swap_out()
                    swap_in()
                    side_ev[i][1].record(side)
            decode()
            evs[i][1].record(stream)
            stream.wait_stream(side)
        torch.cuda.synchronize()
        dec = np.array([e[0].elapsed_time(e[1]) for e in evs])
        sw = np.array([e[0].elapsed_time(e[1]) for e in side_ev]) if with_swap else None
        return dec, sw

    dec_alone, _ = timed_decodes(False)
    dec_busy, swap_busy = timed_decodes(True)
    out_gbs = nbytes / (out_ms.mean() / 1e3) / 1e9
    in_gbs = nbytes / (in_ms.mean() / 1e3) / 1e9
    gbs = 2 * nbytes / ((out_ms + in_ms).mean() / 1e3) / 1e9
    res = base_record(args, w, K)
    res["metric"] = "pa_swap_out + pa_swap_in GB/s per direction (pinned host), 70B layer pool"
    res.update({"value": round(gbs, 2), "ms_per_step": round(float((out_ms + in_ms).mean()), 4)})
    res["config"].update({"workload": args.workload, "blocks": n, "block_bytes_per_cache": block_bytes,
                          "bytes_per_direction": nbytes, "partition_tokens": 0})
    res.update({
        "swap_out": {"ms": round(float(out_ms.mean()), 4), "gbs": round(out_gbs, 2)},
        "swap_in": {"ms": round(float(in_ms.mean()), 4), "gbs": round(in_gbs, 2)},
        "overlap": {"decode_alone_us": round(float(dec_alone.mean()) * 1e3, 2),
                    "decode_with_swap_us": round(float(dec_busy.mean()) * 1e3, 2),
                    "swap_beside_decode_ms": round(float(swap_busy.mean()), 4)},
        "roofline": {"bound": "host_link", "achieved": round(gbs, 2), "peak": HOST_LINK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HOST_LINK_GBS, 4), "traffic": None,
                     "kernel": "move_blocks_kernel on a capped grid (pa_swap_out / pa_swap_in are one launch each)",
                     "bytes_per_launch": nbytes},
    })
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama70b_layer_bs64", choices=sorted(WORKLOADS))
    ap.add_argument("--no-scrub", action="store_true", help="do not read 512 MiB between steps")
    ap.add_argument("--skip-cpu", action="store_true", help="do not time the CPU oracle")
    ap.add_argument("--partition-tokens", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()
    if args.workload == "fp8_80layer_bs128":
        res = bench_model_step(args, dev)
    elif args.workload == "copy_blocks_llama70b":
        res = bench_copy_blocks(args, dev)
    elif args.workload == "swap_blocks_llama70b":
        res = bench_swap(args, dev)
    elif args.workload.startswith("quest_"):
        res = bench_quest(args, dev)
    elif args.workload == "cascade_prefix_shared_bs256":
        res = bench_cascade(args, dev)
    elif args.workload == "bulk_write_llama70b":
        res = bench_bulk_write(args, dev)
    else:
        res = bench_layer(args, dev)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
