"""Benchmark: paged-attention decode on a Llama-70B-shaped layer, batch 64.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-scrub] [--skip-cpu]

One step = the whole hot path over one batch: pa_cache_write of the 64 new
tokens (one per sequence) into their slots, then pa_decode of the 64
sequences (64 query heads, 8 KV heads, head_dim 128, bf16 KV cache, block
size 16, lognormal lengths with median 2,400 and p95 about 18,000 clipped to
[16, 32768]).  Inputs are synthetic and already resident in HBM.

Before every timed step a 512 MiB buffer is read (a reduction) so the KV
blocks of the previous step are not served from the 256 MiB Infinity Cache
(a read leaves clean lines, so the decode pays no write-back for the scrub);
the write and the decode are each bracketed by HIP events recorded on the
stream they run on, so the scrub is not timed.  `value` is KV bytes read per
decode call (sum of sequence lengths x 2 x 8 heads x 128 x 2 B) divided by
the mean event-timed duration of pa_decode, in GB/s (1e9 B/s).

Prints exactly one JSON line on stdout; everything else goes to stderr.
"""

import argparse
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

METRIC = "paged-decode KV GB/s (% of HBM peak) + decode tok/s, 70B-shaped layer, bs=64"
HBM_PEAK_GBS = 8000.0
MODEL_LAYERS = 80
SCRUB_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w):
    """Bytes one decode call must move at minimum: K and V of every cached
    token, the queries, the outputs, the block-table entries and lengths."""
    S, Hq, D = w.num_seqs, w.num_q_heads, w.head_dim
    kv = w.logical_kv_bytes()
    tables = int(sum(-(-int(L) // w.block_size) for L in w.seq_lens)) * 4
    other = S * Hq * D * 2 + S * Hq * D * 4 + tables + 4 * S
    return kv, kv + other


KERNEL_SOURCES = ("paged_kv_cache_32_amd/csrc/decode.hip", "paged_kv_cache_32_amd/csrc/pa_internal.h",
                  "paged_kv_cache_32_amd/csrc/api.hip")
TRAFFIC_PROFILE = "profiles/decode_kernel_llama70b_bs64_traffic.md"


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, or None when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(w, t, out_gpu, min_seconds=10.0, max_seconds=30.0):
    """Time the CPU oracle (float64 numpy) on the same batch: whole-batch
    passes repeated until about 10 s have elapsed; also report its agreement
    with the GPU output on that batch."""
    from threadpoolctl import threadpool_info

    from oracle import paged
    g = paged.Geom(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)

    def bits(x):
        return x.detach().cpu().view(torch.int16).numpy().view(np.uint16)

    kc, vc, q = bits(t["k_cache"][0]), bits(t["v_cache"][0]), bits(t["q"][0])
    # The oracle's own write of this step's tokens: every slot the kernels
    # wrote is overwritten with the oracle's encoding; all other slots still
    # hold the generator's values.
    paged.cache_write_bf16(g, bits(t["k_new"][0]), bits(t["v_new"][0]), w.slot_mapping, kc, vc)
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    passes, elapsed, ref = 0, 0.0, None
    seqs = list(range(w.num_seqs))
    while elapsed < min_seconds and elapsed < max_seconds:
        t0 = time.perf_counter()
        ref = paged.decode(g, q, kc, vc, w.block_tables, w.seq_lens, w.scale, seqs=seqs)
        elapsed += time.perf_counter() - t0
        passes += 1
        if passes * (elapsed / passes) > max_seconds:
            break
    per_pass = elapsed / passes
    err = np.abs(out_gpu.detach().cpu().double().numpy() - ref)
    kv = w.logical_kv_bytes()
    return {
        "value": kv / per_pass / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"whole {w.num_seqs}-sequence batch of the same workload, float64 numpy oracle, "
                   f"{passes} pass(es) in {elapsed:.1f} s ({per_pass:.2f} s/pass)"),
        "seconds_per_call": per_pass,
        "gpu_vs_oracle_max_abs": float(err.max()), "gpu_vs_oracle_mean_abs": float(err.mean()),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-scrub", action="store_true", help="do not overwrite 512 MiB between steps")
    ap.add_argument("--skip-cpu", action="store_true", help="do not time the CPU oracle")
    ap.add_argument("--partition-tokens", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()

    w = W.config(2)
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

    def step():
        pa.pa_cache_write(kn, vn, sm, kc, vc, block_size=w.block_size)
        pa.pa_decode(q, kc, vc, bt, sl, w.scale, out, num_kv_heads=w.num_kv_heads,
                     block_size=w.block_size, partition_tokens=args.partition_tokens, workspace=ws)

    for i in range(args.warmup):
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=sink)
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if not args.no_scrub:
            torch.sum(scrub, dim=0, out=sink)
        ev[i][0].record(stream)
        pa.pa_cache_write(kn, vn, sm, kc, vc, block_size=w.block_size)
        ev[i][1].record(stream)
        pa.pa_decode(q, kc, vc, bt, sl, w.scale, out, num_kv_heads=w.num_kv_heads,
                     block_size=w.block_size, partition_tokens=args.partition_tokens, workspace=ws)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])

    # Hot-cache reference: the same decode back to back with no scrub.
    hot = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    hot[0].record(stream)
    for _ in range(K):
        pa.pa_decode(q, kc, vc, bt, sl, w.scale, out, num_kv_heads=w.num_kv_heads,
                     block_size=w.block_size, partition_tokens=args.partition_tokens, workspace=ws)
    hot[1].record(stream)
    torch.cuda.synchronize()
    hot_ms = hot[0].elapsed_time(hot[1]) / K

    kv_bytes, alg_bytes = algorithmic_bytes(w)
    dec_s = float(dec_ms.mean()) / 1e3
    step_ms = float((write_ms + dec_ms).mean())
    kv_gbs = kv_bytes / dec_s / 1e9
    alg_gbs = alg_bytes / dec_s / 1e9
    res = {
        "metric": METRIC,
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded lognormal lengths, N(0,1) bf16 q/k/v, shuffled block pool)",
        "config": {"workload": "llama70b_layer_bs64", "num_seqs": w.num_seqs,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "kv_dtype": "bf16",
                   "tokens": int(w.seq_lens.sum()), "kv_bytes_per_call": kv_bytes,
                   "partition_tokens": args.partition_tokens, "scrub_mib_between_steps":
                       0 if args.no_scrub else SCRUB_BYTES >> 20},
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
                     "traffic": measured_traffic(),
                     "kernel": "decode_kernel (pa_decode is one launch)",
                     "bytes_per_launch": alg_bytes},
    }
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_baseline(w, t, out)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
