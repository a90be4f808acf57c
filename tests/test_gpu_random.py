"""Seeded random cases over the decode paths, against the oracle.

The hand-picked cases elsewhere name the shapes and edge cases one by one;
these draw the combinations from one seeded generator instead: group size,
head size, block size, cache type, lengths (empty rows included), automatic
or fixed partitions, sliding windows over linear and ring tables, Quest
budgets below and above the page counts, and prefix-shared batches of
random pool structure and chunk size.  Every case prints its parameters
before it runs, so a failure names what to rerun."""

import os

import numpy as np
import pytest
import torch

import paged_kv_cache_32_amd as pa
from oracle import paged
from paged_kv_cache_32_amd import workloads as W
from tests.gpu_helpers import compare, device_inputs, geom, gpu_write, host_bits, oracle_caches, step_and_check
from tests.test_gpu_cascade import run as cascade_run
from tests.test_gpu_quest import run_select_and_decode

pytestmark = pytest.mark.gpu


def _draw(seed, n, fn):
    rng = np.random.default_rng(seed)
    return [fn(rng) for _ in range(n)]


def _shape(rng):
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    return dict(Hkv=hkv, Hq=hkv * g, D=int(rng.choice([64, 128])), BS=int(rng.choice([16, 32, 48, 64])),
                kv=str(rng.choice(["bf16", "fp8"])), seed=int(rng.integers(0, 1 << 30)))


def _decode_case(rng):
    c = _shape(rng)
    c.update(S=int(rng.integers(1, 24)), max_len=int(rng.choice([20, 300, 1500, 5000])),
             part=int(rng.choice([0, 0, 16, 48, 256])), min_len=int(rng.choice([0, 1])))
    return c


def _window_case(rng):
    c = _shape(rng)
    c.update(S=int(rng.integers(1, 24)), max_len=int(rng.choice([16, 200, 1500, 6000])),
             part=int(rng.choice([0, 0, 16, 128])), win=int(rng.choice([1, 15, 16, 100, 1000])))
    return c


def _quest_case(rng):
    c = _shape(rng)
    c.update(S=int(rng.integers(1, 8)), max_len=int(rng.choice([16, 300, 3000, 12000])),
             budget=int(rng.choice([1, 2, 3, 8, 31, 64, 200])), part=int(rng.choice([0, 0, 32])))
    return c


def _cascade_case(rng):
    c = _shape(rng)
    lo = int(rng.integers(10, 200))
    c.update(S=int(rng.integers(2, 40)), system=int(rng.choice([c["BS"], 50, 100, 300])),
             pools=int(rng.integers(1, 5)), prange=(lo, lo + int(rng.integers(0, 400))),
             med=float(rng.choice([5, 20, 60, 200])), chunk=c["BS"] * int(rng.choice([1, 2, 3, 4, 8, 32])),
             part=int(rng.choice([0, 0, 32, 128])))
    return c


# PA_RANDOM_SCALE=k draws k times as many cases from the same generators
# (the first ones are always the default run's), for longer sweeps.
SCALE = max(1, int(os.environ.get("PA_RANDOM_SCALE", "1")))
DECODE = _draw(101, 24 * SCALE, _decode_case)
WINDOW = _draw(102, 16 * SCALE, _window_case)
QUEST = _draw(103, 10 * SCALE, _quest_case)
CASCADE = _draw(104, 10 * SCALE, _cascade_case)


def _label(kind, i, c):
    return f"[random {kind} {i}] " + " ".join(f"{k}={v}" for k, v in c.items())


@pytest.mark.parametrize("i", range(len(DECODE)))
def test_random_decode(i):
    """Write the new tokens, decode (automatic split or fixed partitions):
    caches bit for bit, outputs against the oracle."""
    c = DECODE[i]
    label = _label("decode", i, c)
    print(label, flush=True)
    w = W.random_workload(c["seed"], c["S"], c["Hq"], c["Hkv"], c["D"], c["BS"], c["max_len"], kv_dtype=c["kv"],
                          min_len=c["min_len"])
    step_and_check(w, device_inputs(w), partition_tokens=c["part"], label=label)


@pytest.mark.parametrize("i", range(len(WINDOW)))
def test_random_window_and_ring(i):
    """Window decode over the linear tables against the oracle; the ring
    tables holding the same blocks give the same output bit for bit."""
    c = WINDOW[i]
    label = _label("window", i, c)
    print(label, flush=True)
    w = W.random_workload(c["seed"], c["S"], c["Hq"], c["Hkv"], c["D"], c["BS"], c["max_len"], kv_dtype=c["kv"],
                          min_len=1)
    t = device_inputs(w)
    kc0, vc0 = host_bits(t["k_cache"][0]), host_bits(t["v_cache"][0])
    fp8 = c["kv"] == "fp8"
    ks = float(t["k_scale"][0]) if fp8 else 1.0
    vs = float(t["v_scale"][0]) if fp8 else 1.0
    gpu_write(w, t)
    kc_ref, vc_ref = oracle_caches(w, kc0, vc0, host_bits(t["k_new"][0]), host_bits(t["v_new"][0]), ks, vs)
    win, BS = c["win"], c["BS"]
    ref = paged.decode(geom(w), host_bits(t["q"][0]), kc_ref, vc_ref, w.block_tables, w.seq_lens, w.scale,
                       k_scale=ks, v_scale=vs, window=win)
    kc, vc = t["k_cache"][0], t["v_cache"][0]
    kw = dict(num_kv_heads=c["Hkv"], block_size=BS, partition_tokens=c["part"])
    scales = (ks, vs) if fp8 else ()
    lin_fn = pa.pa_decode_window_fp8 if fp8 else pa.pa_decode_window
    ring_fn = pa.pa_decode_ring_fp8 if fp8 else pa.pa_decode_ring
    lin = lin_fn(t["q"][0], kc, vc, t["block_tables"], t["seq_lens"], win, w.scale, *scales, **kw)
    E = -(-win // BS) + 1
    rt = np.full((w.num_seqs, E), -1, dtype=np.int32)
    for s, L in enumerate(w.seq_lens):
        for b in range(max(0, int(L) - win) // BS, -(-int(L) // BS)):
            rt[s, b % E] = w.block_tables[s, b]
    ring = ring_fn(t["q"][0], kc, vc, torch.from_numpy(rt).cuda(), t["seq_lens"], win, w.scale, *scales, **kw)
    torch.cuda.synchronize()
    compare(lin, ref, c["kv"], label=label)
    assert torch.equal(ring.view(torch.int32), lin.view(torch.int32)), f"{label}: ring differs from linear"


@pytest.mark.parametrize("i", range(len(QUEST)))
def test_random_quest(i):
    """Summaries, chosen tables and lengths bit for bit; the decode over the
    chosen pages against the oracle's."""
    c = QUEST[i]
    label = _label("quest", i, c)
    print(label, flush=True)
    w = W.random_workload(c["seed"], c["S"], c["Hq"], c["Hkv"], c["D"], c["BS"], c["max_len"], kv_dtype=c["kv"],
                          min_len=0)
    run_select_and_decode(w, device_inputs(w), c["budget"], c["part"], label=label)


@pytest.mark.parametrize("i", range(len(CASCADE)))
def test_random_cascade(i):
    """Prefix-shared batches of random pool structure through the cascade,
    against the oracle's plain decode."""
    c = CASCADE[i]
    label = _label("cascade", i, c)
    print(label, flush=True)
    w = W.prefix_shared(seed=c["seed"], num_seqs=c["S"], block_size=c["BS"], system_tokens=c["system"],
                        num_pools=c["pools"], pool_range=c["prange"], suffix_median=c["med"], max_len=3000,
                        num_q_heads=c["Hq"], num_kv_heads=c["Hkv"], head_dim=c["D"], kv_dtype=c["kv"])
    cascade_run(w, device_inputs(w), c["chunk"], c["part"], label=label)
