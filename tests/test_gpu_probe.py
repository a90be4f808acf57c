"""Read probes on the GPU (include/pa_probe.h): each returns the XOR of every
32-bit word it read, which is checked here against the same XOR taken with
numpy over the bytes the probe is defined to read (the generator's caches,
not anything the kernels wrote)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_32_amd as pa
from paged_kv_cache_32_amd import workloads as W
from tests.gpu_helpers import device_inputs

pytestmark = pytest.mark.gpu


def xor_words(a):
    a = np.ascontiguousarray(a).view(np.uint32)
    return int(np.bitwise_xor.reduce(a)) if a.size else 0


def sink_value(sink):
    return int(sink.cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 1040])
def test_stream_read_reads_every_word_once(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.cuda()
    sink = pa.pa_probe_stream_read(buf)
    torch.cuda.synchronize()
    assert sink_value(sink) == xor_words(host.numpy())


def expected_tile_xor(w, kc, vc, bt, lens, window=0):
    """XOR over the K and V tiles (16 tokens) covering [0, L) of every valid
    (sequence, head), or [L - window, L) when L > window > 0, through the
    tables; block ids outside the pool skip."""
    eb = 1 if w.kv_dtype == "fp8" else 2
    words = 16 * w.head_dim * eb // 4
    subs = w.block_size // 16
    shape = (w.num_blocks, w.num_kv_heads, subs, words)
    per_tile = (np.bitwise_xor.reduce(np.ascontiguousarray(kc).view(np.uint32).reshape(shape), axis=-1)
                ^ np.bitwise_xor.reduce(np.ascontiguousarray(vc).view(np.uint32).reshape(shape), axis=-1))
    maxb = bt.shape[1]
    x = np.uint32(0)
    for s, L in enumerate(lens):
        if not 1 <= L <= maxb * w.block_size:
            continue
        c0 = (int(L) - window) // 16 if 0 < window < int(L) else 0
        t = np.arange(c0, -(-int(L) // 16))
        blk = bt[s, t // subs].astype(np.int64)
        keep = (blk >= 0) & (blk < w.num_blocks)
        sel = per_tile[blk[keep], :, (t % subs)[keep]]        # [tiles, heads]
        if sel.size:
            x ^= np.bitwise_xor.reduce(sel.reshape(-1))
    return int(x)


CASES = [  # seed, S, Hkv, D, BS, max_len, kv
    (1, 7, 2, 128, 16, 300, "bf16"),
    (2, 9, 4, 64, 32, 500, "bf16"),
    (3, 6, 1, 128, 48, 260, "fp8"),
    (4, 11, 8, 64, 16, 200, "fp8"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[6]}_d{c[3]}_bs{c[4]}" for c in CASES])
def test_tile_read_reads_the_decode_tiles(case):
    seed, S, Hkv, D, BS, max_len, kv = case
    w = W.random_workload(seed, S, Hkv * 2, Hkv, D, BS, max_len, kv_dtype=kv, min_len=1)
    t = device_inputs(w, poison=False)
    kc, vc = t["k_cache"][0], t["v_cache"][0]
    bt, lens = w.block_tables.copy(), w.seq_lens.copy()
    lens[0] = 0                                   # empty: nothing read
    lens[1] = bt.shape[1] * BS + 1                # past the table: nothing read
    bt[2, 0] = w.num_blocks + 5                   # outside the pool: that block skipped
    sink = pa.pa_probe_tile_read(kc, vc, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                 num_kv_heads=Hkv, head_dim=D, block_size=BS)
    torch.cuda.synchronize()
    kb, vb = kc.cpu(), vc.cpu()
    if kv == "bf16":
        kb, vb = kb.view(torch.int16), vb.view(torch.int16)
    want = expected_tile_xor(w, kb.numpy(), vb.numpy(), bt, lens)
    print(f"[probe] {kv} D={D} BS={BS} lens={list(lens)}", flush=True)
    assert sink_value(sink) == want


@pytest.mark.parametrize("window", [1, 16, 40, 100])
def test_tile_read_window(window):
    """With a window only the tiles of the last `window` tokens are read; the
    table entries before them are set to -1 (as after pa_bm_trim) and must
    not be read."""
    w = W.random_workload(9, 8, 8, 2, 128, 16, 400, min_len=1)
    t = device_inputs(w, poison=False)
    kc, vc = t["k_cache"][0], t["v_cache"][0]
    bt, lens = w.block_tables.copy(), w.seq_lens.copy()
    for s, L in enumerate(lens):
        if L > window:
            bt[s, :(int(L) - window) // w.block_size] = -1
    sink = pa.pa_probe_tile_read(kc, vc, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                 num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, block_size=w.block_size,
                                 window=window)
    torch.cuda.synchronize()
    kb, vb = kc.cpu().view(torch.int16).numpy(), vc.cpu().view(torch.int16).numpy()
    print(f"[probe] window {window} lens={list(lens)}", flush=True)
    assert sink_value(sink) == expected_tile_xor(w, kb, vb, bt, lens, window)


def test_tile_read_full_size_workload():
    """The 70B-shaped layer at bs=64, as bench.py reads it."""
    w = W.config(2)
    t = device_inputs(w, poison=False)
    sink = pa.pa_probe_tile_read(t["k_cache"][0], t["v_cache"][0], t["block_tables"], t["seq_lens"],
                                 num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, block_size=w.block_size)
    torch.cuda.synchronize()
    kb = t["k_cache"][0].cpu().view(torch.int16).numpy()
    vb = t["v_cache"][0].cpu().view(torch.int16).numpy()
    assert sink_value(sink) == expected_tile_xor(w, kb, vb, w.block_tables, w.seq_lens)
