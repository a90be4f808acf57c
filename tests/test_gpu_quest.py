"""Query-aware page selection on the GPU (include/pa_quest.h) against the
Quest oracle: summaries kept by the writes and recomputed summaries (exact),
the chosen pages (bit-exact tables and lengths), and the decode over them
(within the decode tolerances), from the page's own four-page example up to
the full-size long-context and 70B-layer workloads."""

import numpy as np
import pytest
import torch

import paged_kv_cache_32_amd as pa
from oracle import paged
from oracle import quest as Q
from paged_kv_cache_32_amd import workloads as W
from tests.gpu_helpers import compare, device_inputs, gpu_write, host_bits, oracle_caches

pytestmark = pytest.mark.gpu


def bf16_bits(x):
    f = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def words_to_values(words):
    """Summary words (int32 device tensor, [blocks, D / 4, Hkv, 4] as
    include/pa_quest.h lays them out) -> (min, max) float64 arrays
    [blocks, Hkv, D], the oracle's order."""
    u = words.cpu().numpy().view(np.uint32)
    nb, q4, hkv, _ = u.shape
    u = u.transpose(0, 2, 1, 3).reshape(nb, hkv, 4 * q4)
    return (paged.bf16_bits_to_f64((u & 0xFFFF).astype(np.uint16)),
            paged.bf16_bits_to_f64((u >> 16).astype(np.uint16)))


def seq_items(w):
    """(block, token count) of every block the batch's sequences hold."""
    items = {}
    for s, L in enumerate(w.seq_lens):
        L = int(L)
        for p in range(-(-L // w.block_size)):
            items[int(w.block_tables[s, p])] = min(w.block_size, L - p * w.block_size)
    return sorted(items.items())


def kw(w):
    return dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size)


def test_page_example_on_the_gpu(pages):
    """The four-page example ("KV Cache Engineering for LLM Serving",
    section 7) written through pa_cache_write and pa_quest_update: pages 1 and
    2 are chosen, and the decode attends to their tokens only."""
    c = pages["quest_example"]
    keys = np.array(c["pages"], dtype=np.float64)
    BS, D = 16, 64
    table = [4, 0, 5, 2]
    L = 4 * BS
    K = np.zeros((L, 1, D))
    for p in range(4):
        for t in range(BS):
            K[p * BS + t, 0, :2] = keys[p, t % 2]
    V = np.random.default_rng(1).standard_normal((L, 1, D))
    kb, vb = bf16_bits(K), bf16_bits(V)
    g = paged.Geom(num_blocks=6, block_size=BS, num_kv_heads=1, head_dim=D)
    kc = torch.zeros(g.cache_elems, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    slots = torch.tensor([table[i // BS] * BS + i % BS for i in range(L)], dtype=torch.int64, device="cuda")
    to_dev = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).cuda()
    pa.pa_cache_write(to_dev(kb), to_dev(vb), slots, kc, vc, block_size=BS)
    summ = pa.quest_summaries(kc, num_kv_heads=1, head_dim=D, block_size=BS)
    pa.pa_quest_update(kc, slots, summ, num_kv_heads=1, head_dim=D, block_size=BS)
    q = np.zeros((1, 1, D))
    q[0, 0, :2] = c["query"]
    qd = to_dev(bf16_bits(q))
    bt = torch.tensor([table], dtype=torch.int32, device="cuda")
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    st, sn = pa.pa_quest_select(qd, summ, bt, sl, c["keep"], num_kv_heads=1, block_size=BS)
    out = pa.pa_decode_quest(qd, kc, vc, st, sn, 0.5, num_kv_heads=1, block_size=BS)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [[table[p] for p in c["selected"]]]
    assert sn.cpu().tolist() == [len(c["selected"]) * BS]
    rows = [p * BS + t for p in c["selected"] for t in range(BS)]
    ref = paged.dense_attention(paged.bf16_bits_to_f64(bf16_bits(q))[0], paged.bf16_bits_to_f64(kb)[rows],
                                paged.bf16_bits_to_f64(vb)[rows], 0.5)
    compare(out, ref[None], "bf16", label="page example")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_summaries_kept_by_the_writes(kv_dtype):
    """A stream of prefill writes (many tokens per block, shuffled, with
    padding and out-of-pool slots) and decode writes over a pool whose blocks
    are freed and reused: after every step the GPU summaries equal the
    oracle's write-maintained ones, value for value."""
    rng = np.random.default_rng(2)
    BS, D, Hkv = 16, 128, 2
    g = paged.Geom(num_blocks=24, block_size=BS, num_kv_heads=Hkv, head_dim=D, kv_dtype=kv_dtype)
    ks, vs = np.float32(2.0 / 448), np.float32(1.5 / 448)
    if kv_dtype == "bf16":
        kc0 = bf16_bits(rng.standard_normal(g.cache_elems) * 5)
        kc = torch.from_numpy(kc0.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        kc0 = rng.integers(0, 126, g.cache_elems).astype(np.uint8)
        kc = torch.from_numpy(kc0.copy()).cuda()
    vc = torch.zeros_like(kc)
    k_ref, v_ref = kc0.copy(), host_bits(vc).copy()
    summ = pa.quest_summaries(kc, num_kv_heads=Hkv, head_dim=D, block_size=BS)
    mn, mx = Q.empty_summaries(g)
    free, seqs = list(range(g.num_blocks)), {}
    for step in range(40):
        slots = []
        if not seqs or rng.random() < 0.3:
            L = int(rng.integers(1, 60))
            nb = -(-L // BS)
            if nb <= len(free):
                table = [free.pop(0) for _ in range(nb)]
                seqs[step] = [table, L]
                slots = [table[i // BS] * BS + i % BS for i in range(L)]
        elif rng.random() < 0.2:
            s = list(seqs)[int(rng.integers(len(seqs)))]
            free.extend(seqs.pop(s)[0])
        else:
            for s, (table, L) in list(seqs.items()):
                if L % BS == 0:
                    if not free:
                        continue
                    table.append(free.pop(0))
                slots.append(table[L // BS] * BS + L % BS)
                seqs[s][1] = L + 1
        for _ in range(int(rng.integers(0, 3))):
            slots.insert(int(rng.integers(len(slots) + 1)), int(rng.choice([-1, g.num_blocks * BS])))
        rng.shuffle(slots)
        if not slots:
            continue
        T = len(slots)
        kn = bf16_bits(rng.standard_normal((T, Hkv, D)) * rng.uniform(0.2, 2))
        vn = bf16_bits(rng.standard_normal((T, Hkv, D)))
        sd = torch.tensor(slots, dtype=torch.int64, device="cuda")
        to_dev = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).cuda()
        if kv_dtype == "bf16":
            pa.pa_cache_write(to_dev(kn), to_dev(vn), sd, kc, vc, block_size=BS)
            paged.cache_write_bf16(g, kn, vn, slots, k_ref, v_ref)
        else:
            pa.pa_cache_write_fp8(to_dev(kn), to_dev(vn), sd, kc, vc, float(ks), float(vs), block_size=BS)
            paged.cache_write_fp8(g, kn, vn, slots, k_ref, v_ref, ks, vs)
        pa.pa_quest_update(kc, sd, summ, num_kv_heads=Hkv, head_dim=D, block_size=BS)
        Q.update_summaries(g, k_ref, slots, mn, mx)
        torch.cuda.synchronize()
        gm, gx = words_to_values(summ)
        assert np.array_equal(gm, mn) and np.array_equal(gx, mx), step


@pytest.mark.parametrize("kv_dtype,block_size", [("bf16", 16), ("fp8", 16), ("bf16", 48)])
def test_summaries_kept_by_the_fused_write(kv_dtype, block_size):
    """pa_quest_cache_write(_fp8): sequences start with a prompt (several
    tokens per block: pa_cache_write + pa_quest_update), then grow by one
    token per step through the fused write, crossing block boundaries (a
    token at offset 0 restarts its block's summary), while others end and
    their blocks are reused; padding and out-of-pool slots are mixed in.
    After every step the caches equal the oracle's write bit for bit and the
    summaries equal the oracle's write-maintained ones value for value."""
    rng = np.random.default_rng(3)
    BS, D, Hkv = block_size, 128, 4
    g = paged.Geom(num_blocks=40, block_size=BS, num_kv_heads=Hkv, head_dim=D, kv_dtype=kv_dtype)
    ks, vs = np.float32(2.0 / 448), np.float32(1.5 / 448)
    if kv_dtype == "bf16":
        kc0 = bf16_bits(rng.standard_normal(g.cache_elems) * 5)
        kc = torch.from_numpy(kc0.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        kc0 = rng.integers(0, 126, g.cache_elems).astype(np.uint8)
        kc = torch.from_numpy(kc0.copy()).cuda()
    vc = torch.zeros_like(kc)
    k_ref, v_ref = kc0.copy(), host_bits(vc).copy()
    summ = pa.quest_summaries(kc, num_kv_heads=Hkv, head_dim=D, block_size=BS)
    mn, mx = Q.empty_summaries(g)
    free, seqs = list(range(g.num_blocks)), {}
    to_dev = lambda b: torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).cuda()
    fused_steps = 0
    for step in range(60):
        prompt = not seqs or rng.random() < 0.15
        slots = []
        if prompt:
            L = int(rng.integers(1, 3 * BS))
            nb = -(-L // BS)
            if nb > len(free):
                continue
            table = [free.pop(0) for _ in range(nb)]
            seqs[step] = [table, L]
            slots = [table[i // BS] * BS + i % BS for i in range(L)]
        elif rng.random() < 0.15:
            s = list(seqs)[int(rng.integers(len(seqs)))]
            free.extend(seqs.pop(s)[0])
            continue
        else:
            for s, (table, L) in list(seqs.items()):
                if L % BS == 0:
                    if not free:
                        continue
                    table.append(free.pop(0))
                slots.append(table[L // BS] * BS + L % BS)
                seqs[s][1] = L + 1
            for _ in range(int(rng.integers(0, 3))):
                slots.insert(int(rng.integers(len(slots) + 1)), int(rng.choice([-1, g.num_blocks * BS])))
        if not slots:
            continue
        T = len(slots)
        kn = bf16_bits(rng.standard_normal((T, Hkv, D)) * rng.uniform(0.2, 2))
        vn = bf16_bits(rng.standard_normal((T, Hkv, D)))
        if rng.random() < 0.1:
            kn[0, 0, :7] = 0x7FC0                    # NaN keys: ignored by the summaries
        sd = torch.tensor(slots, dtype=torch.int64, device="cuda")
        if kv_dtype == "bf16":
            paged.cache_write_bf16(g, kn, vn, slots, k_ref, v_ref)
        else:
            paged.cache_write_fp8(g, kn, vn, slots, k_ref, v_ref, ks, vs)
        if prompt:
            if kv_dtype == "bf16":
                pa.pa_cache_write(to_dev(kn), to_dev(vn), sd, kc, vc, block_size=BS)
            else:
                pa.pa_cache_write_fp8(to_dev(kn), to_dev(vn), sd, kc, vc, float(ks), float(vs), block_size=BS)
            pa.pa_quest_update(kc, sd, summ, num_kv_heads=Hkv, head_dim=D, block_size=BS)
        else:
            fused_steps += 1
            if kv_dtype == "bf16":
                pa.pa_quest_cache_write(to_dev(kn), to_dev(vn), sd, kc, vc, summ, block_size=BS)
            else:
                pa.pa_quest_cache_write_fp8(to_dev(kn), to_dev(vn), sd, kc, vc, float(ks), float(vs), summ,
                                            block_size=BS)
        Q.update_summaries(g, k_ref, slots, mn, mx)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(kc), k_ref), f"step {step}: K cache"
        assert np.array_equal(host_bits(vc), v_ref), f"step {step}: V cache"
        gm, gx = words_to_values(summ)
        assert np.array_equal(gm, mn) and np.array_equal(gx, mx), f"step {step}: summaries"
    assert fused_steps > 20


@pytest.mark.parametrize("kv_dtype,block_size,head_dim", [("bf16", 16, 128), ("fp8", 32, 64),
                                                          ("bf16", 48, 64), ("fp8", 16, 128)])
def test_recomputed_summaries(kv_dtype, block_size, head_dim):
    rng = np.random.default_rng(3)
    g = paged.Geom(num_blocks=30, block_size=block_size, num_kv_heads=3, head_dim=head_dim, kv_dtype=kv_dtype)
    if kv_dtype == "bf16":
        kc0 = bf16_bits(rng.standard_normal(g.cache_elems))
        kc = torch.from_numpy(kc0.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        kc0 = rng.integers(0, 256, g.cache_elems).astype(np.uint8)
        kc0[(kc0 & 0x7F) == 0x7F] = 0x22
        kc = torch.from_numpy(kc0.copy()).cuda()
    blocks = [3, 17, 0, 29, 8, -1, 30, 12]
    counts = [block_size, 1, 0, 7, block_size + 5, 4, 4, -3]
    summ = pa.quest_summaries(kc, num_kv_heads=3, head_dim=head_dim, block_size=block_size)
    pa.pa_quest_summarize(kc, torch.tensor(blocks, dtype=torch.int32, device="cuda"),
                          torch.tensor(counts, dtype=torch.int32, device="cuda"), summ,
                          num_kv_heads=3, head_dim=head_dim, block_size=block_size)
    torch.cuda.synchronize()
    mn, mx = Q.empty_summaries(g)
    ok = [(b, min(max(c, 0), block_size)) for b, c in zip(blocks, counts) if 0 <= b < g.num_blocks]
    Q.summarize(g, kc0, [b for b, _ in ok], [c for _, c in ok], mn, mx)
    gm, gx = words_to_values(summ)
    assert np.array_equal(gm, mn) and np.array_equal(gx, mx)


def run_select_and_decode(w, t, budget, part=0, label=""):
    """GPU: summaries of the batch's blocks, selection, decode.  Oracle: its
    own summaries of its own caches, selection, decode.  Tables and lengths
    compared exactly, outputs within tolerance."""
    Hkv, BS = w.num_kv_heads, w.block_size
    kc0, vc0 = host_bits(t["k_cache"][0]), host_bits(t["v_cache"][0])
    ks = float(t["k_scale"][0]) if w.kv_dtype == "fp8" else 1.0
    vs = float(t["v_scale"][0]) if w.kv_dtype == "fp8" else 1.0
    gpu_write(w, t)
    kc_ref, vc_ref = oracle_caches(w, kc0, vc0, host_bits(t["k_new"][0]), host_bits(t["v_new"][0]), ks, vs)
    kc, vc, q = t["k_cache"][0], t["v_cache"][0], t["q"][0]
    items = seq_items(w)
    summ = pa.quest_summaries(kc, num_kv_heads=Hkv, head_dim=w.head_dim, block_size=BS)
    pa.pa_quest_summarize(kc, torch.tensor([b for b, _ in items], dtype=torch.int32, device="cuda"),
                          torch.tensor([c for _, c in items], dtype=torch.int32, device="cuda"), summ,
                          num_kv_heads=Hkv, head_dim=w.head_dim, block_size=BS)
    st, sn = pa.pa_quest_select(q, summ, t["block_tables"], t["seq_lens"], budget, **kw(w))
    st2, sn2 = pa.pa_quest_select(q, summ, t["block_tables"], t["seq_lens"], budget, **kw(w))
    if w.kv_dtype == "bf16":
        out = pa.pa_decode_quest(q, kc, vc, st, sn, w.scale, partition_tokens=part, **kw(w))
    else:
        out = pa.pa_decode_quest_fp8(q, kc, vc, st, sn, w.scale, ks, vs, partition_tokens=part, **kw(w))
    torch.cuda.synchronize()
    assert torch.equal(st, st2) and torch.equal(sn, sn2), f"{label}: selection not deterministic"
    g = paged.Geom(w.num_blocks, BS, Hkv, w.head_dim, w.kv_dtype)
    mn, mx = Q.empty_summaries(g)
    Q.summarize(g, kc_ref, [b for b, _ in items], [c for _, c in items], mn, mx)
    gm, gx = words_to_values(summ)
    assert np.array_equal(gm, mn) and np.array_equal(gx, mx), f"{label}: summaries differ"
    qb = host_bits(q)
    ref, chosen = Q.decode(g, qb, kc_ref, vc_ref, w.block_tables, w.seq_lens, mn, mx, budget, w.scale,
                           float(np.float32(ks)), float(np.float32(vs)))
    st_h, sn_h = st.cpu().numpy(), sn.cpu().numpy()
    for s, L in enumerate(w.seq_lens):
        L = int(L)
        for h in range(Hkv):
            u = s * Hkv + h
            ids = [int(w.block_tables[s, p]) for p in chosen[s][h]]
            assert st_h[u, :len(ids)].tolist() == ids, (label, s, h)
            assert (st_h[u, len(ids):] == -1).all() or len(ids) == budget, (label, s, h)
            toks = sum(min(BS, L - p * BS) for p in chosen[s][h])
            assert int(sn_h[u]) == toks, (label, s, h)
    return compare(out, ref, w.kv_dtype, label=label)


CASES = [  # seed, S, Hq, Hkv, D, BS, max_len, kv, budgets
    (1, 10, 64, 8, 128, 16, 900, "bf16", (1, 4, 20, 100)),
    (2, 7, 8, 8, 64, 32, 700, "bf16", (2, 9)),
    (3, 9, 64, 4, 128, 16, 1200, "fp8", (3, 16, 80)),
    (4, 6, 16, 1, 64, 48, 800, "fp8", (1, 5)),
    (5, 5, 12, 4, 128, 16, 2000, "bf16", (7,)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[7]}_g{c[2] // c[3]}_d{c[4]}_bs{c[5]}" for c in CASES])
def test_selection_and_decode_match_the_oracle(case):
    seed, S, Hq, Hkv, D, BS, max_len, kv, budgets = case
    w = W.random_workload(seed, S, Hq, Hkv, D, BS, max_len, kv_dtype=kv, min_len=0)
    print(f"[quest] {w.name} {kv} lens={list(w.seq_lens)}", flush=True)
    for budget in budgets:
        for part in (0, 32):
            t = device_inputs(w)
            run_select_and_decode(w, t, budget, part, label=f"budget={budget} part={part}")


def test_equal_scores_go_to_the_lower_page():
    """Tables that repeat one block (equal summaries, equal scores) choose the
    first pages; a table of distinct blocks with one copied block keeps the
    earlier copy when only one fits."""
    w = W.random_workload(9, 3, 16, 2, 128, 16, 300, min_len=200)
    bt = w.block_tables.copy()
    bt[0, :] = bt[0, 0]                        # every page the same block
    bt[1, 5] = bt[1, 2]                        # pages 2 and 5 equal
    w2 = W.Workload(w.name, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks,
                    w.seq_lens, bt, w.slot_mapping, w.scale, kv_dtype=w.kv_dtype, seed=w.seed)
    for budget in (1, 3):
        t = device_inputs(w2, poison=False)
        run_select_and_decode(w2, t, budget, label=f"ties budget={budget}")


def test_scores_of_both_signs():
    """Pages scoring on both sides of zero: with q >= 0, a block whose K is
    the constant +0.5 scores 0.5 * sum(q) and one at -0.25 scores
    -0.25 * sum(q).  The choice's key range then spans the sign bit (the
    search takes all 32 bits), and the equal scores on either side go to the
    lower pages."""
    w = W.random_workload(21, 3, 16, 2, 128, 16, 640, min_len=500)
    per_block = w.num_kv_heads * w.block_size * w.head_dim
    for budget in (1, 5, 20):
        t = device_inputs(w, poison=False)
        t["q"][0] = t["q"][0].abs()
        kc = t["k_cache"][0]
        for s_, L in enumerate(w.seq_lens):
            for p in range(-(-int(L) // w.block_size)):
                b = int(w.block_tables[s_, p])
                kc[b * per_block:(b + 1) * per_block] = 0.5 if p % 3 == 0 else -0.25
        run_select_and_decode(w, t, budget, label=f"signs budget={budget}")


@pytest.mark.parametrize("budget", [3, 100, 5000])
def test_wide_tables(budget):
    """Tables wider than 2,048 pages take the 1,024-thread choice kernel.
    Sequences 0 and 1 are short (keys held in registers; their rows padded
    with -1); sequence 2 has 13,000 pages (more keys than LDS holds) whose
    table cycles over its own 25-40 blocks, so that equal scores decide at
    the threshold."""
    w0 = W.random_workload(12, 3, 16, 2, 64, 16, 640, min_len=400)
    maxb = 13000
    bt = np.full((3, maxb), -1, dtype=np.int32)
    for s in range(2):
        n = -(-int(w0.seq_lens[s]) // 16)
        bt[s, :n] = w0.block_tables[s, :n]
    n2 = -(-int(w0.seq_lens[2]) // 16)
    bt[2, :] = np.resize(w0.block_tables[2, :n2], maxb)
    lens = w0.seq_lens.copy()
    lens[2] = maxb * 16 - 5
    slots = np.array([int(bt[s, (int(L) - 1) // 16]) * 16 + (int(L) - 1) % 16 for s, L in enumerate(lens)],
                     dtype=np.int64)
    w = W.Workload("wide_tables", 16, 2, 64, 16, w0.num_blocks, lens, bt, slots, w0.scale, seed=12)
    t = device_inputs(w, poison=False)
    print(f"[quest] wide tables budget={budget} lens={list(lens)}", flush=True)
    run_select_and_decode(w, t, budget, label=f"wide budget={budget}")


def test_invalid_and_empty_rows():
    """Length 0 gives zeros, a length past the table gives NaN rows (as
    pa_decode), and neither disturbs the other sequences."""
    w = W.random_workload(6, 4, 16, 2, 64, 16, 200, min_len=50)
    t = device_inputs(w, poison=False)
    lens = t["seq_lens"].clone()
    lens[1] = 0
    lens[2] = w.block_tables.shape[1] * 16 + 1
    summ = pa.quest_summaries(t["k_cache"][0], num_kv_heads=2, head_dim=64, block_size=16)
    st, sn = pa.pa_quest_select(t["q"][0], summ, t["block_tables"], lens, 2, **kw(w))
    out = pa.pa_decode_quest(t["q"][0], t["k_cache"][0], t["v_cache"][0], st, sn, w.scale, **kw(w))
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert (o[1] == 0).all() and np.isnan(o[2]).all() and np.isfinite(o[[0, 3]]).all()
    assert sn.cpu().tolist()[2 * 2:2 * 2 + 2] == [-1, -1]


@pytest.mark.parametrize("cfg,budget,samples", [(4, 256, [(0, 0), (2, 5), (3, 7)]),
                                                (2, 64, [(0, 3), (17, 0), (40, 6), (63, 7)])])
def test_full_size_workloads(cfg, budget, samples):
    """The long-context (4 x 131,072 tokens) and 70B-layer bs=64 workloads at
    full size, in the launch configuration bench.py times: chosen tables and
    lengths exact and outputs within tolerance on sampled (sequence, KV head)
    pairs, which the oracle computes one by one from gathered sequences."""
    w = W.config(cfg)
    t = device_inputs(w, poison=False)
    print(f"[quest] config {cfg} budget {budget}", flush=True)
    gpu_write(w, t)
    kc, vc, q = t["k_cache"][0], t["v_cache"][0], t["q"][0]
    Hkv, BS, G = w.num_kv_heads, w.block_size, w.num_q_heads // w.num_kv_heads
    items = seq_items(w)
    summ = pa.quest_summaries(kc, num_kv_heads=Hkv, head_dim=w.head_dim, block_size=BS)
    pa.pa_quest_summarize(kc, torch.tensor([b for b, _ in items], dtype=torch.int32, device="cuda"),
                          torch.tensor([c for _, c in items], dtype=torch.int32, device="cuda"), summ,
                          num_kv_heads=Hkv, head_dim=w.head_dim, block_size=BS)
    st, sn = pa.pa_quest_select(q, summ, t["block_tables"], t["seq_lens"], budget, **kw(w))
    out = pa.pa_decode_quest(q, kc, vc, st, sn, w.scale, **kw(w))
    torch.cuda.synchronize()
    g = paged.Geom(w.num_blocks, BS, Hkv, w.head_dim, w.kv_dtype)
    kc_h, vc_h = host_bits(kc), host_bits(vc)
    qf = paged.bf16_bits_to_f64(host_bits(q))
    st_h, sn_h, o = st.cpu().numpy(), sn.cpu().numpy(), out.cpu().double().numpy()
    for s, h in samples:
        L = int(w.seq_lens[s])
        row = w.block_tables[s]
        mn, mx = Q.sequence_page_summaries(g, kc_h, row, L, h)
        sc = Q.page_scores(qf[s, h * G:(h + 1) * G].astype(np.float32), mn, mx)
        chosen = Q.select_pages(sc, budget)
        u = s * Hkv + h
        assert st_h[u, :len(chosen)].tolist() == [int(row[p]) for p in chosen], (s, h)
        assert int(sn_h[u]) == sum(min(BS, L - p * BS) for p in chosen), (s, h)
        K, V = paged.gather(g, kc_h, vc_h, row, L, h)
        pos = [p * BS + i for p in chosen for i in range(BS) if p * BS + i < L]
        ref = paged.softmax_attention(qf[s, h * G:(h + 1) * G], K[pos], V[pos], w.scale)
        compare(o[s, h * G:(h + 1) * G], ref, "bf16", label=f"config {cfg} s={s} h={h}")
