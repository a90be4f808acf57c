"""The shared-prefix (cascade) decode and the query-aware (Quest) step
captured as HIP graphs (torch's CUDAGraph) and replayed several times, with
unrelated eager work and synchronisations between replays: every replay
must reproduce the eager result bit for bit.  Neither path allocates or
issues a memset, and both re-arm the decode workspace's counters."""

import pytest
import torch

import paged_kv_cache_32_amd as pa
from paged_kv_cache_32_amd import workloads as W
from tests.gpu_helpers import device_inputs

pytestmark = pytest.mark.gpu


def replay_and_check(fn, out, label):
    fn()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        out.fill_(float("nan"))
        scratch.mul_(1.0001).add_(1.0)            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"{label}: replay {r} differs"
    return eager


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_cascade_graph_replays(kv):
    w = W.prefix_shared(seed=21, num_seqs=20, block_size=16, system_tokens=96, num_pools=2, pool_range=(48, 160),
                        suffix_median=40, max_len=900, num_q_heads=32, num_kv_heads=4, head_dim=128, kv_dtype=kv)
    t = device_inputs(w, poison=False)
    plan = pa.CascadePlan(w.block_tables, w.seq_lens, block_size=w.block_size, num_kv_heads=w.num_kv_heads,
                          num_q_heads=w.num_q_heads, chunk_tokens=64)
    q, kc, vc = t["q"][0], t["k_cache"][0], t["v_cache"][0]
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    need = pa.lib().pa_decode_cascade_workspace_size(
        pa.make_desc(kc, w.num_kv_heads, w.head_dim, w.block_size), w.num_seqs, w.num_q_heads, plan.max_blocks,
        plan.info["num_slots"], 32)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    kw = dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, partition_tokens=32, workspace=ws, out=out)
    print(f"[graph] cascade {kv}: {plan.info['num_segments']} segments, {plan.info['num_items']} items",
          flush=True)
    if kv == "bf16":
        fn = lambda: pa.pa_decode_cascade(q, kc, vc, plan, w.scale, **kw)
    else:
        ks, vs = float(t["k_scale"][0]), float(t["v_scale"][0])
        fn = lambda: pa.pa_decode_cascade_fp8(q, kc, vc, plan, w.scale, ks, vs, **kw)
    eager = replay_and_check(fn, out, f"cascade {kv}")
    plain = pa.pa_decode(q, kc, vc, t["block_tables"], t["seq_lens"], w.scale, num_kv_heads=w.num_kv_heads,
                         block_size=w.block_size) if kv == "bf16" else None
    if plain is not None:
        torch.cuda.synchronize()
        assert float((eager - plain).abs().max()) < 1e-4


def test_quest_graph_replays():
    w = W.random_workload(seed=31, num_seqs=6, num_q_heads=32, num_kv_heads=4, head_dim=128, block_size=16,
                          max_len=2500, min_len=1)
    t = device_inputs(w, poison=False)
    kc, vc, q = t["k_cache"][0], t["v_cache"][0], t["q"][0]
    Hkv, D, BS = w.num_kv_heads, w.head_dim, w.block_size
    summ = pa.quest_summaries(kc, num_kv_heads=Hkv, head_dim=D, block_size=BS)
    items = {}
    for s, L in enumerate(w.seq_lens):
        for pg in range(-(-int(L) // BS)):
            items[int(w.block_tables[s, pg])] = min(BS, int(L) - pg * BS)
    pa.pa_quest_summarize(kc, torch.tensor(list(items), dtype=torch.int32, device="cuda"),
                          torch.tensor(list(items.values()), dtype=torch.int32, device="cuda"), summ,
                          num_kv_heads=Hkv, head_dim=D, block_size=BS)
    budget = 12
    lib, desc = pa.lib(), pa.make_desc(kc, Hkv, D, BS)
    sel_ws = torch.empty(lib.pa_quest_select_workspace_size(w.num_seqs, Hkv, w.block_tables.shape[1]),
                         dtype=torch.uint8, device="cuda")
    dec_ws = torch.zeros(lib.pa_decode_quest_workspace_size(desc, w.num_seqs, w.num_q_heads, budget, 0),
                         dtype=torch.uint8, device="cuda")
    sel_t, sel_l = pa.pa_quest_select(q, summ, t["block_tables"], t["seq_lens"], budget, num_kv_heads=Hkv,
                                      block_size=BS, workspace=sel_ws)
    out = torch.empty((w.num_seqs, w.num_q_heads, D), dtype=torch.float32, device="cuda")

    def step():
        pa.pa_quest_select(q, summ, t["block_tables"], t["seq_lens"], budget, num_kv_heads=Hkv, block_size=BS,
                           sel_tables=sel_t, sel_lens=sel_l, workspace=sel_ws)
        pa.pa_decode_quest(q, kc, vc, sel_t, sel_l, w.scale, out, num_kv_heads=Hkv, block_size=BS,
                           workspace=dec_ws)
    print(f"[graph] quest: lens={list(w.seq_lens)}", flush=True)
    replay_and_check(step, out, "quest")
