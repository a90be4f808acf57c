"""pa_copy_blocks on the GPU, and decode steps whose block tables, slots and
copy-on-write copies come from the native block manager.  The expected
values come from the oracle alone: its own block-manager model, driven with
the same operations (its tables are also checked equal to the native ones),
its block copy, its cache write and its decode."""

import numpy as np
import pytest
import torch

import paged_kv_cache_32_amd as pa
from oracle import blocks as B
from oracle import paged
from tests.gpu_helpers import BF16_ENVELOPE, BF16_TOL, host_bits

pytestmark = pytest.mark.gpu


def random_cache(g, dtype, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    if dtype == "bf16":
        x = torch.randn(g.cache_elems, generator=gen, device="cuda").to(torch.bfloat16)
    else:
        x = torch.randint(0, 256, (g.cache_elems,), generator=gen, device="cuda", dtype=torch.int32).to(torch.uint8)
    return x


@pytest.mark.parametrize("kv_dtype,block_size,head_dim,hkv", [("bf16", 16, 128, 8), ("fp8", 32, 64, 2),
                                                               ("bf16", 48, 64, 3)])
def test_copy_blocks_bit_exact(kv_dtype, block_size, head_dim, hkv):
    g = paged.Geom(num_blocks=40, block_size=block_size, num_kv_heads=hkv, head_dim=head_dim,
                   kv_dtype=kv_dtype)
    kc, vc = random_cache(g, kv_dtype, 1), random_cache(g, kv_dtype, 2)
    rng = np.random.default_rng(3)
    perm = rng.permutation(g.num_blocks)
    pairs = [(int(perm[i]), int(perm[20 + i])) for i in range(13)]          # independent pairs
    pairs += [(-1, 3), (2, g.num_blocks), (g.num_blocks + 5, 1)]            # skipped
    k_ref, v_ref = host_bits(kc).copy(), host_bits(vc).copy()
    E = hkv * block_size * head_dim
    B.copy_blocks(k_ref, v_ref, pairs[:13], E)
    pa.pa_copy_blocks(kc, vc, torch.tensor(pairs, dtype=torch.int32, device="cuda"),
                      num_kv_heads=hkv, head_dim=head_dim, block_size=block_size)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kc), k_ref) and np.array_equal(host_bits(vc), v_ref)
    pa.pa_copy_blocks(kc, vc, torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
                      num_kv_heads=hkv, head_dim=head_dim, block_size=block_size)


def test_decode_steps_driven_by_the_block_manager():
    """Shared prompts, forks and copy-on-write over several decode steps: the
    caches after each step equal the oracle's bit for bit and the outputs
    match the oracle's decode."""
    Hq, Hkv, D, BS, NB = 8, 2, 128, 16, 96
    g = paged.Geom(NB, BS, Hkv, D, "bf16")
    rng = np.random.default_rng(11)
    native = pa.BlockManager(NB, BS)
    model = B.BlockManager(NB, BS)
    system = list(rng.integers(0, 50, 40))
    seqs = []
    for s in range(6):
        prompt = system + list(rng.integers(0, 50, int(rng.integers(1, 30))))
        if len(prompt) % BS == 0:
            prompt.append(1)                       # keep a partial last block to share on fork
        assert native.add_sequence(s, prompt) == model.add_sequence(s, prompt)
        seqs.append(s)
    for parent, child in ((1, 10), (4, 11), (4, 12)):
        native.fork(parent, child)
        model.fork(parent, child)
        seqs.append(child)
    kc, vc = random_cache(g, "bf16", 5), random_cache(g, "bf16", 6)
    k_ref, v_ref = host_bits(kc).copy(), host_bits(vc).copy()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    scale = 1.0 / np.sqrt(D)
    copies = 0
    for step in range(5):
        slots, pairs = [], []
        for s in seqs:
            tok = int(rng.integers(0, 50))
            got = native.append_token(s, tok)
            assert got == model.append_token(s, tok)
            slots.append(got[0])
            if got[1] >= 0:
                pairs.append((got[1], got[2]))
        copies += len(pairs)
        S = len(seqs)
        k_new = torch.randn((S, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
        v_new = torch.randn((S, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
        q = torch.randn((S, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
        maxb = 8
        bt_n, sl_n = native.batch(seqs, maxb)
        bt_o = np.full((S, maxb), -1, dtype=np.int32)
        sl_o = np.array([model.length(s) for s in seqs], dtype=np.int32)
        for i, s in enumerate(seqs):
            t = model.table(s)
            bt_o[i, :len(t)] = t
        assert np.array_equal(bt_n, bt_o) and np.array_equal(sl_n, sl_o)
        # GPU: copies, then the write, then the decode
        if pairs:
            pa.pa_copy_blocks(kc, vc, torch.tensor(pairs, dtype=torch.int32, device="cuda"),
                              num_kv_heads=Hkv, head_dim=D, block_size=BS)
        pa.pa_cache_write(k_new, v_new, torch.tensor(slots, dtype=torch.int64, device="cuda"), kc, vc,
                          block_size=BS)
        out = pa.pa_decode(q, kc, vc, torch.from_numpy(bt_n).cuda(), torch.from_numpy(sl_n).cuda(),
                           scale, num_kv_heads=Hkv, block_size=BS)
        torch.cuda.synchronize()
        # oracle: same steps on host copies, with the oracle's own tables
        B.copy_blocks(k_ref, v_ref, pairs, Hkv * BS * D)
        paged.cache_write_bf16(g, host_bits(k_new), host_bits(v_new), np.array(slots), k_ref, v_ref)
        assert np.array_equal(host_bits(kc), k_ref) and np.array_equal(host_bits(vc), v_ref), step
        ref = paged.decode(g, host_bits(q), k_ref, v_ref, bt_o, sl_o, scale)
        err = np.abs(out.cpu().double().numpy() - ref)
        assert err.max() <= min(BF16_TOL[0], BF16_ENVELOPE) and err.mean() <= BF16_TOL[1], (step, err.max())
    assert copies == 3          # one copy per sequence that wrote first into a shared partial block
