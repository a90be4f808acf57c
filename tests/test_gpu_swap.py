"""Block swap to host memory and back (pa_swap_out / pa_swap_in) on the GPU:
the host copy and the restored caches bit for bit against the oracle's swap
image, decode steps around a swap driven by the block manager, and a swap on
a second stream that overlaps a decode on the first."""

import numpy as np
import pytest
import torch

import paged_kv_cache_32_amd as pa
from oracle import blocks as B
from oracle import paged
from tests.gpu_helpers import BF16_ENVELOPE, BF16_TOL, host_bits

pytestmark = pytest.mark.gpu


def random_cache(g, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    if g.kv_dtype == "bf16":
        return torch.randn(g.cache_elems, generator=gen, device="cuda").to(torch.bfloat16)
    return torch.randint(0, 256, (g.cache_elems,), generator=gen, device="cuda",
                         dtype=torch.int32).to(torch.uint8)


def bits_to_bytes(x):
    return np.ascontiguousarray(x).view(np.uint8)


@pytest.mark.parametrize("kv_dtype,block_size,head_dim,hkv", [("bf16", 16, 128, 8), ("fp8", 32, 64, 2),
                                                               ("bf16", 48, 64, 3), ("fp8", 16, 64, 4)])
def test_swap_round_trip_bit_exact(kv_dtype, block_size, head_dim, hkv):
    g = paged.Geom(num_blocks=50, block_size=block_size, num_kv_heads=hkv, head_dim=head_dim,
                   kv_dtype=kv_dtype)
    E = hkv * block_size * head_dim
    eb = 2 if kv_dtype == "bf16" else 1
    kw = dict(num_kv_heads=hkv, head_dim=head_dim, block_size=block_size)
    kc, vc = random_cache(g, 1), random_cache(g, 2)
    k0, v0 = host_bits(kc).copy(), host_bits(vc).copy()
    rng = np.random.default_rng(4)
    perm = [int(b) for b in rng.permutation(g.num_blocks)]
    out_blocks, in_blocks = perm[:17], perm[17:34]
    n = len(out_blocks)
    host = torch.full((2 * n * E * eb,), 0xA5, dtype=torch.uint8, pin_memory=True)
    pa.pa_swap_out(kc, vc, torch.tensor(out_blocks, dtype=torch.int32, device="cuda"), host, **kw)
    torch.cuda.synchronize()
    image = B.swap_image(k0, v0, out_blocks, E)
    assert np.array_equal(host.numpy(), bits_to_bytes(image))
    assert np.array_equal(host_bits(kc), k0) and np.array_equal(host_bits(vc), v0)   # source untouched
    # back in, to other blocks
    pa.pa_swap_in(kc, vc, torch.tensor(in_blocks, dtype=torch.int32, device="cuda"), host, **kw)
    torch.cuda.synchronize()
    k_ref, v_ref = k0.copy(), v0.copy()
    B.swap_restore(k_ref, v_ref, in_blocks, image, E)
    assert np.array_equal(host_bits(kc), k_ref) and np.array_equal(host_bits(vc), v_ref)
    # ids outside the cache are skipped: their slots of the host copy are
    # left as they were; a host buffer at an offset into a pinned allocation
    host.fill_(0x5A)
    off = 4096 + 16
    pa.pa_swap_out(kc, vc, torch.tensor([3, -1, g.num_blocks], dtype=torch.int32, device="cuda"),
                   host[off:], **kw)
    torch.cuda.synchronize()
    h = host.numpy()
    assert (h[:off] == 0x5A).all()
    h = h[off:]
    assert np.array_equal(h[:E * eb], bits_to_bytes(k_ref[3 * E:4 * E]))
    assert (h[E * eb:3 * E * eb] == 0x5A).all()
    assert np.array_equal(h[3 * E * eb:4 * E * eb], bits_to_bytes(v_ref[3 * E:4 * E]))
    assert (h[6 * E * eb:] == 0x5A).all()
    # an empty list is a no-op; a short or unpinned host buffer is refused
    pa.pa_swap_out(kc, vc, torch.zeros(0, dtype=torch.int32, device="cuda"), host, **kw)
    with pytest.raises(ValueError):
        pa.pa_swap_out(kc, vc, torch.tensor(in_blocks, dtype=torch.int32, device="cuda"), host[:-1], **kw)
    for fn in (pa.pa_swap_out, pa.pa_swap_in):
        with pytest.raises(pa.PagedAttentionError) as e:
            fn(kc, vc, torch.tensor(in_blocks, dtype=torch.int32, device="cuda"),
               torch.zeros(host.numel(), dtype=torch.uint8), **kw)
        assert e.value.status == -10
    assert np.array_equal(host_bits(kc), k_ref) and np.array_equal(host_bits(vc), v_ref)


def test_decode_around_a_swap_driven_by_the_block_manager():
    """Sequence 0 is paused and swapped out (its private blocks freed, the
    shared prompt blocks kept), a new request reuses the freed blocks and
    overwrites them, sequence 0 comes back into other blocks: its decode
    output is the oracle's for its unchanged contents."""
    Hq, Hkv, D, BS, NB = 16, 2, 128, 16, 24
    g = paged.Geom(NB, BS, Hkv, D, "bf16")
    E = Hkv * BS * D
    kw = dict(num_kv_heads=Hkv, head_dim=D, block_size=BS)
    rng = np.random.default_rng(5)
    native, model = pa.BlockManager(NB, BS), B.BlockManager(NB, BS)
    system = list(rng.integers(0, 50, 32))                        # two shared full blocks
    for s, n in ((0, 70), (1, 20)):
        prompt = system + list(rng.integers(0, 50, n))
        assert native.add_sequence(s, prompt) == model.add_sequence(s, prompt)
    kc, vc = random_cache(g, 7), random_cache(g, 8)
    k_ref, v_ref = host_bits(kc).copy(), host_bits(vc).copy()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    scale = 1.0 / np.sqrt(D)

    def decode(seqs):
        bt, sl = native.batch(seqs, NB)
        bt_o = np.full((len(seqs), NB), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            bt_o[i, :len(model.table(s))] = model.table(s)
        assert np.array_equal(bt, bt_o)
        q = torch.randn((len(seqs), Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
        out = pa.pa_decode(q, kc, vc, torch.from_numpy(bt).cuda(), torch.from_numpy(sl).cuda(), scale,
                           num_kv_heads=Hkv, block_size=BS)
        torch.cuda.synchronize()
        ref = paged.decode(g, host_bits(q), k_ref, v_ref, bt_o, sl, scale)
        err = np.abs(out.cpu().double().numpy() - ref)
        assert err.max() <= min(BF16_TOL[0], BF16_ENVELOPE) and err.mean() <= BF16_TOL[1], err.max()

    decode([0, 1])
    t0 = model.table(0)
    out = native.swap_out(0)
    assert out == model.swap_out(0) == t0[2:]                    # the shared prompt blocks stay
    host = torch.empty(2 * len(out) * E * 2, dtype=torch.uint8, pin_memory=True)
    pa.pa_swap_out(kc, vc, torch.tensor(out, dtype=torch.int32, device="cuda"), host, **kw)
    torch.cuda.synchronize()
    image = B.swap_image(k_ref, v_ref, out, E)
    # a new request takes the freed blocks; its K/V overwrite them
    prompt = list(rng.integers(50, 99, BS * model.num_free()))
    assert native.add_sequence(2, prompt) == model.add_sequence(2, prompt) == 0
    assert native.num_free() == model.num_free() == 0 and set(out) <= set(model.table(2))
    T = len(prompt)
    slots = np.array([model.table(2)[i // BS] * BS + i % BS for i in range(T)])
    k_new = torch.randn((T, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    v_new = torch.randn((T, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
    pa.pa_cache_write(k_new, v_new, torch.from_numpy(slots).cuda(), kc, vc, block_size=BS)
    paged.cache_write_bf16(g, host_bits(k_new), host_bits(v_new), slots, k_ref, v_ref)
    decode([1, 2])
    with pytest.raises(pa.PagedAttentionError):
        native.swap_in(0)                                       # no room until 2 finishes
    native.free_sequence(2)
    model.free_sequence(2)
    back = native.swap_in(0)
    assert back == model.swap_in(0) and model.table(0) == t0[:2] + back
    pa.pa_swap_in(kc, vc, torch.tensor(back, dtype=torch.int32, device="cuda"), host, **kw)
    B.swap_restore(k_ref, v_ref, back, image, E)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kc), k_ref) and np.array_equal(host_bits(vc), v_ref)
    decode([0, 1])


def test_swap_on_a_second_stream_overlaps_a_decode():
    """A swap-out and swap-in of blocks no decode reads, on their own stream,
    while decodes run on the current stream: both results stay exact."""
    Hq, Hkv, D, BS, NB = 64, 8, 128, 16, 4096
    g = paged.Geom(NB, BS, Hkv, D, "bf16")
    E = Hkv * BS * D
    kw = dict(num_kv_heads=Hkv, head_dim=D, block_size=BS)
    kc, vc = random_cache(g, 11), random_cache(g, 12)
    k0, v0 = host_bits(kc).copy(), host_bits(vc).copy()
    S, maxb = 16, 128
    rng = np.random.default_rng(13)
    bt = rng.permutation(NB // 2)[:S * maxb].reshape(S, maxb).astype(np.int32)   # decode: first half
    sl = rng.integers(1, maxb * BS + 1, S).astype(np.int32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(14)
    q = torch.randn((S, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    out_blocks = [int(b) for b in rng.permutation(np.arange(NB // 2, NB))[:512]]  # swap: second half
    in_blocks = sorted(out_blocks)[::-1]
    n = len(out_blocks)
    host = torch.empty(2 * n * E * 2, dtype=torch.uint8, pin_memory=True)
    image = bits_to_bytes(B.swap_image(k0, v0, out_blocks, E))
    host_in = torch.from_numpy(image.copy()).pin_memory()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(sl).cuda()
    with torch.cuda.stream(side):
        pa.pa_swap_out(kc, vc, torch.tensor(out_blocks, dtype=torch.int32, device="cuda"), host, **kw)
        pa.pa_swap_in(kc, vc, torch.tensor(in_blocks, dtype=torch.int32, device="cuda"), host_in, **kw)
    outs = [pa.pa_decode(q, kc, vc, btd, sld, 0.088, num_kv_heads=Hkv, block_size=BS) for _ in range(3)]
    torch.cuda.synchronize()
    assert np.array_equal(host.numpy(), image)
    k_ref, v_ref = k0.copy(), v0.copy()
    B.swap_restore(k_ref, v_ref, in_blocks, np.ascontiguousarray(image).view(k0.dtype), E)
    assert np.array_equal(host_bits(kc), k_ref) and np.array_equal(host_bits(vc), v_ref)
    rows = [0, 5, 15]                         # the oracle on a few sequences
    ref = paged.decode(g, host_bits(q)[rows], k0, v0, bt[rows], sl[rows], 0.088)
    for o in outs:
        err = np.abs(o.cpu().double().numpy()[rows] - ref)
        assert err.max() <= min(BF16_TOL[0], BF16_ENVELOPE) and err.mean() <= BF16_TOL[1], err.max()
