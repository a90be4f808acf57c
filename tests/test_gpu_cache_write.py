"""pa_cache_write / pa_cache_write_fp8 on the GPU: bit-exact against the
oracle's slot scatter and e4m3 encoder."""

import numpy as np
import pytest
import torch

import paged_kv_cache_32_amd as pa
from oracle import paged
from paged_kv_cache_32_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _flat_caches(g, fill, dev="cuda"):
    if g.kv_dtype == "bf16":
        kc = torch.full((g.cache_elems,), fill, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        kc = torch.full((g.cache_elems,), fill, dtype=torch.uint8, device=dev)
    return kc, kc.clone()


@pytest.mark.parametrize("scale", [1.0, 0.0123, 1 / 448, 3.75, 2.0 ** -12, 97.0])
def test_fp8_encode_every_bf16_pattern(scale):
    """All 65,536 bf16 bit patterns (NaNs and infinities included) written as
    512 tokens of 1 KV head x 128 dims; V gets them in reverse order."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    kb = pats.reshape(512, 1, 128)
    vb = pats[::-1].copy().reshape(512, 1, 128)
    g = paged.Geom(33, 16, 1, 128, "fp8")
    slots = np.random.default_rng(11).permutation(33 * 16)[:512].astype(np.int64)
    kc, vc = _flat_caches(g, 0x55)
    k = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
    v = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
    pa.pa_cache_write_fp8(k, v, torch.from_numpy(slots).cuda(), kc, vc, scale, scale, block_size=16)
    torch.cuda.synchronize()
    kref = np.full(g.cache_elems, 0x55, dtype=np.uint8)
    vref = kref.copy()
    paged.cache_write_fp8(g, kb, vb, slots, kref, vref, np.float32(scale), np.float32(scale))
    got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    bad = np.nonzero(got_k != kref)[0]
    assert bad.size == 0, f"{bad.size} K codes differ, first at {bad[:5]}: {got_k[bad[:5]]} vs {kref[bad[:5]]}"
    assert np.array_equal(got_v, vref)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_size,head_dim", [(16, 128), (32, 64), (48, 128)])
def test_scatter_skips_and_leaves_other_slots(kv_dtype, block_size, head_dim):
    rng = np.random.default_rng(block_size + head_dim)
    Hkv, NB, T = 3, 7, 20
    g = paged.Geom(NB, block_size, Hkv, head_dim, kv_dtype)
    slots = rng.permutation(NB * block_size)[:T].astype(np.int64)
    slots[3] = -1
    slots[7] = NB * block_size          # past the pool: skipped
    slots[11] = -12345
    kb = (rng.standard_normal((T, Hkv, head_dim)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (rng.standard_normal((T, Hkv, head_dim)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    fill = 0x7FC0 if kv_dtype == "bf16" else 0x7F
    kc, vc = _flat_caches(g, fill if kv_dtype == "fp8" else 0x7FC0)
    k = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
    v = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
    sm = torch.from_numpy(slots).cuda()
    ks, vs = 0.02, 0.013
    if kv_dtype == "bf16":
        pa.pa_cache_write(k, v, sm, kc, vc, block_size=block_size)
    else:
        pa.pa_cache_write_fp8(k, v, sm, kc, vc, ks, vs, block_size=block_size)
    torch.cuda.synchronize()
    kref = np.full(g.cache_elems, fill, dtype=g.np_dtype)
    vref = kref.copy()
    if kv_dtype == "bf16":
        paged.cache_write_bf16(g, kb, vb, slots, kref, vref)
    else:
        paged.cache_write_fp8(g, kb, vb, slots, kref, vref, np.float32(ks), np.float32(vs))
    assert np.array_equal(H.host_bits(kc), kref)
    assert np.array_equal(H.host_bits(vc), vref)


def test_tiny_workload_write_is_bit_exact():
    w = W.config(1)
    t = H.device_inputs(w)
    kc0, vc0 = H.host_bits(t["k_cache"][0]), H.host_bits(t["v_cache"][0])
    H.gpu_write(w, t)
    torch.cuda.synchronize()
    kref, vref = H.oracle_caches(w, kc0, vc0, H.host_bits(t["k_new"][0]), H.host_bits(t["v_new"][0]))
    assert np.array_equal(H.host_bits(t["k_cache"][0]), kref)
    assert np.array_equal(H.host_bits(t["v_cache"][0]), vref)


def test_zero_tokens_is_a_noop():
    g = paged.Geom(2, 16, 1, 64)
    kc, vc = _flat_caches(g, 0x1234)
    e = torch.empty((0, 1, 64), dtype=torch.bfloat16, device="cuda")
    pa.pa_cache_write(e, e, torch.empty(0, dtype=torch.int64, device="cuda"), kc, vc, block_size=16)
    torch.cuda.synchronize()
    assert np.all(H.host_bits(kc) == 0x1234)
