"""Shared plumbing for the GPU parity tests: move a seeded workload to the
device, run the library's entry points, and build the oracle's expected
caches and outputs from the generator's inputs (never from the kernels'
results)."""

import numpy as np
import torch

import paged_kv_cache_32_amd as pa
from oracle import paged

BF16_TOL = (1e-2, 1e-3)   # max-abs, mean-abs: the contract
FP8_TOL = (5e-2, None)
# Accuracy envelope, checked beside the contract: the kernels accumulate in
# float32 over bf16-exact products, with probabilities carried as a bf16
# pair (about 16 significant bits), so against the fp64 oracle on the same
# cache bytes their error stays near 1e-5 of the values involved.  A lost or
# doubled split-K piece moves a row by about 1/pieces of its magnitude, far
# outside this envelope, while the contract bounds alone could miss it.
BF16_ENVELOPE = 1e-4          # max-abs
FP8_ENVELOPE_REL_RMS = 1e-3   # max-abs / rms of the oracle's outputs


def device_inputs(w, dev="cuda", layers=None, poison=True):
    t = w.make_tensors(dev, layers=layers, poison=poison)
    t["block_tables"] = torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(dev)
    t["seq_lens"] = torch.from_numpy(np.ascontiguousarray(w.seq_lens)).to(dev)
    t["slot_mapping"] = torch.from_numpy(np.ascontiguousarray(w.slot_mapping)).to(dev)
    return t


def host_bits(t):
    """Device tensor -> numpy bit patterns (uint16 for bf16, uint8 for fp8)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def geom(w):
    return paged.Geom(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)


def oracle_caches(w, kc_bits, vc_bits, k_new_bits, v_new_bits, k_scale=1.0, v_scale=1.0):
    """The caches after this step's write, as the oracle computes them from
    the pre-write caches and the new tokens."""
    kc, vc = kc_bits.copy(), vc_bits.copy()
    g = geom(w)
    if w.kv_dtype == "bf16":
        paged.cache_write_bf16(g, k_new_bits, v_new_bits, w.slot_mapping, kc, vc)
    else:
        paged.cache_write_fp8(g, k_new_bits, v_new_bits, w.slot_mapping, kc, vc,
                              np.float32(k_scale), np.float32(v_scale))
    return kc, vc


def gpu_write(w, t, layer=0):
    kc, vc = t["k_cache"][layer], t["v_cache"][layer]
    if w.kv_dtype == "bf16":
        pa.pa_cache_write(t["k_new"][layer], t["v_new"][layer], t["slot_mapping"], kc, vc,
                          block_size=w.block_size)
    else:
        pa.pa_cache_write_fp8(t["k_new"][layer], t["v_new"][layer], t["slot_mapping"], kc, vc,
                              float(t["k_scale"][layer]), float(t["v_scale"][layer]),
                              block_size=w.block_size)


def gpu_decode(w, t, layer=0, partition_tokens=0, out=None, workspace=None):
    kc, vc = t["k_cache"][layer], t["v_cache"][layer]
    if w.kv_dtype == "bf16":
        return pa.pa_decode(t["q"][layer], kc, vc, t["block_tables"], t["seq_lens"], w.scale, out,
                            num_kv_heads=w.num_kv_heads, block_size=w.block_size,
                            partition_tokens=partition_tokens, workspace=workspace)
    return pa.pa_decode_fp8(t["q"][layer], kc, vc, t["block_tables"], t["seq_lens"], w.scale,
                            float(t["k_scale"][layer]), float(t["v_scale"][layer]), out,
                            num_kv_heads=w.num_kv_heads, block_size=w.block_size,
                            partition_tokens=partition_tokens, workspace=workspace)


def oracle_decode(w, q_bits, kc, vc, k_scale=1.0, v_scale=1.0, seqs=None):
    return paged.decode(geom(w), q_bits, kc, vc, w.block_tables, w.seq_lens, w.scale,
                        k_scale=float(np.float32(k_scale)), v_scale=float(np.float32(v_scale)),
                        seqs=seqs)


def compare(got, ref, kv_dtype, seqs=None, label="", envelope=True):
    """Element-wise comparison over the computed rows against the contract
    bounds and (unless ``envelope`` is false) the accuracy envelope; returns
    (max, mean)."""
    got = got.detach().cpu().double().numpy() if isinstance(got, torch.Tensor) else got
    if seqs is not None:
        got, ref = got[list(seqs)], ref[list(seqs)]
    assert np.all(np.isfinite(ref)), f"{label}: oracle output not finite"
    assert np.all(np.isfinite(got)), f"{label}: GPU output has non-finite values"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    tol_max, tol_mean = BF16_TOL if kv_dtype == "bf16" else FP8_TOL
    assert mx <= tol_max, f"{label}: max-abs {mx:.3e} > {tol_max}"
    if tol_mean is not None:
        assert mean <= tol_mean, f"{label}: mean-abs {mean:.3e} > {tol_mean}"
    if envelope:
        if kv_dtype == "bf16":
            assert mx <= BF16_ENVELOPE, f"{label}: max-abs {mx:.3e} outside the accuracy envelope {BF16_ENVELOPE}"
        else:
            rms = float(np.sqrt(np.mean(ref * ref)))
            assert mx <= FP8_ENVELOPE_REL_RMS * rms, \
                f"{label}: max-abs {mx:.3e} outside the accuracy envelope {FP8_ENVELOPE_REL_RMS} x rms {rms:.3e}"
    return mx, mean


def step_and_check(w, t, layer=0, partition_tokens=0, seqs=None, label="", write=True):
    """Write the new tokens and decode on the GPU; check the caches bit for
    bit and the output against the oracle.  Returns (max, mean) error."""
    kc0, vc0 = host_bits(t["k_cache"][layer]), host_bits(t["v_cache"][layer])
    kn, vn = host_bits(t["k_new"][layer]), host_bits(t["v_new"][layer])
    ks = float(t["k_scale"][layer]) if w.kv_dtype == "fp8" else 1.0
    vs = float(t["v_scale"][layer]) if w.kv_dtype == "fp8" else 1.0
    if write:
        gpu_write(w, t, layer)
        kc_ref, vc_ref = oracle_caches(w, kc0, vc0, kn, vn, ks, vs)
    else:
        kc_ref, vc_ref = kc0, vc0
    out = gpu_decode(w, t, layer, partition_tokens)
    torch.cuda.synchronize()
    kc1, vc1 = host_bits(t["k_cache"][layer]), host_bits(t["v_cache"][layer])
    assert np.array_equal(kc1, kc_ref), f"{label}: K cache differs from the oracle's write"
    assert np.array_equal(vc1, vc_ref), f"{label}: V cache differs from the oracle's write"
    ref = oracle_decode(w, host_bits(t["q"][layer]), kc_ref, vc_ref, ks, vs, seqs=seqs)
    return compare(out, ref, w.kv_dtype, seqs=seqs, label=label)
