"""paged_kv_cache_32_amd: paged-attention decode over a block-table KV cache
for AMD Instinct MI355X (gfx950).

The compute lives in ``lib/libpa.so`` (hand-written HIP kernels behind the C
ABI in ``include/pa.h``).  This module is the thin Python binding: it checks
torch tensors (device, dtype, contiguity, shapes), passes their device
pointers and the current HIP stream to the C entry points of the same name,
and raises on any non-OK status.  It computes nothing itself and has no
fallback: without the built library every call raises.

    pa_cache_write(k, v, slot_mapping, k_cache, v_cache, block_size=...)
    pa_cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, block_size=...)
    pa_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, out, block_size=...)
    pa_decode_fp8(q, k_cache, v_cache, block_tables, seq_lens, scale, out, k_scale, v_scale, ...)
    pa_decode_workspace_size(...), pa_decode_workspace_init(workspace)
    pa_copy_blocks(k_cache, v_cache, pairs, ...)
    BlockManager(num_blocks, block_size)   (host block manager, include/pa_blocks.h)

Cache tensors are flat (or any contiguous shape) with num_blocks *
num_kv_heads * block_size * head_dim elements, bfloat16 for the bf16 cache
and uint8 (e4m3fn codes) for the fp8 cache, in the tiled layout documented
in ``include/pa.h``.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libpa.so")

PA_OK = 0
_STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
           -4: "PA_ERR_WORKSPACE", -5: "PA_ERR_LAUNCH", -6: "PA_ERR_DEVICE",
           -7: "PA_ERR_NO_BLOCKS", -8: "PA_ERR_NOT_FOUND", -9: "PA_ERR_SWAPPED",
           -10: "PA_ERR_HOST_MEMORY"}


class PagedAttentionError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class CascadePlanInfo(ctypes.Structure):
    _fields_ = [("num_segments", ctypes.c_int32), ("num_items", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("num_seg_blocks", ctypes.c_int32), ("num_members", ctypes.c_int32),
                ("num_parts", ctypes.c_int32), ("members_per_workgroup", ctypes.c_int32),
                ("chunk_blocks", ctypes.c_int32), ("shared_tokens", ctypes.c_int64),
                ("segment_tokens", ctypes.c_int64)]


class CascadeDevicePlan(ctypes.Structure):
    _fields_ = [("items", ctypes.c_void_p), ("num_items", ctypes.c_int32), ("seg_blocks", ctypes.c_void_p),
                ("members", ctypes.c_void_p), ("parts_off", ctypes.c_void_p), ("parts", ctypes.c_void_p),
                ("num_slots", ctypes.c_int32), ("private_tables", ctypes.c_void_p),
                ("private_lens", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpa.so is not built ({LIB_PATH}); run "
                          "`python -m paged_kv_cache_32_amd.build` (gfx950 HIP library)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(CacheDesc)
    sigs = {
        "pa_cache_write": ([dp, vp, vp, vp, i32, vp, vp, vp], i32),
        "pa_cache_write_fp8": ([dp, vp, vp, vp, i32, vp, vp, f32, f32, vp], i32),
        "pa_decode_workspace_size": ([dp, i32, i32, i32, i32], sz),
        "pa_decode_workspace_init": ([vp, sz, vp], i32),
        "pa_decode_workspace_check": ([vp, sz, i32, i32, vp, vp], i32),
        "pa_decode": ([dp, vp, i32, i32, vp, vp, vp, i32, vp, f32, vp, i32, vp, sz, vp], i32),
        "pa_decode_fp8": ([dp, vp, i32, i32, vp, vp, vp, i32, vp, f32, f32, f32, vp, i32, vp, sz,
                           vp], i32),
        "pa_decode_noalloc": ([dp, vp, i32, i32, vp, vp, vp, i32, vp, f32, vp, i32, vp], i32),
        "pa_status_string": ([i32], ctypes.c_char_p),
        "pa_abi_version": ([], i32),
        "pa_copy_blocks": ([dp, i32, vp, vp, vp, i32, vp], i32),
        "pa_bm_create": ([i32, i32, ctypes.POINTER(vp)], i32),
        "pa_bm_destroy": ([vp], None),
        "pa_bm_add_sequence": ([vp, i64, ctypes.POINTER(i32), i32, ctypes.c_uint64,
                                ctypes.POINTER(i32)], i32),
        "pa_bm_fork": ([vp, i64, i64], i32),
        "pa_bm_append_token": ([vp, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i32),
                                ctypes.POINTER(i32)], i32),
        "pa_bm_free_sequence": ([vp, i64], i32),
        "pa_bm_trim": ([vp, i64, i32, ctypes.POINTER(i32)], i32),
        "pa_bm_swap_out": ([vp, i64, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)], i32),
        "pa_bm_swap_in": ([vp, i64, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)], i32),
        "pa_swap_out": ([dp, i32, vp, vp, vp, i32, vp, vp], i32),
        "pa_swap_in": ([dp, i32, vp, vp, vp, i32, vp, vp], i32),
        "pa_decode_window": ([dp, vp, i32, i32, vp, vp, vp, i32, vp, i32, f32, vp, i32, vp, sz, vp], i32),
        "pa_decode_window_fp8": ([dp, vp, i32, i32, vp, vp, vp, i32, vp, i32, f32, f32, f32, vp, i32, vp,
                                  sz, vp], i32),
        "pa_decode_append": ([dp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp, i32, f32, vp, i32, vp, sz, vp],
                             i32),
        "pa_decode_append_fp8": ([dp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp, i32, f32, f32, f32, vp, i32,
                                  vp, sz, vp], i32),
        "pa_decode_ring": ([dp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp, i32, f32, vp, i32, vp, sz, vp], i32),
        "pa_decode_ring_fp8": ([dp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp, i32, f32, f32, f32, vp, i32,
                                vp, sz, vp], i32),
        "pa_bm_add_ring_sequence": ([vp, i64, i32, i32, ctypes.POINTER(i32)], i32),
        "pa_bm_slots": ([vp, i64, i32, i32, ctypes.POINTER(i64)], i32),
        "pa_quest_clear": ([dp, vp, vp], i32),
        "pa_quest_update": ([dp, i32, vp, vp, i32, vp, vp], i32),
        "pa_quest_cache_write": ([dp, vp, vp, vp, i32, vp, vp, vp, vp], i32),
        "pa_quest_cache_write_fp8": ([dp, vp, vp, vp, i32, vp, vp, f32, f32, vp, vp], i32),
        "pa_quest_summarize": ([dp, i32, vp, vp, vp, i32, vp, vp], i32),
        "pa_quest_select_workspace_size": ([i32, i32, i32], sz),
        "pa_quest_select": ([dp, vp, i32, i32, vp, vp, i32, vp, i32, vp, vp, vp, sz, vp], i32),
        "pa_decode_quest_workspace_size": ([dp, i32, i32, i32, i32], sz),
        "pa_decode_quest": ([dp, vp, i32, i32, vp, vp, vp, i32, vp, f32, vp, i32, vp, sz, vp], i32),
        "pa_decode_quest_fp8": ([dp, vp, i32, i32, vp, vp, vp, i32, vp, f32, f32, f32, vp, i32, vp, sz,
                                 vp], i32),
        "pa_cascade_plan_build": ([vp, i32, i32, vp, i32, i32, i32, i32, ctypes.POINTER(vp)], i32),
        "pa_cascade_plan_destroy": ([vp], None),
        "pa_cascade_plan_get_info": ([vp, ctypes.POINTER(CascadePlanInfo)], i32),
        "pa_cascade_plan_export": ([vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "pa_decode_cascade_workspace_size": ([dp, i32, i32, i32, i32, i32], sz),
        "pa_decode_cascade": ([dp, vp, i32, i32, vp, vp, i32, ctypes.POINTER(CascadeDevicePlan), f32, vp, i32,
                               vp, sz, vp], i32),
        "pa_decode_cascade_fp8": ([dp, vp, i32, i32, vp, vp, i32, ctypes.POINTER(CascadeDevicePlan), f32, f32,
                                   f32, vp, i32, vp, sz, vp], i32),
        "pa_probe_stream_read": ([vp, sz, vp, vp], i32),
        "pa_probe_tile_read": ([dp, i32, vp, vp, vp, i32, i32, vp, i32, vp, vp], i32),
        "pa_bm_num_free": ([vp], i32),
        "pa_bm_sequence_info": ([vp, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "pa_bm_block_table": ([vp, i64, ctypes.POINTER(i32), i32], i32),
        "pa_bm_refcount": ([vp, i32, ctypes.POINTER(i32)], i32),
        "pa_bm_stats": ([vp, ctypes.POINTER(i64), ctypes.POINTER(i64)], i32),
        "pa_bm_batch": ([vp, ctypes.POINTER(i64), i32, i32, ctypes.POINTER(i32),
                         ctypes.POINTER(i32)], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _load()


def _check(fn, status):
    if status != PA_OK:
        msg = _load().pa_status_string(status).decode()
        raise PagedAttentionError(fn, status, msg)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, dtype, device, ndim=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def make_desc(k_cache, num_kv_heads, head_dim, block_size):
    per_block = num_kv_heads * block_size * head_dim
    if per_block <= 0 or k_cache.numel() % per_block:
        raise ValueError("cache size is not a whole number of blocks")
    return CacheDesc(k_cache.numel() // per_block, block_size, num_kv_heads, head_dim)


def _cache_write(fp8, k, v, slot_mapping, k_cache, v_cache, block_size, k_scale, v_scale):
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("pa_cache_write needs device tensors")
    _need(k, "k", torch.bfloat16, dev, 3)
    T, Hkv, D = k.shape
    _need(v, "v", torch.bfloat16, dev, shape=k.shape)
    _need(slot_mapping, "slot_mapping", torch.int64, dev, shape=(T,))
    cdt = torch.uint8 if fp8 else torch.bfloat16
    _need(k_cache, "k_cache", cdt, dev)
    _need(v_cache, "v_cache", cdt, dev)
    if v_cache.numel() != k_cache.numel():
        raise ValueError("k_cache and v_cache differ in size")
    desc = make_desc(k_cache, Hkv, D, block_size)
    L = _load()
    with torch.cuda.device(dev):
        if fp8:
            st = L.pa_cache_write_fp8(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping), T,
                                      _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale),
                                      _stream(k))
        else:
            st = L.pa_cache_write(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping), T,
                                  _ptr(k_cache), _ptr(v_cache), _stream(k))
    _check("pa_cache_write_fp8" if fp8 else "pa_cache_write", st)


def pa_cache_write(k, v, slot_mapping, k_cache, v_cache, block_size):
    """Scatter k, v [T, Hkv, D] bf16 into the bf16 caches at slot_mapping [T]
    int64 (slot < 0: skip).  See pa_cache_write in include/pa.h."""
    _cache_write(False, k, v, slot_mapping, k_cache, v_cache, block_size, 1.0, 1.0)


def pa_cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, block_size):
    """As pa_cache_write into uint8 e4m3fn caches with per-tensor scales."""
    _cache_write(True, k, v, slot_mapping, k_cache, v_cache, block_size, k_scale, v_scale)


def pa_decode_workspace_size(num_blocks, block_size, num_kv_heads, head_dim, num_seqs,
                             num_q_heads, max_blocks_per_seq, partition_tokens=0):
    """Workspace bytes pa_decode needs on the current device."""
    desc = CacheDesc(num_blocks, block_size, num_kv_heads, head_dim)
    return int(_load().pa_decode_workspace_size(ctypes.byref(desc), num_seqs, num_q_heads,
                                                max_blocks_per_seq, partition_tokens))


def pa_decode_workspace_init(workspace):
    """Zero-fill a decode workspace (uint8 device tensor) on the current stream."""
    _need(workspace, "workspace", torch.uint8, workspace.device)
    with torch.cuda.device(workspace.device):
        st = _load().pa_decode_workspace_init(_ptr(workspace), workspace.numel(), _stream(workspace))
    _check("pa_decode_workspace_init", st)


def pa_decode_workspace_check(workspace, num_seqs, num_kv_heads, nonzero=None):
    """Number of non-zero merge counters in a decode workspace (0 after every
    completed call).  The count is written on the current stream into
    ``nonzero`` (int32 device tensor of one element, allocated if None),
    which is returned; ``int(...)`` of it synchronizes."""
    _need(workspace, "workspace", torch.uint8, workspace.device)
    if nonzero is None:
        nonzero = torch.empty((1,), dtype=torch.int32, device=workspace.device)
    _need(nonzero, "nonzero", torch.int32, workspace.device, shape=(1,))
    with torch.cuda.device(workspace.device):
        st = _load().pa_decode_workspace_check(_ptr(workspace), workspace.numel(), num_seqs, num_kv_heads,
                                               _ptr(nonzero), _stream(workspace))
    _check("pa_decode_workspace_check", st)
    return nonzero


def alloc_workspace(num_blocks, block_size, num_kv_heads, head_dim, num_seqs, num_q_heads,
                    max_blocks_per_seq, partition_tokens=0, device="cuda"):
    """A zero-filled workspace of the size pa_decode needs for these sizes."""
    dev = torch.device(device)
    with torch.cuda.device(dev):
        n = pa_decode_workspace_size(num_blocks, block_size, num_kv_heads, head_dim, num_seqs,
                                     num_q_heads, max_blocks_per_seq, partition_tokens)
    if n == 0:
        raise PagedAttentionError("pa_decode_workspace_size", -6, "no gfx950 device or invalid sizes")
    return torch.zeros(n, dtype=torch.uint8, device=dev)


def _decode(fp8, q, k_cache, v_cache, block_tables, seq_lens, scale, out, num_kv_heads,
            block_size, k_scale, v_scale, partition_tokens, workspace, window=None):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("pa_decode needs device tensors")
    _need(q, "q", torch.bfloat16, dev, 3)
    S, Hq, D = q.shape
    cdt = torch.uint8 if fp8 else torch.bfloat16
    _need(k_cache, "k_cache", cdt, dev)
    _need(v_cache, "v_cache", cdt, dev)
    if v_cache.numel() != k_cache.numel():
        raise ValueError("k_cache and v_cache differ in size")
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    _need(seq_lens, "seq_lens", torch.int32, dev, shape=(S,))
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, shape=(S, Hq, D))
    desc = make_desc(k_cache, num_kv_heads, D, block_size)
    maxb = block_tables.shape[1]
    L = _load()
    with torch.cuda.device(dev):
        if workspace is None:
            need = L.pa_decode_workspace_size(ctypes.byref(desc), S, Hq, maxb, partition_tokens)
            if need == 0 and S > 0:
                raise PagedAttentionError("pa_decode_workspace_size", -6,
                                          "no gfx950 device or invalid sizes")
            workspace = torch.zeros(max(int(need), 1), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, dev)
        args = [ctypes.byref(desc), _ptr(q), S, Hq, _ptr(k_cache), _ptr(v_cache),
                _ptr(block_tables), maxb, _ptr(seq_lens)]
        if window is not None:
            args += [int(window)]
        args += [float(scale)]
        if fp8:
            args += [float(k_scale), float(v_scale)]
        args += [_ptr(out), int(partition_tokens), _ptr(workspace), workspace.numel(), _stream(q)]
        name = "pa_decode" + ("_window" if window is not None else "") + ("_fp8" if fp8 else "")
        st = getattr(L, name)(*args)
    _check(name, st)
    return out


def pa_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, out=None, *, num_kv_heads,
              block_size, partition_tokens=0, workspace=None):
    """Paged decode over a bf16 cache: q [S, Hq, D] bf16 -> out [S, Hq, D]
    float32.  See pa_decode in include/pa.h."""
    return _decode(False, q, k_cache, v_cache, block_tables, seq_lens, scale, out, num_kv_heads,
                   block_size, 1.0, 1.0, partition_tokens, workspace)


def pa_decode_fp8(q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale, v_scale, out=None,
                  *, num_kv_heads, block_size, partition_tokens=0, workspace=None):
    """Paged decode over an e4m3fn cache with per-tensor scales."""
    return _decode(True, q, k_cache, v_cache, block_tables, seq_lens, scale, out, num_kv_heads,
                   block_size, k_scale, v_scale, partition_tokens, workspace)


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, scale, out=None, *, num_kv_heads,
                      block_size, partition_tokens=0):
    """pa_decode with no workspace: the library's own per-GPU scratch array
    serves as one (include/pa.h).  Calls on one GPU must not overlap."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    S, Hq, D = q.shape
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev, shape=tuple(k_cache.shape))
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, shape=(S,))
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, shape=(S, Hq, D))
    desc = make_desc(k_cache, num_kv_heads, D, block_size)
    with torch.cuda.device(dev):
        st = _load().pa_decode_noalloc(ctypes.byref(desc), _ptr(q), S, Hq, _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), float(scale),
                                       _ptr(out), int(partition_tokens), _stream(q))
    _check("pa_decode_noalloc", st)
    return out


def pa_copy_blocks(k_cache, v_cache, pairs, *, num_kv_heads, head_dim, block_size):
    """Copy whole blocks of both caches on the GPU: pairs is an int32 device
    tensor [n, 2] of {src, dst} block ids.  See pa_copy_blocks in
    include/pa_blocks.h."""
    dev = k_cache.device
    if dev.type != "cuda":
        raise ValueError("pa_copy_blocks needs device tensors")
    if k_cache.dtype not in (torch.bfloat16, torch.uint8):
        raise TypeError("caches must be bfloat16 or uint8 (e4m3fn codes)")
    _need(k_cache, "k_cache", k_cache.dtype, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev, shape=tuple(k_cache.shape))
    _need(pairs, "pairs", torch.int32, dev, 2)
    if pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    desc = make_desc(k_cache, num_kv_heads, head_dim, block_size)
    eb = 2 if k_cache.dtype == torch.bfloat16 else 1
    with torch.cuda.device(dev):
        st = _load().pa_copy_blocks(ctypes.byref(desc), eb, _ptr(k_cache), _ptr(v_cache), _ptr(pairs),
                                    pairs.shape[0], _stream(k_cache))
    _check("pa_copy_blocks", st)



def pa_probe_stream_read(buf, sink=None):
    """Read a contiguous device tensor once (include/pa_probe.h): returns the
    int32 device tensor ``sink`` (zeroed when not given) into which the XOR
    of all the buffer's 32-bit words is folded."""
    dev = buf.device
    if dev.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(sink, "sink", torch.int32, dev)
    nbytes = buf.numel() * buf.element_size()
    with torch.cuda.device(dev):
        st = _load().pa_probe_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf))
    _check("pa_probe_stream_read", st)
    return sink


def pa_probe_tile_read(k_cache, v_cache, block_tables, seq_lens, *, num_kv_heads, head_dim, block_size,
                       window=0, sink=None):
    """Read the cache tiles pa_decode (pa_decode_window with a window) reads
    for these tables and lengths, with no arithmetic (include/pa_probe.h);
    bf16 or uint8 (e4m3fn) caches.  Returns the int32 device tensor ``sink``
    holding the XOR of their words."""
    dev = k_cache.device
    if k_cache.dtype not in (torch.bfloat16, torch.uint8):
        raise TypeError("caches must be bfloat16 or uint8 (e4m3fn codes)")
    _need(k_cache, "k_cache", k_cache.dtype, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev, shape=tuple(k_cache.shape))
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    S, maxb = block_tables.shape
    _need(seq_lens, "seq_lens", torch.int32, dev, shape=(S,))
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(sink, "sink", torch.int32, dev)
    desc = make_desc(k_cache, num_kv_heads, head_dim, block_size)
    eb = 2 if k_cache.dtype == torch.bfloat16 else 1
    with torch.cuda.device(dev):
        st = _load().pa_probe_tile_read(ctypes.byref(desc), eb, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                        S, maxb, _ptr(seq_lens), int(window), _ptr(sink), _stream(k_cache))
    _check("pa_probe_tile_read", st)
    return sink

def _swap(out, k_cache, v_cache, blocks, host, num_kv_heads, head_dim, block_size):
    dev = k_cache.device
    _need(k_cache, "k_cache", k_cache.dtype, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev, shape=tuple(k_cache.shape))
    _need(blocks, "blocks", torch.int32, dev, 1)
    if not isinstance(host, torch.Tensor) or host.device.type != "cpu" or not host.is_contiguous() \
            or host.dtype != torch.uint8:
        raise ValueError("host must be a contiguous uint8 CPU tensor in pinned memory")
    desc = make_desc(k_cache, num_kv_heads, head_dim, block_size)
    eb = 2 if k_cache.dtype == torch.bfloat16 else 1
    need = 2 * blocks.numel() * num_kv_heads * block_size * head_dim * eb
    if host.numel() < need:
        raise ValueError(f"host buffer holds {host.numel()} bytes, {need} needed")
    L = _load()
    fn = L.pa_swap_out if out else L.pa_swap_in
    with torch.cuda.device(dev):
        st = fn(ctypes.byref(desc), eb, _ptr(k_cache), _ptr(v_cache), _ptr(blocks), blocks.numel(),
                ctypes.c_void_p(host.data_ptr()), _stream(k_cache))
    _check("pa_swap_out" if out else "pa_swap_in", st)


def pa_swap_out(k_cache, v_cache, blocks, host, *, num_kv_heads, head_dim, block_size):
    """Copy blocks (int32 device tensor) of both caches into `host` (uint8
    CPU tensor in pinned memory, e.g. torch.empty(..., pin_memory=True)): the
    K blocks in list order, then the V blocks.  Asynchronous on the current
    stream.  See include/pa_blocks.h."""
    _swap(True, k_cache, v_cache, blocks, host, num_kv_heads, head_dim, block_size)


def pa_swap_in(k_cache, v_cache, blocks, host, *, num_kv_heads, head_dim, block_size):
    """Copy the i-th K and V blocks of `host` (as pa_swap_out wrote it) into
    blocks[i] of the caches.  Asynchronous on the current stream."""
    _swap(False, k_cache, v_cache, blocks, host, num_kv_heads, head_dim, block_size)


class BlockManager:
    """Host block manager of include/pa_blocks.h (FIFO free list, reference
    counts, exact prefix keys with a model key, fork, copy-on-write).  Thin
    wrapper: every method is one C call."""

    def __init__(self, num_blocks, block_size):
        L = _load()
        h = ctypes.c_void_p()
        _check("pa_bm_create", L.pa_bm_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            _load().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq, tokens, model_key=0):
        """Returns the number of reused (prefix-shared) blocks."""
        arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        reused = ctypes.c_int32()
        _check("pa_bm_add_sequence", _load().pa_bm_add_sequence(
            self._h, seq, arr, len(tokens), model_key, ctypes.byref(reused)))
        return reused.value

    def add_ring_sequence(self, seq, n, window):
        """A local layer's sequence of n tokens with a ring table for a
        window of `window` tokens; returns the ring's entry count."""
        e = ctypes.c_int32()
        _check("pa_bm_add_ring_sequence", _load().pa_bm_add_ring_sequence(
            self._h, seq, int(n), int(window), ctypes.byref(e)))
        return e.value

    def slots(self, seq, first, count):
        """numpy int64 slots of positions first .. first + count - 1 (-1
        where the sequence holds no block for a position)."""
        import numpy as np
        out = np.empty(max(int(count), 1), dtype=np.int64)
        _check("pa_bm_slots", _load().pa_bm_slots(
            self._h, seq, int(first), int(count), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return out[:int(count)]

    def fork(self, parent, child):
        _check("pa_bm_fork", _load().pa_bm_fork(self._h, parent, child))

    def append_token(self, seq, token):
        """Returns (slot, copy_src, copy_dst); copy ids are -1 when no
        copy-on-write is needed."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_bm_append_token", _load().pa_bm_append_token(
            self._h, seq, int(token), ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def free_sequence(self, seq):
        _check("pa_bm_free_sequence", _load().pa_bm_free_sequence(self._h, seq))

    def trim(self, seq, keep_tokens):
        """Release the blocks holding only positions before the last
        keep_tokens tokens; returns how many table entries were released."""
        n = ctypes.c_int32()
        _check("pa_bm_trim", _load().pa_bm_trim(self._h, seq, keep_tokens, ctypes.byref(n)))
        return n.value

    def swap_out(self, seq):
        """Release the blocks only `seq` holds; returns them (to copy out
        with pa_swap_out), in table order."""
        n = ctypes.c_int32()
        cap = len(self.table(seq))
        out = (ctypes.c_int32 * max(cap, 1))()
        _check("pa_bm_swap_out", _load().pa_bm_swap_out(self._h, seq, out, cap, ctypes.byref(n)))
        return list(out[:n.value])

    def swap_in(self, seq):
        """New blocks for the swapped entries of `seq` (for pa_swap_in), in
        the order swap_out listed the blocks they replace."""
        n = ctypes.c_int32()
        cap = len(self.table(seq))
        out = (ctypes.c_int32 * max(cap, 1))()
        _check("pa_bm_swap_in", _load().pa_bm_swap_in(self._h, seq, out, cap, ctypes.byref(n)))
        return list(out[:n.value])

    def num_free(self):
        return _load().pa_bm_num_free(self._h)

    def length(self, seq):
        n, b = ctypes.c_int32(), ctypes.c_int32()
        _check("pa_bm_sequence_info", _load().pa_bm_sequence_info(self._h, seq, ctypes.byref(n), ctypes.byref(b)))
        return n.value

    def table(self, seq):
        n, b = ctypes.c_int32(), ctypes.c_int32()
        L = _load()
        _check("pa_bm_sequence_info", L.pa_bm_sequence_info(self._h, seq, ctypes.byref(n), ctypes.byref(b)))
        out = (ctypes.c_int32 * max(b.value, 1))()
        _check("pa_bm_block_table", L.pa_bm_block_table(self._h, seq, out, b.value))
        return list(out[:b.value])

    def refcount(self, block):
        r = ctypes.c_int32()
        _check("pa_bm_refcount", _load().pa_bm_refcount(self._h, block, ctypes.byref(r)))
        return r.value

    def stats(self):
        h, m = ctypes.c_int64(), ctypes.c_int64()
        _check("pa_bm_stats", _load().pa_bm_stats(self._h, ctypes.byref(h), ctypes.byref(m)))
        return h.value, m.value

    def batch(self, seqs, max_blocks):
        """Host numpy arrays (block_tables [n, max_blocks] int32, padded with
        -1; seq_lens [n] int32) for a decode batch of these sequences."""
        import numpy as np
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*seqs)
        bt = np.empty((n, max_blocks), dtype=np.int32)
        sl = np.empty(n, dtype=np.int32)
        _check("pa_bm_batch", _load().pa_bm_batch(
            self._h, ids, n, max_blocks, bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return bt, sl


def pa_decode_window(q, k_cache, v_cache, block_tables, seq_lens, window, scale, out=None, *,
                     num_kv_heads, block_size, partition_tokens=0, workspace=None):
    """Sliding-window decode over a bf16 cache: each sequence attends to its
    last `window` tokens (0 = all).  See pa_decode_window in include/pa.h."""
    return _decode(False, q, k_cache, v_cache, block_tables, seq_lens, scale, out, num_kv_heads,
                   block_size, 1.0, 1.0, partition_tokens, workspace, window)


def pa_decode_window_fp8(q, k_cache, v_cache, block_tables, seq_lens, window, scale, k_scale,
                         v_scale, out=None, *, num_kv_heads, block_size, partition_tokens=0,
                         workspace=None):
    """Sliding-window decode over an e4m3fn cache."""
    return _decode(True, q, k_cache, v_cache, block_tables, seq_lens, scale, out, num_kv_heads,
                   block_size, k_scale, v_scale, partition_tokens, workspace, window)


def _decode_append(fp8, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, out,
                   num_kv_heads, block_size, k_scale, v_scale, window, partition_tokens, workspace,
                   ring=False):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("pa_decode_append needs device tensors")
    _need(q, "q", torch.bfloat16, dev, 3)
    S, Hq, D = q.shape
    if ring and (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if not ring or k_new is not None:
        _need(k_new, "k_new", torch.bfloat16, dev, shape=(S, num_kv_heads, D))
        _need(v_new, "v_new", torch.bfloat16, dev, shape=(S, num_kv_heads, D))
    cdt = torch.uint8 if fp8 else torch.bfloat16
    _need(k_cache, "k_cache", cdt, dev)
    _need(v_cache, "v_cache", cdt, dev, shape=tuple(k_cache.shape))
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    _need(seq_lens, "seq_lens", torch.int32, dev, shape=(S,))
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, shape=(S, Hq, D))
    desc = make_desc(k_cache, num_kv_heads, D, block_size)
    maxb = block_tables.shape[1]
    L = _load()
    with torch.cuda.device(dev):
        if workspace is None:
            need = L.pa_decode_workspace_size(ctypes.byref(desc), S, Hq, maxb, partition_tokens)
            if need == 0 and S > 0:
                raise PagedAttentionError("pa_decode_workspace_size", -6,
                                          "no gfx950 device or invalid sizes")
            workspace = torch.zeros(max(int(need), 1), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, dev)
        kn = _ptr(k_new) if k_new is not None else None
        vn = _ptr(v_new) if v_new is not None else None
        args = [ctypes.byref(desc), _ptr(q), kn, vn, S, Hq, _ptr(k_cache), _ptr(v_cache),
                _ptr(block_tables), maxb, _ptr(seq_lens), int(window), float(scale)]
        if fp8:
            args += [float(k_scale), float(v_scale)]
        args += [_ptr(out), int(partition_tokens), _ptr(workspace), workspace.numel(), _stream(q)]
        name = ("pa_decode_ring" if ring else "pa_decode_append") + ("_fp8" if fp8 else "")
        st = getattr(L, name)(*args)
    _check(name, st)
    return out


def pa_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, out=None, *,
                     num_kv_heads, block_size, window=0, partition_tokens=0, workspace=None):
    """Write each sequence's new token (k_new, v_new [S, Hkv, D] bf16) at
    position seq_lens[s] - 1 and decode, in one launch: the same caches and
    output as pa_cache_write then pa_decode_window.  See pa_decode_append in
    include/pa.h."""
    return _decode_append(False, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, out,
                          num_kv_heads, block_size, 1.0, 1.0, window, partition_tokens, workspace)


def pa_decode_append_fp8(q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, k_scale,
                         v_scale, out=None, *, num_kv_heads, block_size, window=0, partition_tokens=0,
                         workspace=None):
    """pa_decode_append over an e4m3fn cache: the new token is stored as
    codes of x / scale, as pa_cache_write_fp8 stores it."""
    return _decode_append(True, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, out,
                          num_kv_heads, block_size, k_scale, v_scale, window, partition_tokens, workspace)


def pa_decode_ring(q, k_cache, v_cache, ring_tables, seq_lens, window, scale, out=None, *, num_kv_heads,
                   block_size, k_new=None, v_new=None, partition_tokens=0, workspace=None):
    """Local-layer decode from ring tables ([S, ring_entries] int32, logical
    block b at entry b % ring_entries) over a bf16 cache; with k_new / v_new
    the new tokens are written first in the same launch.  See pa_decode_ring
    in include/pa.h."""
    return _decode_append(False, q, k_new, v_new, k_cache, v_cache, ring_tables, seq_lens, scale, out,
                          num_kv_heads, block_size, 1.0, 1.0, window, partition_tokens, workspace, ring=True)


def pa_decode_ring_fp8(q, k_cache, v_cache, ring_tables, seq_lens, window, scale, k_scale, v_scale, out=None,
                       *, num_kv_heads, block_size, k_new=None, v_new=None, partition_tokens=0,
                       workspace=None):
    """pa_decode_ring over an e4m3fn cache."""
    return _decode_append(True, q, k_new, v_new, k_cache, v_cache, ring_tables, seq_lens, scale, out,
                          num_kv_heads, block_size, k_scale, v_scale, window, partition_tokens, workspace,
                          ring=True)


# -- query-aware page selection (include/pa_quest.h) -------------------------

def summary_shape(num_blocks, num_kv_heads, head_dim):
    """Shape of a pool's summary array: [num_blocks, head_dim / 4,
    num_kv_heads, 4] (include/pa_quest.h)."""
    return (num_blocks, head_dim // 4, num_kv_heads, 4)


def quest_summaries(k_cache, *, num_kv_heads, head_dim, block_size):
    """A new summary array for the pool of ``k_cache``: int32 device tensor
    of summary_shape() (uint32 words, (max bf16 << 16) | min bf16), every
    word empty."""
    desc = make_desc(k_cache, num_kv_heads, head_dim, block_size)
    words = torch.empty(summary_shape(desc.num_blocks, num_kv_heads, head_dim), dtype=torch.int32,
                        device=k_cache.device)
    with torch.cuda.device(k_cache.device):
        st = _load().pa_quest_clear(ctypes.byref(desc), _ptr(words), _stream(k_cache))
    _check("pa_quest_clear", st)
    return words


def _summary_args(k_cache, summaries, num_kv_heads, head_dim, block_size):
    dev = k_cache.device
    _need(k_cache, "k_cache", k_cache.dtype, dev)
    desc = make_desc(k_cache, num_kv_heads, head_dim, block_size)
    _need(summaries, "summaries", torch.int32, dev, shape=summary_shape(desc.num_blocks, num_kv_heads, head_dim))
    eb = 2 if k_cache.dtype == torch.bfloat16 else 1
    return dev, desc, eb


def _quest_cache_write(fp8, k, v, slot_mapping, k_cache, v_cache, summaries, block_size, k_scale, v_scale):
    dev = k.device
    _need(k, "k", torch.bfloat16, dev, 3)
    T, Hkv, D = k.shape
    _need(v, "v", torch.bfloat16, dev, shape=k.shape)
    _need(slot_mapping, "slot_mapping", torch.int64, dev, shape=(T,))
    _need(k_cache, "k_cache", torch.uint8 if fp8 else torch.bfloat16, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev, shape=tuple(k_cache.shape))
    desc = make_desc(k_cache, Hkv, D, block_size)
    _need(summaries, "summaries", torch.int32, dev, shape=summary_shape(desc.num_blocks, Hkv, D))
    L = _load()
    with torch.cuda.device(dev):
        if fp8:
            st = L.pa_quest_cache_write_fp8(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping), T,
                                            _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale),
                                            _ptr(summaries), _stream(k))
        else:
            st = L.pa_quest_cache_write(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping), T,
                                        _ptr(k_cache), _ptr(v_cache), _ptr(summaries), _stream(k))
    _check("pa_quest_cache_write" + ("_fp8" if fp8 else ""), st)


def pa_quest_cache_write(k, v, slot_mapping, k_cache, v_cache, summaries, *, block_size):
    """pa_cache_write and the summary update in one launch (no two tokens of
    the call in one block).  See include/pa_quest.h."""
    _quest_cache_write(False, k, v, slot_mapping, k_cache, v_cache, summaries, block_size, 1.0, 1.0)


def pa_quest_cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, summaries, *, block_size):
    """The same into an e4m3fn cache."""
    _quest_cache_write(True, k, v, slot_mapping, k_cache, v_cache, summaries, block_size, k_scale, v_scale)


def pa_quest_update(k_cache, slot_mapping, summaries, *, num_kv_heads, head_dim, block_size):
    """Keep the summaries current after pa_cache_write(_fp8) of slot_mapping
    (int64 device tensor), on the same stream.  See include/pa_quest.h."""
    dev, desc, eb = _summary_args(k_cache, summaries, num_kv_heads, head_dim, block_size)
    _need(slot_mapping, "slot_mapping", torch.int64, dev, 1)
    with torch.cuda.device(dev):
        st = _load().pa_quest_update(ctypes.byref(desc), eb, _ptr(k_cache), _ptr(slot_mapping),
                                     slot_mapping.numel(), _ptr(summaries), _stream(k_cache))
    _check("pa_quest_update", st)


def pa_quest_summarize(k_cache, blocks, counts, summaries, *, num_kv_heads, head_dim, block_size):
    """Recompute the summaries of blocks[i] from their first counts[i]
    tokens (int32 device tensors)."""
    dev, desc, eb = _summary_args(k_cache, summaries, num_kv_heads, head_dim, block_size)
    _need(blocks, "blocks", torch.int32, dev, 1)
    _need(counts, "counts", torch.int32, dev, shape=tuple(blocks.shape))
    with torch.cuda.device(dev):
        st = _load().pa_quest_summarize(ctypes.byref(desc), eb, _ptr(k_cache), _ptr(blocks), _ptr(counts),
                                        blocks.numel(), _ptr(summaries), _stream(k_cache))
    _check("pa_quest_summarize", st)


def pa_quest_select(q, summaries, block_tables, seq_lens, budget, *, num_kv_heads, block_size,
                    sel_tables=None, sel_lens=None, workspace=None):
    """Choose the `budget` best pages per (sequence, KV head).  Returns
    (sel_tables [S * Hkv, budget] int32, sel_lens [S * Hkv] int32)."""
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    S, Hq, D = q.shape
    _need(summaries, "summaries", torch.int32, dev, 4)
    if tuple(summaries.shape[1:]) != summary_shape(1, num_kv_heads, D)[1:]:
        raise ValueError("summaries must be [num_blocks, head_dim / 4, num_kv_heads, 4]")
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    if block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per sequence")
    _need(seq_lens, "seq_lens", torch.int32, dev, shape=(S,))
    desc = CacheDesc(summaries.shape[0], block_size, num_kv_heads, D)
    units = S * num_kv_heads
    if sel_tables is None:
        sel_tables = torch.empty((units, budget), dtype=torch.int32, device=dev)
    if sel_lens is None:
        sel_lens = torch.empty((units,), dtype=torch.int32, device=dev)
    _need(sel_tables, "sel_tables", torch.int32, dev, shape=(units, budget))
    _need(sel_lens, "sel_lens", torch.int32, dev, shape=(units,))
    maxb = block_tables.shape[1]
    L = _load()
    if workspace is None:
        need = L.pa_quest_select_workspace_size(S, num_kv_heads, maxb)
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    with torch.cuda.device(dev):
        st = L.pa_quest_select(ctypes.byref(desc), _ptr(q), S, Hq, _ptr(summaries), _ptr(block_tables), maxb,
                               _ptr(seq_lens), int(budget), _ptr(sel_tables), _ptr(sel_lens), _ptr(workspace),
                               workspace.numel(), _stream(q))
    _check("pa_quest_select", st)
    return sel_tables, sel_lens


def _decode_quest(fp8, q, k_cache, v_cache, sel_tables, sel_lens, scale, out, num_kv_heads, block_size,
                  k_scale, v_scale, partition_tokens, workspace):
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    S, Hq, D = q.shape
    cdt = torch.uint8 if fp8 else torch.bfloat16
    _need(k_cache, "k_cache", cdt, dev)
    _need(v_cache, "v_cache", cdt, dev, shape=tuple(k_cache.shape))
    _need(sel_tables, "sel_tables", torch.int32, dev, 2)
    if sel_tables.shape[0] != S * num_kv_heads:
        raise ValueError("sel_tables must have one row per (sequence, KV head)")
    _need(sel_lens, "sel_lens", torch.int32, dev, shape=(S * num_kv_heads,))
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, shape=(S, Hq, D))
    desc = make_desc(k_cache, num_kv_heads, D, block_size)
    budget = sel_tables.shape[1]
    L = _load()
    with torch.cuda.device(dev):
        if workspace is None:
            need = L.pa_decode_quest_workspace_size(ctypes.byref(desc), S, Hq, budget, partition_tokens)
            if need == 0 and S > 0:
                raise PagedAttentionError("pa_decode_quest_workspace_size", -6,
                                          "no gfx950 device or invalid sizes")
            workspace = torch.zeros(max(int(need), 1), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, dev)
        args = [ctypes.byref(desc), _ptr(q), S, Hq, _ptr(k_cache), _ptr(v_cache), _ptr(sel_tables), budget,
                _ptr(sel_lens), float(scale)]
        if fp8:
            args += [float(k_scale), float(v_scale)]
        args += [_ptr(out), int(partition_tokens), _ptr(workspace), workspace.numel(), _stream(q)]
        name = "pa_decode_quest" + ("_fp8" if fp8 else "")
        st = getattr(L, name)(*args)
    _check(name, st)
    return out


def pa_decode_quest(q, k_cache, v_cache, sel_tables, sel_lens, scale, out=None, *, num_kv_heads,
                    block_size, partition_tokens=0, workspace=None):
    """Decode over the pages pa_quest_select chose (bf16 cache)."""
    return _decode_quest(False, q, k_cache, v_cache, sel_tables, sel_lens, scale, out, num_kv_heads,
                         block_size, 1.0, 1.0, partition_tokens, workspace)


def pa_decode_quest_fp8(q, k_cache, v_cache, sel_tables, sel_lens, scale, k_scale, v_scale, out=None, *,
                        num_kv_heads, block_size, partition_tokens=0, workspace=None):
    """Decode over the chosen pages of an e4m3fn cache."""
    return _decode_quest(True, q, k_cache, v_cache, sel_tables, sel_lens, scale, out, num_kv_heads,
                         block_size, k_scale, v_scale, partition_tokens, workspace)


# -- shared-prefix (cascade) decode (include/pa_cascade.h) --------------------

class CascadePlan:
    """Shared-prefix plan of one batch, built on the host from its block
    tables and lengths (numpy int32 arrays, as BlockManager.batch returns
    them) and copied to ``device``.  ``info`` holds the sizes and token
    counts; ``segments`` is [num_segments, 4] (first block, blocks, members
    offset, members) and ``members`` the member sequences, for inspection."""

    def __init__(self, block_tables, seq_lens, *, block_size, num_kv_heads, num_q_heads, chunk_tokens=1024,
                 device="cuda"):
        import numpy as np
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if bt.ndim != 2 or sl.shape != (bt.shape[0],):
            raise ValueError("block_tables must be [S, max_blocks] and seq_lens [S]")
        S, maxb = bt.shape
        L = _load()
        h = ctypes.c_void_p()
        _check("pa_cascade_plan_build", L.pa_cascade_plan_build(
            bt.ctypes.data_as(ctypes.c_void_p), S, maxb, sl.ctypes.data_as(ctypes.c_void_p), block_size,
            num_kv_heads, num_q_heads, chunk_tokens, ctypes.byref(h)))
        try:
            info = CascadePlanInfo()
            _check("pa_cascade_plan_get_info", L.pa_cascade_plan_get_info(h, ctypes.byref(info)))
            arr = lambda n: np.zeros(max(int(n), 1), dtype=np.int32)
            items, seg_blocks, members = arr(8 * info.num_items), arr(info.num_seg_blocks), arr(info.num_members)
            parts_off, parts = arr(S + 1), arr(info.num_parts)
            ptab, plens, segs = arr(S * maxb), arr(S), arr(4 * info.num_segments)
            ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
            _check("pa_cascade_plan_export", L.pa_cascade_plan_export(
                h, ptr(items), ptr(seg_blocks), ptr(members), ptr(parts_off), ptr(parts), ptr(ptab), ptr(plens),
                ptr(segs)))
        finally:
            L.pa_cascade_plan_destroy(h)
        self.info = {f: getattr(info, f) for f, _ in CascadePlanInfo._fields_}
        self.num_seqs, self.max_blocks = S, maxb
        self.segments = segs[:4 * info.num_segments].reshape(-1, 4)
        self.members = members[:info.num_members]
        self.items_host = items[:8 * info.num_items].reshape(-1, 8)
        self.parts_off_host, self.parts_host = parts_off, parts[:info.num_parts]
        self.private_tables_host = ptab[:S * maxb].reshape(S, maxb)
        self.private_lens_host = plens[:S]
        dev = torch.device(device)
        t = lambda a: torch.from_numpy(a).to(dev)
        self._dev = [t(items), t(seg_blocks), t(members), t(parts_off), t(parts), t(ptab), t(plens)]
        d = self._dev
        self.device_plan = CascadeDevicePlan(_ptr(d[0]), info.num_items, _ptr(d[1]), _ptr(d[2]), _ptr(d[3]),
                                             _ptr(d[4]), info.num_slots, _ptr(d[5]), _ptr(d[6]))


def _decode_cascade(fp8, q, k_cache, v_cache, plan, scale, out, num_kv_heads, block_size, k_scale, v_scale,
                    partition_tokens, workspace):
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    S, Hq, D = q.shape
    if S != plan.num_seqs:
        raise ValueError("the plan was built for another batch size")
    cdt = torch.uint8 if fp8 else torch.bfloat16
    _need(k_cache, "k_cache", cdt, dev)
    _need(v_cache, "v_cache", cdt, dev, shape=tuple(k_cache.shape))
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, shape=(S, Hq, D))
    desc = make_desc(k_cache, num_kv_heads, D, block_size)
    L = _load()
    with torch.cuda.device(dev):
        if workspace is None:
            need = L.pa_decode_cascade_workspace_size(ctypes.byref(desc), S, Hq, plan.max_blocks,
                                                      plan.info["num_slots"], partition_tokens)
            if need == 0 and S > 0:
                raise PagedAttentionError("pa_decode_cascade_workspace_size", -6,
                                          "no gfx950 device or invalid sizes")
            workspace = torch.zeros(max(int(need), 1), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, dev)
        args = [ctypes.byref(desc), _ptr(q), S, Hq, _ptr(k_cache), _ptr(v_cache), plan.max_blocks,
                ctypes.byref(plan.device_plan), float(scale)]
        if fp8:
            args += [float(k_scale), float(v_scale)]
        args += [_ptr(out), int(partition_tokens), _ptr(workspace), workspace.numel(), _stream(q)]
        name = "pa_decode_cascade" + ("_fp8" if fp8 else "")
        st = getattr(L, name)(*args)
    _check(name, st)
    return out


def pa_decode_cascade(q, k_cache, v_cache, plan, scale, out=None, *, num_kv_heads, block_size,
                      partition_tokens=0, workspace=None):
    """Decode of the batch ``plan`` (a CascadePlan) was built from, attending
    to its shared segments once for all of their sequences (bf16 cache)."""
    return _decode_cascade(False, q, k_cache, v_cache, plan, scale, out, num_kv_heads, block_size, 1.0, 1.0,
                           partition_tokens, workspace)


def pa_decode_cascade_fp8(q, k_cache, v_cache, plan, scale, k_scale, v_scale, out=None, *, num_kv_heads,
                          block_size, partition_tokens=0, workspace=None):
    """The same over an e4m3fn cache."""
    return _decode_cascade(True, q, k_cache, v_cache, plan, scale, out, num_kv_heads, block_size, k_scale,
                           v_scale, partition_tokens, workspace)
