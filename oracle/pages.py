"""The pages' own arithmetic, written out (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

These small functions restate the sizing rules and toy examples that the
pages print, so that tests can pin them to the printed numbers and so that
the benchmark can state its algorithmic byte counts from the same formula.
"""

import numpy as np


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_value):
    """Cache bytes one token costs: 2 (K and V) x layers x KV heads x head
    dimension x bytes per value.

    rajatmohan.com serving design, "What is actually being cached"
    (2 x 80 x 8 x 128 x 2 B, about 320 KB); "KV Cache Engineering for LLM
    Serving", "The cache formula" (the leading 2 counts keys and values; BF16
    is two bytes per value, FP8 one).
    """
    return 2 * layers * kv_heads * head_dim * bytes_per_value


def sequence_cache_bytes(tokens, layers, kv_heads, head_dim, bytes_per_value):
    """Raw cache size of one sequence: per-token bytes times retained tokens
    ("KV Cache Engineering for LLM Serving", intro and section 1)."""
    return tokens * kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_value)


def gqa_kv_head(q_head, num_q_heads, num_kv_heads):
    """KV head read by a query head: q_head // (query heads per KV head)
    ("KV Cache Engineering for LLM Serving", section 1, GQA and MQA)."""
    return q_head // (num_q_heads // num_kv_heads)


def cached_scalars(kv_heads, tokens, head_size):
    """Scalars cached for one layer: 2 x KV heads x tokens x head size
    ("KV Cache Engineering for LLM Serving", section 1 example)."""
    return 2 * kv_heads * tokens * head_size


def pool_capacity_tokens(pool_bytes, bytes_per_token):
    """Whole tokens a fixed-size block pool holds
    ("KV Cache Engineering for LLM Serving", section 10, Paging)."""
    return pool_bytes // bytes_per_token


def symmetric_quantize(values, bits):
    """Symmetric max-abs quantizer with a single shared scale.

    scale = max|x| / largest code with largest = 2**(bits-1) - 1; codes are
    x / scale rounded half-to-even and clipped to +-largest; the restored
    values are codes * scale ("KV Cache Engineering for LLM Serving",
    section 8, Quantization).  Returns (codes, restored, scale).
    """
    values = np.asarray(values, dtype=np.float64)
    largest = 2 ** (bits - 1) - 1
    scale = np.max(np.abs(values)) / largest
    codes = np.clip(np.rint(values / scale), -largest, largest)
    return codes.astype(np.int64), codes * scale, scale
