"""OCP fp8 e4m3fn codec, written from the format's definition (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Format (OCP 8-bit floating point, E4M3 "fn" flavour): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, no infinities.  Exponent field 0 holds the
subnormals m * 2**-9; the pattern S.1111.111 is NaN, so the largest finite
magnitude is S.1111.110 = 1.75 * 2**8 = 448.

The pages ask for an fp8 KV cache that "roughly halves" the cache
("KV Cache Engineering for LLM Serving", section 8 "Quantization"; the
rajatmohan.com serving design, "Offloading and the memory hierarchy").  The
same section's quantizer rounds with ``rint`` (round half to even) and clips
to the largest code; this codec does the same for e4m3: round to the nearest
representable value, ties to the even mantissa, and saturate to +-448 instead
of overflowing.  NaN keeps its sign (0x7F / 0xFF).  The pages say nothing
about NaN; that reading is recorded in the design notes.
"""

import numpy as np

MAX_FINITE = 448.0
_NAN_CODE = 0x7F


def decode(codes):
    """e4m3fn codes (uint8 array) -> exact float64 values (NaN for 0x7F/0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man.astype(np.float64) * 2.0 ** -9
    nrm = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    mag = np.where(exp == 0, sub, nrm)
    mag = np.where((c & 0x7F) == _NAN_CODE, np.nan, mag)
    return sign * mag


def _code_of_exact(mag):
    """Code (without sign) of a non-negative float64 that is exactly an
    e4m3fn finite value."""
    code = np.zeros(mag.shape, dtype=np.int64)
    sub = mag < 2.0 ** -6
    code[sub] = np.rint(mag[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        f, e = np.frexp(mag[nrm])          # mag = f * 2**e, f in [0.5, 1)
        unbiased = e - 1                   # mag = (2f) * 2**(e-1), 2f in [1, 2)
        man = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
        code[nrm] = ((unbiased + 7) << 3) | man
    return code


def encode_rne_sat(x):
    """float32 (or exactly-float32 float64) values -> e4m3fn codes (uint8).

    Round to nearest, ties to even mantissa, saturating at +-448; NaN -> 0x7F
    with the input's sign; -0 and negative values that round to zero -> 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    # Quantum of the binade that holds a: 2**(e-3) for normals (e >= -6),
    # 2**-9 for the subnormal range.
    e = np.full(a.shape, -6, dtype=np.int64)
    pos = a >= 2.0 ** -6
    if np.any(pos):
        _, fe = np.frexp(a[pos])
        e[pos] = fe - 1
    quantum = np.exp2((e - 3).astype(np.float64))
    n = np.rint(a / quantum)              # a / quantum is exact: a is a float32
    r = n * quantum                       # may step up one binade: still exact
    r = np.minimum(r, MAX_FINITE)         # saturate (ties at 464 already -> 448)
    code = _code_of_exact(r)
    code = np.where(nan, _NAN_CODE, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def quantize(x_f32, scale):
    """Cache-write encoding of one tensor with a per-tensor scale.

    inv = float32(1 / scale), correctly rounded; y = float32(x * inv) with one
    round-to-nearest-even float32 multiply; code = encode_rne_sat(y).
    The stored code therefore represents y, and the value it stands for is
    decode(code) * scale.
    """
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.asarray(x_f32, dtype=np.float32) * inv
    return encode_rne_sat(y.astype(np.float32))


def dequantize(codes, scale):
    """decode(code) * scale, exact in float64."""
    return decode(codes) * float(np.float32(scale))
