"""Oracle fp8 e4m3fn codec, pinned to the format definition and to torch's
own float8_e4m3fn cast (a library routine) over every bf16 bit pattern."""

import numpy as np
import pytest
import torch

from oracle import e4m3

ALL_BF16 = np.arange(65536, dtype=np.uint32)


def bf16_values():
    return (ALL_BF16 << 16).view(np.float32)


def test_decode_all_codes():
    v = e4m3.decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    fin = np.delete(np.arange(256), [0x7F, 0xFF])
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    assert v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    # Matches torch's decode of the same bytes.
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(v[fin], t[fin])
    # Positive finite codes are strictly increasing.
    assert np.all(np.diff(v[:0x7F]) > 0)


def test_encode_roundtrip_of_exact_values():
    codes = np.delete(np.arange(256, dtype=np.uint8), [0x7F, 0xFF])
    vals = e4m3.decode(codes)
    assert np.array_equal(e4m3.encode_rne_sat(vals), codes)


def _torch_ref(y32):
    """torch's cast after clamping into the finite range: the same as a
    saturating round-to-nearest-even encode."""
    t = torch.from_numpy(np.clip(y32, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [1.0, 0.0123, 1 / 448, 3.75, 1e-3, 2.0 ** -12, 97.0])
def test_quantize_matches_library_cast_all_bf16(scale):
    x = bf16_values()
    ours = e4m3.quantize(x, scale)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):
        y = x * inv
    ref = _torch_ref(y)
    fin = ~np.isnan(y)
    assert np.array_equal(ours[fin], ref[fin])
    # NaN keeps its sign.
    nan_codes = ours[~fin]
    assert set(nan_codes.tolist()) <= {0x7F, 0xFF}
    assert np.array_equal(nan_codes == 0xFF, np.signbit(y[~fin]))


def test_rounding_and_saturation_cases():
    cases = {
        1.0625: 0x38,   # tie between 1.0 and 1.125 -> even (1.0)
        1.1875: 0x3A,   # tie between 1.125 and 1.25 -> even (1.25)
        17.0: 0x58,     # tie between 16 and 18 -> 16
        464.0: 0x7E,    # tie between 448 and (unrepresentable) 480 -> 448
        465.0: 0x7E,    # saturates
        1e9: 0x7E,
        np.inf: 0x7E,
        -np.inf: 0xFE,
        2.0 ** -10: 0x00,  # tie between 0 and the smallest subnormal -> 0
        3 * 2.0 ** -11: 0x01,
        -1e-30: 0x80,
        -0.0: 0x80,
        2.0 ** -9 * 7.5: 0x08,  # rounds up into the first normal binade
    }
    for x, code in cases.items():
        assert int(e4m3.encode_rne_sat(np.array([x], dtype=np.float64))[0]) == code, x


def test_dequantize_scales_exactly():
    codes = np.array([0x38, 0x7E, 0x01, 0xB8], dtype=np.uint8)
    s = np.float32(0.01)
    assert np.array_equal(e4m3.dequantize(codes, s), e4m3.decode(codes) * float(s))
