"""Pins for the oracle's group-wise low-bit KV codec (ReKV, section 2.2).

* The payload size of an encoded prefix equals eq. (7) and reproduces the
  page's figures for the Qwen2.5-7B shape at 8K tokens: 8.25 MiB per Q8
  layer, 179.75 MiB for a 15-layer Q8 prefix plus the 56 MiB boundary, 231 MiB
  for all 28 layers (tests/golden/rekv_bytes.json).
* Codes worked out by hand from the reading (symmetric groups of 64, fp16
  scale = max|x| / q_max, codes x / scale rounded to nearest with ties to
  even, Q4 low nibble first), including an exact tie that a per-group
  reciprocal would round the other way.
* Codes equal the nearest integer to the exact rational quotient x / scale
  wherever that quotient is not within fp32 rounding of a half-integer.
* The symmetric quantizer's error bound, zero groups, pack/unpack inverses,
  and the payload layout decoding back to the same values.
"""

import numpy as np
import pytest

from oracle.accounting import lowbit_payload_bytes
from oracle.codec import (GROUP, decode, dequantize_groups, encode, pack, payload_bytes, q_max,
                          quantize_groups, unpack)


def test_payload_size_is_eq7_and_the_pages_figures(golden):
    g = golden("rekv_bytes.json")
    E = 2 * g["seq"] * g["kv_heads"] * g["head_dim"]           # KV elements of one layer
    mib = 1 << 20
    assert payload_bytes(E, 8) / mib == g["q8_layer_mib"]
    assert (g["q8_prefix_layers"] * payload_bytes(E, 8) / mib + g["boundary_mib"]
            == g["q8_prefix_plus_boundary_mib"])
    assert g["layers"] * payload_bytes(E, 8) / mib == g["full_q8_mib"]
    for bits in (4, 8):
        assert payload_bytes(E, bits) == lowbit_payload_bytes(1, g["seq"], g["kv_heads"], g["head_dim"],
                                                             bits, GROUP, 0)
    # the encoder's actual output has exactly that many bytes
    rng = np.random.default_rng(0)
    k = rng.standard_normal((37, 4, 128)).astype(np.float32)
    v = rng.standard_normal((37, 4, 128)).astype(np.float32)
    for bits in (4, 8):
        assert encode(k, v, bits).size == payload_bytes(2 * k.size, bits)


def test_q8_hand_worked_group():
    # max|x| = fp32(1.27); / 127 = 0.0099999998 -> fp16 0.01000213623046875;
    # 1.27 / s = 126.97 -> 127, -0.5 / s = -49.99 -> -50, 0.02 / s = 2.00 -> 2
    x = np.zeros(64, np.float32)
    x[:3] = [1.27, -0.5, 0.02]
    codes, scales = quantize_groups(x, 8)
    assert scales.dtype == np.float16 and float(scales[0]) == 0.01000213623046875
    assert codes[:4].tolist() == [127, -50, 2, 0] and not codes[4:].any()


def test_q4_hand_worked_group_and_packing():
    # max 7 -> scale exactly 1; -3.5 is a tie -> -4 (even); 0.4 -> 0
    x = np.zeros(64, np.float32)
    x[:4] = [7.0, -3.5, 1.0, 0.4]
    codes, scales = quantize_groups(x, 4)
    assert float(scales[0]) == 1.0 and codes[:4].tolist() == [7, -4, 1, 0]
    packed = pack(codes, 4)
    assert packed.size == 32 and packed[0] == 0xC7 and packed[1] == 0x01   # low nibble first
    assert unpack(packed, 4, 64).tolist() == codes.tolist()


def test_exact_tie_is_divided_not_multiplied_by_a_reciprocal():
    # max 1.53125 -> scale 1.53125 / 7 = 0.21875 = 7/32 exactly (fp16 exact);
    # 1.421875 = 6.5 * 7/32 exactly, an exact tie -> 6 (even).  The fp32
    # reciprocal 1/0.21875 = 4.5714285... is rounded up, and 1.421875 times it
    # lands above 6.5, so a reciprocal-based code would be 7.  Likewise
    # 0.65625 = 3 * 7/32 -> 3 and -1.421875 -> -6.
    x = np.zeros(64, np.float32)
    x[:4] = [1.53125, 1.421875, 0.65625, -1.421875]
    codes, scales = quantize_groups(x, 4)
    assert float(scales[0]) == 0.21875
    assert codes[:4].tolist() == [7, 6, 3, -6]
    inv = np.float32(1) / np.float32(0.21875)
    assert np.rint(np.float32(np.float32(1.421875) * inv)) == 7       # the other reading differs here


@pytest.mark.parametrize("bits", [4, 8])
def test_codes_round_the_exact_quotient(bits):
    """Where the exact quotient x / scale16 (rational arithmetic) lies more
    than 2^-16 from a half-integer, fp32 rounding cannot move it across one,
    so the code must be its nearest integer, clamped."""
    from fractions import Fraction
    rng = np.random.default_rng(100 + bits)
    x = (rng.standard_normal((24, 128)) * rng.uniform(0.05, 30, size=(24, 1))).astype(np.float32)
    x = synth_bf16(x)
    codes, scales = quantize_groups(x, bits)
    qm = q_max(bits)
    checked = 0
    for r in range(x.shape[0]):
        for j in range(x.shape[1]):
            s = Fraction(float(np.float32(scales[r, j // GROUP])))
            t = Fraction(float(x[r, j])) / s
            frac = t - (t.numerator // t.denominator)
            if abs(frac - Fraction(1, 2)) <= Fraction(1, 1 << 16):
                continue
            near = t.numerator // t.denominator + (1 if frac > Fraction(1, 2) else 0)
            assert codes[r, j] == max(-qm, min(qm, near)), (r, j)
            checked += 1
    assert checked > 0.99 * x.size


def synth_bf16(x):
    """Round fp32 values to bf16 (nearest, ties to even) and back, so the
    inputs are bf16 pool values."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def test_zero_group_and_clamp():
    x = np.zeros((2, 128), np.float32)
    x[1, 64:] = 3.0                      # second group of row 1: all equal, codes q_max
    codes, scales = quantize_groups(x, 8)
    assert (scales[0] == 0).all() and scales[1, 0] == 0 and not codes[0].any()
    assert (codes[1, 64:] == 127).all()
    assert (np.abs(codes.astype(int)) <= 127).all()


@pytest.mark.parametrize("bits", [4, 8])
def test_round_trip_error_bound(bits):
    rng = np.random.default_rng(bits)
    x = (rng.standard_normal((50, 8, 128)) * rng.uniform(0.01, 20, size=(50, 8, 1))).astype(np.float32)
    codes, scales = quantize_groups(x, bits)
    back = dequantize_groups(codes, scales)
    sf = scales.astype(np.float64).repeat(GROUP, axis=-1)
    amax = np.abs(x.astype(np.float64)).reshape(50, 8, 2, 64).max(-1).repeat(GROUP, axis=-1)
    # nearest code under the stored scale: half a step, plus the clamp when the
    # fp16 rounding of the scale went down (at most 2^-11 relative)
    assert (np.abs(x - back) <= 0.5 * sf + amax * 2.0 ** -10).all()
    assert np.abs(codes.astype(int)).max() == q_max(bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_unpack_and_payload_layout(bits):
    rng = np.random.default_rng(10 + bits)
    c = rng.integers(-q_max(bits), q_max(bits) + 1, size=640).astype(np.int8)
    assert unpack(pack(c, bits), bits, c.size).tolist() == c.tolist()
    k = rng.standard_normal((9, 2, 64)).astype(np.float32)
    v = rng.standard_normal((9, 2, 64)).astype(np.float32)
    dk, dv = decode(encode(k, v, bits), k.shape, bits)
    assert np.array_equal(dk, dequantize_groups(*quantize_groups(k, bits)))
    assert np.array_equal(dv, dequantize_groups(*quantize_groups(v, bits)))
