"""Pins for the oracle's INT8 KV pages (TileInfer.jl docs, "KV cache",
section "INT8 cache").

Nothing here re-types the quantizer.  The checks are:
* values worked out by hand from the page's rule (scale = max|x| / 127,
  x ~ scale * code), including the rounding reading (ties to even);
* closed forms: a zero vector; the largest-magnitude element gets code
  +-127; the symmetric quantizer's error bound |x - scale * code| <= scale / 2
  (plus the float32 rounding of x / scale);
* placement by slot on the page's 4-slot example layout;
* brute force of the page's own formulation of attention over INT8 pages
  (key scale times the scores, value scale times the probabilities, scalar
  math.exp loops) against the oracle's dequantize-then-attend;
* invariance of paged INT8 attention to where pages sit, and a one-key
  closed form.
"""

import math

import numpy as np
import pytest

from oracle.attention import attend
from oracle.paging import Allocator
from oracle.quant import (attend_int8, dequantize, paged_attention_int8, quantize,
                          quantize_then_attend, store_rows_int8)


def test_hand_worked_vector():
    # max|x| = fp32(1.27) = 1.26999998...; / 127 = 0.0099999999857 rounds to
    # fp32(0.01) = 0.00999999977648; then 1.27 / 0.01 -> 127, -0.5 / 0.01 ->
    # -50.0000011 -> -50, 0.02 / 0.01 -> 2.0000000 -> 2, 0 -> 0.
    codes, scale = quantize(np.array([1.27, -0.5, 0.02, 0.0], np.float32))
    assert codes.tolist() == [127, -50, 2, 0]
    assert codes.dtype == np.int8
    assert scale.dtype == np.float32 and scale == np.float32(0.01)


def test_ties_round_to_even():
    # max|x| = 127/16 makes the scale exactly 1/16, so x = k.5 / 16 sits on a tie
    x = np.array([127 / 16, 2.5 / 16, 3.5 / 16, -0.5 / 16, -1.5 / 16, 0.5 / 16], np.float32)
    codes, scale = quantize(x)
    assert scale == np.float32(1 / 16)
    assert codes.tolist() == [127, 2, 4, 0, -2, 0]


def test_zero_vector():
    codes, scale = quantize(np.zeros((3, 64), np.float32))
    assert (codes == 0).all() and (scale == 0).all()


@pytest.mark.parametrize("magnitude", [1e-30, 1e-3, 1.0, 7.5, 1e30])
def test_peak_code_and_error_bound(magnitude):
    rng = np.random.default_rng(int(abs(math.log10(magnitude))) + 5)
    x = (rng.standard_normal((200, 128)) * magnitude).astype(np.float32)
    codes, scales = quantize(x)
    assert (scales > 0).all()
    peak = np.abs(x).argmax(axis=1)
    rows = np.arange(x.shape[0])
    assert (np.abs(codes[rows, peak].astype(int)) == 127).all()
    assert (np.sign(codes[rows, peak]) == np.sign(x[rows, peak])).all()
    assert np.abs(codes.astype(int)).max() <= 127
    # rounding to the nearest code: |x / s - code| <= 1/2, plus the float32
    # rounding of x / s (at most 127.5 * 2^-24)
    err = np.abs(x.astype(np.float64) - dequantize(codes, scales))
    bound = scales.astype(np.float64)[:, None] * (0.5 + 127.5 * 2.0 ** -24)
    assert (err <= bound).all()


def test_input_must_be_float32_exact():
    with pytest.raises(ValueError):
        quantize(np.array([0.1, 0.2]))          # float64 values not exact in fp32


def test_store_places_codes_and_scales_by_slot():
    # the 4-slot block layout of "KV Cache Management and PagedAttention":
    # B's positions 0..3 in physical block 3, 4..6 in block 0
    ps, hkv, d = 4, 2, 8
    codes = np.full((6, hkv, ps, d), -1, np.int8)
    scales = np.full((6, hkv, ps), np.nan, np.float32)
    rng = np.random.default_rng(4)
    rows = rng.standard_normal((7, hkv, d)).astype(np.float32)
    slots = [12, 13, 14, 15, 0, 1, 2]
    store_rows_int8(codes, scales, slots + [-1], list(rows) + [rows[0]])
    for t, slot in enumerate(slots):
        c, s = quantize(rows[t])
        assert np.array_equal(codes[slot // ps, :, slot % ps], c)
        assert np.array_equal(scales[slot // ps, :, slot % ps], s)
    # slot 3 of block 0 and blocks 1, 2, 4, 5 untouched
    assert (codes[0, :, 3] == -1).all() and np.isnan(scales[0, :, 3]).all()
    assert (codes[[1, 2, 4, 5]] == -1).all()


def _folded_bruteforce(q, kc, ks, vc, vs, scale):
    """The page's formulation, scalar by scalar: the key's scale multiplies its
    row of scores; the value's scale multiplies its probability before the PV
    product; the normaliser is the sum of the plain probabilities."""
    n, hq, d = q.shape
    L, hkv, _ = kc.shape
    grp = hq // hkv
    out = np.zeros((n, hq, d))
    for i in range(n):
        pos = L - n + i
        for h in range(hq):
            g = h // grp
            z = []
            for j in range(pos + 1):
                dot = sum(float(q[i, h, e]) * float(kc[j, g, e]) for e in range(d))
                z.append(scale * float(ks[j, g]) * dot)
            m = max(z)
            p = [math.exp(t - m) for t in z]
            den = sum(p)
            for e in range(d):
                out[i, h, e] = sum(p[j] * float(vs[j, g]) * float(vc[j, g, e]) for j in range(pos + 1)) / den
    return out


@pytest.mark.parametrize("n,L,hq,hkv,d", [(1, 1, 1, 1, 4), (2, 6, 4, 2, 8), (5, 9, 2, 1, 6)])
def test_int8_attention_matches_folded_bruteforce(n, L, hq, hkv, d):
    rng = np.random.default_rng(n * 100 + L)
    q = rng.standard_normal((n, hq, d)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((L, hkv, d)).astype(np.float32)
    v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    kc, ks = quantize(k)
    vc, vs = quantize(v)
    got = attend_int8(q, (kc, ks), (vc, vs), 0.4)
    expect = _folded_bruteforce(q, kc, ks, vc, vs, 0.4)
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-12)


def test_one_visible_key_returns_its_dequantized_value():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((3, 1, 16)).astype(np.float32)
    v = rng.standard_normal((3, 1, 16)).astype(np.float32)
    q = rng.standard_normal((3, 2, 16))
    out = quantize_then_attend(q, k, v, 0.25)
    vc, vs = quantize(v[0, 0])
    expect = np.array([float(vs) * float(c) for c in vc])
    assert np.array_equal(out[0, 0], expect) and np.array_equal(out[0, 1], expect)


def test_quantization_error_is_small():
    """Attention over the INT8 values stays close to attention over the exact
    ones (N(0,1) data: per-vector steps of about max|x| / 127)."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4, 8, 128)).astype(np.float32)
    k = rng.standard_normal((300, 2, 128)).astype(np.float32)
    v = rng.standard_normal((300, 2, 128)).astype(np.float32)
    exact = attend(q, k, v, 1 / math.sqrt(128))
    approx = quantize_then_attend(q, k, v, 1 / math.sqrt(128))
    err = np.abs(exact - approx)
    assert err.max() < 0.02 and err.mean() < 0.003
    # and it is not exact: the codes really are 8-bit
    assert err.max() > 1e-5


def test_paged_int8_attention_independent_of_page_placement():
    ps, hkv, d, hq = 4, 2, 8, 4
    rng = np.random.default_rng(10)
    lens = [7, 6, 11]
    k_rows = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    v_rows = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    q = rng.standard_normal((sum(lens), hq, d))
    cu = np.concatenate([[0], np.cumsum(lens)])
    outs = []
    for order in ([0, 1, 2, 3, 4, 5, 6, 7, 8], [8, 3, 5, 0, 7, 1, 6, 2, 4]):
        alloc = Allocator(9, ps, order)
        pools = [(np.zeros((9, hkv, ps, d), np.int8), np.zeros((9, hkv, ps), np.float32)) for _ in range(2)]
        tables = []
        for b, L in enumerate(lens):
            s = alloc.seq_new()
            alloc.reserve(s, L)
            sl = alloc.slots(s, 0, L)
            store_rows_int8(*pools[0], sl, k_rows[b])
            store_rows_int8(*pools[1], sl, v_rows[b])
            tables.append(alloc.block_table(s))
        outs.append(paged_attention_int8(q, cu, lens, tables, pools[0], pools[1], 0.3))
    assert np.array_equal(outs[0], outs[1])
    # and equal to the unpaged computation over each sequence's quantized rows
    for b, L in enumerate(lens):
        e = quantize_then_attend(q[cu[b]:cu[b + 1]], k_rows[b], v_rows[b], 0.3)
        assert np.array_equal(outs[0][cu[b]:cu[b + 1]], e)
