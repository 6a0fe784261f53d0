"""GPU parity of INT8 KV pages (TileInfer.jl docs, "KV cache", "INT8 cache")
against the oracle.

Bars: the stored codes and scales are bit-exact with the oracle's quantizer
(both take the same fp32 steps); attention is within the bf16 bars (2e-2
max-abs, 1e-2 mean-abs) of the fp64 oracle over the dequantized values.
Unwritten pool bytes are 0xFF (codes -1, scales NaN), so a read of a slot
that was never written would turn an output into NaN.

The pool layout read back here is the one include/pkv.h states for PKV_I8:
per (page, KV head) block, page_size rows of head_dim codes, then page_size
fp32 scales, padded to a multiple of 16 bytes.
"""

import numpy as np
import pytest
import torch

import oracle_path as ref
import pagedattention_pkv_store_amd as pkv
import synth
from conftest import ensure_library
from gpu_path import (DEV, Session, dev_tensor, host_f64, i64, run_decode, run_prefix, run_rewind,
                      run_spec)
from oracle.attention import attend
from oracle.quant import dequantize, quantize, quantize_then_attend, store_rows_int8

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def check_close(out, expect, what):
    assert out.shape == expect.shape, what
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - expect)
    assert err.max() <= BF16_MAX, f"{what}: max abs err {err.max():.3g}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3g}"


def unpack(pool: torch.Tensor, desc: pkv.PoolDesc):
    """(codes int8 [P][H][ps][D], scales float32 [P][H][ps], padding bytes)."""
    b = pool.view(torch.uint8).cpu().numpy()
    P, H, ps, D = desc.num_pages, desc.num_kv_heads, desc.page_size, desc.head_dim
    assert b.shape == (P, H, ps * D + ((4 * ps + 15) // 16) * 16)
    codes = np.ascontiguousarray(b[..., :ps * D]).view(np.int8).reshape(P, H, ps, D)
    scales = np.ascontiguousarray(b[..., ps * D:ps * D + 4 * ps]).view(np.float32).reshape(P, H, ps)
    return codes, scales, b[..., ps * D + 4 * ps:]


# ---------------------------------------------------------------------------
# store_kv: quantize on write
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D,ps,hkv", [(128, 16, 8), (64, 3, 2), (128, 1, 1), (64, 64, 4)])
def test_store_kv_int8_bit_exact(D, ps, hkv):
    print(f"store_kv int8 D={D} ps={ps} hkv={hkv}", flush=True)
    rng = np.random.default_rng(17)
    num_pages, T = 29, 60
    slots = rng.permutation(num_pages * ps)[:T].astype(np.int64)
    slots[3] = -1                              # padding token: skipped
    slots[7] = num_pages * ps                  # out of range: skipped
    kv = synth.normal_values(rng, (2, T, hkv, D), synth.BF16)
    kv[0, 5, 0] = 0                            # a zero vector: scale 0, codes 0
    kv[1, 9, hkv - 1] = synth.f32_to_bf16_bits(
        rng.standard_normal(D).astype(np.float32) * np.float32(3e4))   # large magnitudes
    kv[1, 11, 0] = synth.f32_to_bf16_bits(
        rng.standard_normal(D).astype(np.float32) * np.float32(1e-20))  # tiny magnitudes
    desc = pkv.PoolDesc(pkv.PKV_I8, num_pages, ps, hkv, D)
    kp, vp = desc.new_pools(DEV, fill=0xA5)
    pkv.store_kv(desc, kp, vp, dev_tensor(kv[0], synth.BF16), dev_tensor(kv[1], synth.BF16), i64(slots))
    torch.cuda.synchronize()
    for pool, vals in ((kp, kv[0]), (vp, kv[1])):
        codes, scales, pad = unpack(pool, desc)
        e_codes = np.full(codes.shape, np.uint8(0xA5).view(np.int8), np.int8)
        e_scales = np.full(scales.shape, np.uint32(0xA5A5A5A5).view(np.float32), np.float32)
        store_rows_int8(e_codes, e_scales, slots, synth.to_f64(vals, synth.BF16))
        assert np.array_equal(codes, e_codes)
        assert np.array_equal(scales.view(np.uint32), e_scales.view(np.uint32))
        assert (pad == 0xA5).all()               # padding never written


# ---------------------------------------------------------------------------
# decode (and the short-append path it shares)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D,ps,hq,hkv,n,len_hi", [
    (128, 16, 32, 8, 24, 1500),
    (128, 16, 32, 8, 3, 9000),
    (64, 4, 16, 1, 9, 900),
    (128, 3, 8, 8, 9, 500),
    (128, 256, 16, 1, 9, 2000),
    (128, 64, 64, 8, 9, 5000),
    (64, 1, 4, 4, 9, 300),
])
def test_decode_int8(D, ps, hq, hkv, n, len_hi):
    print(f"decode int8 D={D} ps={ps} hq={hq} hkv={hkv} n={n}", flush=True)
    w = synth.decode_batch(n_seqs=n, len_lo=1, len_hi=len_hi, page_size=ps,
                           num_pages=n * (-(-len_hi // ps)) + 5, num_q_heads=hq,
                           num_kv_heads=hkv, head_dim=D, dtype=synth.BF16, seed=D + ps + n)
    s, seqs, out = run_decode(w, kv_int8=True)
    expect = ref.decode_reference(w, s.scale, kv_int8=True)
    o = host_f64(out)
    e = np.stack([np.stack([expect[(b, h)] for h in range(hq)]) for b in range(n)])
    check_close(o, e, "decode int8")


def test_decode_int8_page_permutation_bit_exact():
    w = synth.decode_batch(n_seqs=16, len_lo=1, len_hi=1200, num_pages=2000, seed=3)
    outs = []
    for k in range(3):
        order = np.random.default_rng(200 + k).permutation(w.num_pages).astype(np.int32)
        _, _, out = run_decode(w, free_order=order, kv_int8=True)
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_decode_int8_is_close_to_bf16():
    """The INT8 cache changes the result by about the quantization step only."""
    w = synth.decode_batch(n_seqs=8, len_lo=100, len_hi=2000, num_pages=1200, seed=4)
    _, _, o8 = run_decode(w, kv_int8=True)
    _, _, o16 = run_decode(w)
    d = (o8.float() - o16.float()).abs()
    assert d.max().item() < 0.05 and d.mean().item() < 0.01
    assert d.max().item() > 0                  # and the codes really were 8-bit


# ---------------------------------------------------------------------------
# prefill / append
# ---------------------------------------------------------------------------
class _Pools:
    def __init__(self, D, ps, hkv, num_pages, seed):
        self.dtype, self.head_dim, self.page_size = synth.BF16, D, ps
        self.num_kv_heads, self.num_pages = hkv, num_pages
        self.free_order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)


@pytest.mark.parametrize("D,ps,hq,hkv,ctx,news", [
    (128, 16, 32, 8, [300, 0, 1000], [200, 64, 150]),
    (64, 3, 8, 8, [100, 37], [49, 130]),
    (128, 64, 16, 2, [500, 20, 90, 0], [80, 300, 13, 64]),
    (128, 1, 1, 1, [3000], [60]),
    (64, 16, 6, 3, [2500, 700], [100, 20]),
    (128, 4, 32, 8, [200, 50], [100, 300]),
])
def test_prefill_int8_variants(D, ps, hq, hkv, ctx, news):
    """Append of several queries per sequence over cached INT8 positions: page
    sizes below, at and above the rows a wave stages per pass, one or several
    KV splits, contexts within and above 2048 positions (both prefill
    kernels)."""
    print(f"prefill int8 D={D} ps={ps} hq={hq} hkv={hkv} ctx={ctx} new={news}", flush=True)
    rng = np.random.default_rng(D * 11 + ps)
    lens = [c + n for c, n in zip(ctx, news)]
    pages = sum(-(-L // ps) for L in lens) + 3
    s = Session.open(_Pools(D, ps, hkv, pages, seed=ps + hq), kv_int8=True)
    seqs = [s.alloc.seq_new() for _ in lens]
    kv = [synth.normal_values(rng, (2, L, hkv, D), synth.BF16) for L in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
        s.store(seq, 0, kv[b][0], kv[b][1], synth.BF16)
    qs = [synth.normal_values(rng, (n, hq, D), synth.BF16) for n in news]
    out = host_f64(s.append(seqs, news, dev_tensor(np.concatenate(qs), synth.BF16)))
    row = 0
    for b in range(len(lens)):
        if news[b]:
            e = quantize_then_attend(synth.to_f64(qs[b], synth.BF16), synth.to_f64(kv[b][0], synth.BF16),
                                     synth.to_f64(kv[b][1], synth.BF16), s.scale)
            check_close(out[row:row + news[b]], e, f"prefill int8 seq {b}")
        row += news[b]



# Error budget of the append kernel, per output element (row r, dim d), against
# the exact result O over the dequantized values:
#  * the probabilities enter O^T rounded to bf16 (p times the value's scale for
#    INT8 pages) and the row sum rounded to bf16: at most 2^-8 relative each
#    (bf16 keeps 8 significant bits), so at most 2^-7 max_j |v_jd| over the
#    positions j the row attends to;
#  * fp32 scores, exponentials and sums: well under 2^-10 max_j |v_jd| at
#    these lengths (head_dim 128, a few thousand positions);
#  * the output's own rounding to bf16: 2^-8 |O_rd|.
# INT8 codes are exact bf16 integers and the scales are applied in fp32, so
# the quantization adds no term beyond the dequantized values themselves.
BUDGET_V, BUDGET_O = 2.0 ** -7 + 2.0 ** -10, 2.0 ** -8


@pytest.mark.parametrize("kv_int8", [False, True])
@pytest.mark.parametrize("ctx,news", [
    ([2600, 0, 900], [120, 200, 64]),       # a context above 2048: the tiled kernel
    ([1500, 0, 300], [200, 250, 40]),       # every context within 2048: the stream kernel
])
def test_prefill_error_budget(kv_int8, ctx, news):
    """Every output element is within the error budget above, for bf16 and
    INT8 pages."""
    print(f"prefill error budget int8={kv_int8} ctx={ctx} new={news}", flush=True)
    D, ps, hq, hkv = 128, 16, 32, 8
    rng = np.random.default_rng(77 + len(ctx) + int(kv_int8))
    lens = [c + n for c, n in zip(ctx, news)]
    pages = sum(-(-L // ps) for L in lens) + 3
    s = Session.open(_Pools(D, ps, hkv, pages, seed=5), kv_int8=kv_int8)
    seqs = [s.alloc.seq_new() for _ in lens]
    kv = [synth.normal_values(rng, (2, L, hkv, D), synth.BF16) for L in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
        s.store(seq, 0, kv[b][0], kv[b][1], synth.BF16)
    qs = [synth.normal_values(rng, (n, hq, D), synth.BF16) for n in news]
    out = host_f64(s.append(seqs, news, dev_tensor(np.concatenate(qs), synth.BF16)))
    row, worst = 0, 0.0
    for b in range(len(lens)):
        n = news[b]
        if n:
            k64, v64 = synth.to_f64(kv[b][0], synth.BF16), synth.to_f64(kv[b][1], synth.BF16)
            if kv_int8:
                k64, v64 = dequantize(*quantize(k64)), dequantize(*quantize(v64))
            e = attend(synth.to_f64(qs[b], synth.BF16), k64, v64, s.scale)         # [n][hq][D]
            vmax = np.maximum.accumulate(np.abs(v64), axis=0)[lens[b] - n:]        # [n][hkv][D]
            vmax = np.repeat(vmax, hq // hkv, axis=1)                              # per query head
            bound = BUDGET_V * vmax + BUDGET_O * np.abs(e)
            err = np.abs(out[row:row + n] - e)
            assert np.isfinite(out[row:row + n]).all()
            assert (err <= bound).all(), f"seq {b}: worst err/bound {(err / bound).max():.3f}"
            worst = max(worst, float((err / bound).max()))
        row += n
    print(f"worst error / budget {worst:.3f}", flush=True)

def test_prefix_shared_prefill_int8_reduced():
    w = synth.prefix_traces(n_rows=20, n_traces=5, first_rows=(100, 140, 190), len_lo=100,
                            len_hi=600, trace_len=600, num_pages=1200)
    s, (order, parent, shared), seqs, n_new, out = run_prefix(w, kv_int8=True)
    check_close(host_f64(out), ref.prefix_reference_full(w, shared.tolist(), s.scale, kv_int8=True),
                "prefix int8")


def test_rewind_int8_reduced():
    w = synth.rewind_docs(n_docs=24, num_pages=24 * 22 + 10)
    s, seqs, outs = run_rewind(w, kv_int8=True)
    expect = ref.rewind_reference(w, s.scale, kv_int8=True)
    for p in range(2):
        o = host_f64(outs[p]).reshape(24, w.q_len, w.num_q_heads, w.head_dim)
        check_close(o, np.stack([expect[p][d] for d in range(24)]), f"rewind int8 pass {p + 1}")


def test_spec_rollback_int8_reduced():
    w = synth.spec_decode(n_seqs=3, len_lo=2000, len_hi=6000, steps=4)
    s, seqs, outs = run_spec(w, kv_int8=True)
    expect = ref.spec_reference(w, s.scale, 4, kv_int8=True)
    for st in range(4):
        o = host_f64(outs[st]).reshape(3, w.drafts, w.num_q_heads, w.head_dim)
        check_close(o, np.stack([expect[st][b] for b in range(3)]), f"spec int8 step {st}")


# ---------------------------------------------------------------------------
# full-size decode batch (64 sequences, 300k-page pool): stored codes; every
# output row is compared in test_gpu_full.py
# ---------------------------------------------------------------------------
def test_decode_workload2_int8_stored_codes():
    print("workload 2 int8 stored codes", flush=True)
    w = synth.decode_batch()
    s, seqs, out = run_decode(w, kv_int8=True)
    torch.cuda.synchronize()
    # the stored codes of one sequence's first page match the oracle's
    codes, scales, _ = unpack(s.k_pool, s.desc)
    page = int(s.alloc.block_table(seqs[0])[0])
    e_codes, e_scales = quantize(synth.to_f64(w.k[0:16], w.dtype))      # [16][Hkv][D]
    assert np.array_equal(codes[page].transpose(1, 0, 2), e_codes)
    assert np.array_equal(scales[page].T.view(np.uint32), e_scales.view(np.uint32))
