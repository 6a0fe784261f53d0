"""Seeded random shapes through the HIP path, against the oracle.

Each case draws, from a fixed seed: bf16 or INT8 pages, head_dim 64 or 128,
a page size from 1 to 256 (powers of two and not), 1 to 8 KV heads with GQA
groups 1 to 8, 1 to 6 sequences with cached contexts of up to 1,800 or up to
4,500 positions and up to 6 or up to 300 new queries each (at least one query
in the call), and a shuffled pool.  The same sequences then decode one more
token.  Outputs are compared element by element with the oracle's attention
("KV Cache Management and PagedAttention", "Compute attention over scattered
KV") within the bf16 bars, so combinations no hand-written case names
(page-lookup modes, KV splits, the persistent and tiled prefill kernels, the
decode kernel's row blocks) are covered too.
"""

import numpy as np
import pytest
import torch

import synth
from conftest import ensure_library
from gpu_path import Session, dev_tensor, host_f64
from oracle.attention import attend
from oracle.quant import dequantize, quantize

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 1e-2
PAGE_SIZES = [1, 2, 3, 5, 8, 16, 32, 64, 128, 256]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


class _Pools:
    def __init__(self, D, ps, hkv, num_pages, seed):
        self.dtype, self.head_dim, self.page_size = synth.BF16, D, ps
        self.num_kv_heads, self.num_pages = hkv, num_pages
        self.free_order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)


def _draw(seed):
    r = np.random.default_rng(1000 + seed)
    kv_int8 = bool(r.integers(0, 2))
    D = int(r.choice([64, 128]))
    ps = int(r.choice(PAGE_SIZES))
    hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    n = int(r.integers(1, 7))
    ctx_hi = int(r.choice([1800, 4500]))          # the persistent or the tiled prefill kernel
    new_hi = int(r.choice([6, 300]))              # a few rows per unit take the decode kernels
    ctx = [int(x) for x in r.integers(0, ctx_hi + 1, size=n)]
    news = [int(x) for x in r.integers(0, new_hi + 1, size=n)]
    if sum(news) == 0:
        news[0] = 1
    return kv_int8, D, ps, hkv, hkv * G, ctx, news


def _check(out, expect, what):
    assert out.shape == expect.shape, what
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - expect)
    assert err.max() <= BF16_MAX, f"{what}: max abs err {err.max():.3g}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3g}"


@pytest.mark.parametrize("seed", range(20))
def test_random_shapes_append_then_decode(seed):
    kv_int8, D, ps, hkv, hq, ctx, news = _draw(seed)
    print(f"random shape {seed}: int8={kv_int8} D={D} ps={ps} hkv={hkv} hq={hq} ctx={ctx} new={news}",
          flush=True)
    rng = np.random.default_rng(seed)
    lens = [c + n for c, n in zip(ctx, news)]
    pages = sum(-(-(L + 1) // ps) for L in lens) * 2 + 4
    s = Session.open(_Pools(D, ps, hkv, pages, seed=seed), kv_int8=kv_int8)
    seqs = [s.alloc.seq_new() for _ in lens]
    kv = [synth.normal_values(rng, (2, L + 1, hkv, D), synth.BF16) for L in lens]   # one more for decode
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
    s.store_many([(seq, 0, kv[b][0][:lens[b]], kv[b][1][:lens[b]]) for b, seq in enumerate(seqs)], synth.BF16)
    qs = [synth.normal_values(rng, (n, hq, D), synth.BF16) for n in news]
    out = host_f64(s.append(seqs, news, dev_tensor(np.concatenate(qs), synth.BF16)))

    def values(b, L):
        k = synth.to_f64(kv[b][0][:L], synth.BF16)
        v = synth.to_f64(kv[b][1][:L], synth.BF16)
        if kv_int8:
            k, v = dequantize(*quantize(k)), dequantize(*quantize(v))
        return k, v

    row = 0
    for b, L in enumerate(lens):
        if news[b]:
            k, v = values(b, L)
            _check(out[row:row + news[b]], attend(synth.to_f64(qs[b], synth.BF16), k, v, s.scale),
                   f"append seq {b}")
        row += news[b]
    # one decode step on the same sequences
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, 1)
    s.store_many([(seq, lens[b], kv[b][0][lens[b]:], kv[b][1][lens[b]:]) for b, seq in enumerate(seqs)],
                 synth.BF16)
    qd = synth.normal_values(rng, (len(lens), hq, D), synth.BF16)
    dec = host_f64(s.decode(seqs, dev_tensor(qd, synth.BF16)))
    for b, L in enumerate(lens):
        k, v = values(b, L + 1)
        _check(dec[b:b + 1], attend(synth.to_f64(qd[b:b + 1], synth.BF16), k, v, s.scale), f"decode seq {b}")
