"""Closed forms of the attention definition, checked on the HIP path.

"KV Cache Management and PagedAttention", "Compute attention over scattered
KV": a query attends to the stored positions of its own sequence up to and
including its own.  Two cases have an answer that needs no oracle:

* A query that sees exactly one position (the first query of a causal prefill
  over an empty context, or the query of a one-position sequence) returns that
  position's value.  Its one weight is exp(0) = 1 and the normaliser is the
  same 1, so the output equals the stored value bit for bit (bf16 and fp32
  pools; through the KV-split merge too).
* A zero query weighs its visible positions equally, so the output is their
  mean.  Every weight is exactly 1, so the only errors are the fp32 sum of the
  values (at most n * 2^-24 * max|v| for n positions) and the output's own
  rounding (2^-8 relative for bf16; two fp32 roundings for fp32): the test
  allows exactly that.

Both run in the decode kernel, the persistent short-context prefill kernel,
the tiled prefill kernel (a context above 2048 positions, with KV splits) and
the fp32 tile kernel.
"""

import numpy as np
import pytest
import torch

import synth
from conftest import ensure_library
from gpu_path import Session, dev_tensor, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


class _Pools:
    def __init__(self, dtype, D, ps, hkv, num_pages, seed):
        self.dtype, self.head_dim, self.page_size = dtype, D, ps
        self.num_kv_heads, self.num_pages = hkv, num_pages
        self.free_order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)


def _fresh(dtype, D, ps, hq, hkv, lens, seed):
    """Sequences of the given lengths, every position stored (values N(0,1))."""
    rng = np.random.default_rng(seed)
    pages = sum(-(-L // ps) for L in lens) + 5
    s = Session.open(_Pools(dtype, D, ps, hkv, pages, seed=seed))
    seqs = [s.alloc.seq_new() for _ in lens]
    kv = [synth.normal_values(rng, (2, L, hkv, D), dtype) for L in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
    s.store_many([(seq, 0, kv[b][0], kv[b][1]) for b, seq in enumerate(seqs)], dtype)
    for b, seq in enumerate(seqs):
        assert s.alloc.seq_len(seq) == lens[b]
    return s, seqs, kv, rng


def _bits(a: torch.Tensor) -> np.ndarray:
    t = a.detach().cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _value_bits(v: np.ndarray, dtype) -> np.ndarray:
    """synth values -> the same bit patterns the pools hold."""
    return v.view(np.int16) if dtype == synth.BF16 else np.ascontiguousarray(v, np.float32).view(np.int32)


# (dtype, D, ps, hq, hkv, fresh sequence lengths): every sequence is appended
# from position 0, so query 0 of each sees only position 0
PREFILL_CASES = [
    (synth.BF16, 128, 16, 32, 8, [1, 50, 300, 1200]),       # persistent short-context kernel
    (synth.BF16, 128, 16, 32, 8, [2300, 40, 1]),            # tiled kernel, KV splits
    (synth.BF16, 64, 3, 8, 2, [2100, 7]),                   # page size 3, D 64
    (synth.F32, 64, 4, 4, 2, [90, 1, 33]),                  # fp32 tile kernel
]


@pytest.mark.parametrize("dtype,D,ps,hq,hkv,lens", PREFILL_CASES)
def test_first_causal_query_returns_its_value_exactly(dtype, D, ps, hq, hkv, lens):
    print(f"closed form: first causal row {dtype} D={D} ps={ps} lens={lens}", flush=True)
    s, seqs, kv, rng = _fresh(dtype, D, ps, hq, hkv, lens, seed=D + ps)
    qs = [synth.normal_values(rng, (L, hq, D), dtype) for L in lens]
    out = s.append(seqs, lens, dev_tensor(np.concatenate(qs), dtype))
    torch.cuda.synchronize()
    got = _bits(out)
    row, G = 0, hq // hkv
    for b, L in enumerate(lens):
        want = _value_bits(kv[b][1][0], dtype)              # [hkv][D]: V at position 0
        for h in range(hq):
            assert np.array_equal(got[row, h], want[h // G]), f"seq {b} head {h}"
        row += L


@pytest.mark.parametrize("dtype,D,ps,hq,hkv,lens", PREFILL_CASES)
def test_zero_query_prefill_returns_the_mean(dtype, D, ps, hq, hkv, lens):
    print(f"closed form: zero-query prefill {dtype} D={D} ps={ps} lens={lens}", flush=True)
    s, seqs, kv, rng = _fresh(dtype, D, ps, hq, hkv, lens, seed=D + ps + 1)
    q = np.zeros((sum(lens), hq, D), np.float32)
    if dtype == synth.BF16:
        q = synth.f32_to_bf16_bits(q)
    out = host_f64(s.append(seqs, lens, dev_tensor(q, dtype)))
    row, G = 0, hq // hkv
    out_rel = 2.0 ** -8 if dtype == synth.BF16 else 2.0 ** -22
    for b, L in enumerate(lens):
        v = synth.to_f64(kv[b][1], dtype)                    # [L][hkv][D]
        n = np.arange(1, L + 1, dtype=np.float64)[:, None, None]
        mean = np.cumsum(v, axis=0) / n                       # row i: mean of positions 0..i
        vmax = np.maximum.accumulate(np.abs(v), axis=0)
        tol = out_rel * np.abs(mean) + (n + 2) * 2.0 ** -24 * vmax
        for h in range(hq):
            err = np.abs(out[row:row + L, h] - mean[:, h // G])
            assert (err <= tol[:, h // G]).all(), f"seq {b} head {h}: worst {(err / tol[:, h // G]).max():.3f}"
        row += L


@pytest.mark.parametrize("dtype,D,ps", [(synth.BF16, 128, 16), (synth.F32, 64, 4)])
def test_decode_closed_forms(dtype, D, ps):
    """One-position sequences return their value exactly and a zero query
    returns the mean, in a batch whose long sequences are split across waves."""
    print(f"closed form: decode {dtype} D={D} ps={ps}", flush=True)
    hq, hkv = 32, 8
    lens = [1, 3000, 1, 700, 4096, 1, 2] * 3
    s, seqs, kv, rng = _fresh(dtype, D, ps, hq, hkv, lens, seed=D + 2)
    G = hq // hkv
    q = synth.normal_values(rng, (len(lens), hq, D), dtype)
    got = _bits(s.decode(seqs, dev_tensor(q, dtype)))
    for b, L in enumerate(lens):
        if L == 1:
            want = _value_bits(kv[b][1][0], dtype)
            for h in range(hq):
                assert np.array_equal(got[b, h], want[h // G]), f"seq {b} head {h}"
    zq = np.zeros((len(lens), hq, D), np.float32)
    if dtype == synth.BF16:
        zq = synth.f32_to_bf16_bits(zq)
    out = host_f64(s.decode(seqs, dev_tensor(zq, dtype)))
    out_rel = 2.0 ** -8 if dtype == synth.BF16 else 2.0 ** -22
    for b, L in enumerate(lens):
        v = synth.to_f64(kv[b][1], dtype)
        mean = v.mean(axis=0)                                 # [hkv][D]
        tol = out_rel * np.abs(mean) + (L + 2) * 2.0 ** -24 * np.abs(v).max(axis=0)
        for h in range(hq):
            err = np.abs(out[b, h] - mean[h // G])
            assert (err <= tol[h // G]).all(), f"seq {b} head {h}: worst {(err / tol[h // G]).max():.3f}"
