"""Score patterns that drive the online softmax's reference maximum.

The attention a query computes is softmax attention over the positions of
its own sequence ("KV Cache Management and PagedAttention", "Compute
attention over scattered KV").  The kernels evaluate it block by block with
a running reference maximum per query row that is raised only when a score
exceeds it by more than 8 (log2 units); the rescale of the running sum and
output sits in a branch that most blocks skip.  N(0,1) inputs take that
branch almost only on a row's first block.  Here every key carries a large
component along its KV head's query direction, sized by a pattern over
positions, so that the scores

* rise steadily (the reference moves on nearly every 16-position block),
* fall (it never moves after the first block),
* jump at isolated positions (it moves on the spikes' blocks only),
* climb in steps that straddle block and tile boundaries, or
* are dominated by one position (every other weight underflows to zero),

and the outputs must match the fp64 oracle to the bf16 tolerance on bf16
and on INT8 pages, in the decode kernel (one query, and short appends of
several queries per sequence), the persistent prefill kernel (contexts up to
2048 positions) and the tiled prefill kernel with KV splits (a longer
context).
"""

import numpy as np
import pytest
import torch

import pagedattention_pkv_store_amd as pkv
import synth
from conftest import ensure_library
from gpu_path import Session, dev_tensor, host_f64
from oracle.attention import attend
from oracle.quant import dequantize, quantize

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def _beta(pattern: str, length: int, rng) -> np.ndarray:
    """Score offset (natural units) of each position of a sequence."""
    p = np.arange(length, dtype=np.float64)
    if pattern == "rising":
        return 0.45 * p                                   # +10.4 log2 units per 16 positions
    if pattern == "falling":
        return 0.45 * (length - 1 - p)
    if pattern == "spikes":
        b = np.zeros(length)
        if length > 1:
            at = np.sort(rng.choice(length, size=min(6, length), replace=False))
            b[at] = 12.0 * np.arange(1, at.size + 1)      # each spike 12 above the last
        return b
    if pattern == "steps":
        return 9.0 * np.floor(p / 37.0)                   # 13 log2 units every 37 positions
    if pattern == "dominant":
        b = np.zeros(length)
        b[length // 2] = 90.0                             # every other weight is below e^-90
        return b
    raise ValueError(pattern)


class _Pools:
    def __init__(self, D, ps, hkv, num_pages, seed):
        self.dtype, self.head_dim, self.page_size = synth.BF16, D, ps
        self.num_kv_heads, self.num_pages = hkv, num_pages
        self.free_order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)


def _bf16(x: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32))


def _workload(pattern, lens, n_new, hq, hkv, D, seed):
    """Per sequence: K/V [L][Hkv][D] and the new queries [n][Hq][D] (bf16 bits).
    Query head h of KV head g is sqrt(D) * u_g plus N(0, 0.3^2) noise, and
    key p is beta_p * u_g plus N(0, 0.5^2) noise, so a score is beta_p plus
    noise of a few tenths."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((hkv, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    group = hq // hkv
    ks, vs, qs = [], [], []
    for L, n in zip(lens, n_new):
        beta = _beta(pattern, L, rng)
        k = beta[:, None, None] * u[None, :, :] + 0.5 * rng.standard_normal((L, hkv, D))
        v = rng.standard_normal((L, hkv, D))
        q = np.sqrt(D) * np.repeat(u, group, axis=0)[None, :, :] + 0.3 * rng.standard_normal((n, hq, D))
        ks.append(_bf16(k))
        vs.append(_bf16(v))
        qs.append(_bf16(q))
    return ks, vs, qs


def _check(out, expect, what):
    assert out.shape == expect.shape, what
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - expect)
    assert err.max() <= BF16_MAX, f"{what}: max abs err {err.max():.3g}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3g}"


def _expected(q, k, v, kv_int8, scale):
    k64, v64 = synth.to_f64(k, synth.BF16), synth.to_f64(v, synth.BF16)
    if kv_int8:
        k64, v64 = dequantize(*quantize(k64)), dequantize(*quantize(v64))
    return attend(synth.to_f64(q, synth.BF16), k64, v64, scale)


def _session(lens, ps, hkv, D, kv_int8, seed, ks, vs):
    pages = sum(-(-L // ps) for L in lens) + 7
    s = Session.open(_Pools(D, ps, hkv, pages, seed), kv_int8=kv_int8)
    seqs = [s.alloc.seq_new() for _ in lens]
    for b, seq in enumerate(seqs):
        s.alloc.reserve(seq, lens[b])
    s.store_many([(seq, 0, ks[b], vs[b]) for b, seq in enumerate(seqs)], synth.BF16)
    return s, seqs


PATTERNS = ["rising", "falling", "spikes", "steps", "dominant"]


@pytest.mark.parametrize("kv_int8", [False, True])
@pytest.mark.parametrize("ps", [16, 3])
@pytest.mark.parametrize("pattern", PATTERNS)
def test_decode_score_patterns(pattern, ps, kv_int8):
    """One query per sequence at its last position, lengths around block and
    page boundaries up to 2,500 positions (several waves per unit)."""
    print(f"decode pattern={pattern} ps={ps} int8={kv_int8}", flush=True)
    hq, hkv, D = 16, 4, 128
    lens = [1, 2, 15, 16, 17, 33, 700, 2500]
    seed = PATTERNS.index(pattern) * 10 + ps
    ks, vs, qs = _workload(pattern, lens, [1] * len(lens), hq, hkv, D, seed)
    s, seqs = _session(lens, ps, hkv, D, kv_int8, seed, ks, vs)
    out = host_f64(s.decode(seqs, dev_tensor(np.concatenate(qs), synth.BF16)))
    for b in range(len(lens)):
        e = _expected(qs[b], ks[b], vs[b], kv_int8, s.scale)
        _check(out[b:b + 1], e, f"{pattern} ps={ps} int8={kv_int8} seq {b} (L={lens[b]})")


@pytest.mark.parametrize("kv_int8", [False, True])
@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("lens,n_new", [
    ([9, 40, 300], [3, 5, 5]),            # short appends: the decode kernel, several 16-row blocks
    ([60, 350, 1200], [50, 50, 120]),     # contexts within 2,048: the persistent prefill kernel
    ([120, 3100], [70, 160]),             # a longer context: the tiled prefill kernel, KV splits
])
def test_append_score_patterns(pattern, kv_int8, lens, n_new):
    """Causal appends: query i of sequence b sits at position L_b - n_b + i
    and sees positions 0 .. L_b - n_b + i, so each query meets the pattern up
    to its own position."""
    print(f"append pattern={pattern} int8={kv_int8} lens={lens} new={n_new}", flush=True)
    hq, hkv, D, ps = 16, 4, 128, 16
    seed = PATTERNS.index(pattern) * 10 + 7 + sum(lens) % 5
    ks, vs, qs = _workload(pattern, lens, n_new, hq, hkv, D, seed)
    s, seqs = _session(lens, ps, hkv, D, kv_int8, seed, ks, vs)
    out = host_f64(s.append(seqs, n_new, dev_tensor(np.concatenate(qs), synth.BF16)))
    off = 0
    for b in range(len(lens)):
        e = _expected(qs[b], ks[b], vs[b], kv_int8, s.scale)
        _check(out[off:off + n_new[b]], e, f"{pattern} int8={kv_int8} seq {b} (L={lens[b]}, n={n_new[b]})")
        off += n_new[b]
