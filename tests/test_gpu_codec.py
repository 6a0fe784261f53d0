"""GPU parity of the group-wise low-bit KV codec (ReKV, section 2.2) against
the oracle: payload bytes and restored pool bytes are bit-exact (codes are the
correctly rounded fp32 quotient x / scale rounded to nearest, ties to even, on
both sides), and attention over restored pages is within
the bf16 bars of the oracle over the dequantized values.  Destination pools
start NaN-filled, so a slot the restore should not touch stays NaN."""

import numpy as np
import pytest
import torch

import pagedattention_pkv_store_amd as pkv
import synth
from conftest import ensure_library
from gpu_path import DEV, Session, dev_tensor, host_f64, i32
from oracle.attention import attend
from oracle.codec import decode as oracle_decode
from oracle.codec import encode as oracle_encode

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


class _Pools:
    def __init__(self, D, ps, hkv, num_pages, seed):
        self.dtype, self.head_dim, self.page_size = synth.BF16, D, ps
        self.num_kv_heads, self.num_pages = hkv, num_pages
        self.free_order = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)


def _stored_sequence(L, D, ps, hkv, seed):
    rng = np.random.default_rng(seed)
    s = Session.open(_Pools(D, ps, hkv, -(-L // ps) * 2 + 5, seed))
    seq = s.alloc.seq_new()
    s.alloc.reserve(seq, L)
    k, v = synth.normal_values(rng, (2, L, hkv, D), synth.BF16)
    k[0, 0, :64] = 0                                 # a zero group
    s.store(seq, 0, k, v, synth.BF16)
    return s, seq, k, v


def _bf16_bits(x64):
    return synth.f32_to_bf16_bits(np.asarray(x64, dtype=np.float32))


@pytest.mark.parametrize("bits,L,D,ps,hkv", [(8, 53, 128, 16, 8), (4, 53, 128, 16, 8), (8, 100, 64, 3, 2),
                                             (4, 37, 64, 1, 1), (8, 4096, 128, 64, 8)])
def test_encode_bit_exact(bits, L, D, ps, hkv):
    print(f"codec encode bits={bits} L={L} D={D} ps={ps} hkv={hkv}", flush=True)
    s, seq, k, v = _stored_sequence(L, D, ps, hkv, seed=L + bits)
    n = pkv.codec_payload_bytes(L, hkv, D, bits)
    payload = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)
    pkv.codec_encode(s.desc, s.k_pool, s.v_pool, i32(s.alloc.block_table(seq)), L, bits, payload)
    torch.cuda.synchronize()
    expect = oracle_encode(synth.to_f64(k, synth.BF16), synth.to_f64(v, synth.BF16), bits)
    assert np.array_equal(payload.cpu().numpy(), expect)


@pytest.mark.parametrize("bits,L,D,ps,hkv", [(8, 53, 128, 16, 8), (4, 100, 64, 3, 2), (8, 37, 64, 1, 1)])
def test_restore_bit_exact_and_attention(bits, L, D, ps, hkv):
    """Encode on the device, restore into other pages of a second pool, and
    attend over the restored sequence."""
    print(f"codec restore bits={bits} L={L} D={D} ps={ps} hkv={hkv}", flush=True)
    s, seq, k, v = _stored_sequence(L, D, ps, hkv, seed=7 * L + bits)
    n = pkv.codec_payload_bytes(L, hkv, D, bits)
    payload = torch.empty((n,), dtype=torch.uint8, device=DEV)
    pkv.codec_encode(s.desc, s.k_pool, s.v_pool, i32(s.alloc.block_table(seq)), L, bits, payload)
    r = Session.open(_Pools(D, ps, hkv, -(-L // ps) * 3 + 7, seed=L + 99))
    rseq = r.alloc.seq_new()
    r.alloc.reserve(rseq, L)
    pkv.codec_decode(r.desc, r.k_pool, r.v_pool, i32(r.alloc.block_table(rseq)), L, bits, payload)
    torch.cuda.synchronize()
    dk, dv = oracle_decode(payload.cpu().numpy(), (L, hkv, D), bits)
    # restored pool rows are bf16(scale * code), bit for bit; the rest is untouched NaN
    kp = r.k_pool.view(torch.int16).cpu().numpy().view(np.uint16)
    vp = r.v_pool.view(torch.int16).cpu().numpy().view(np.uint16)
    slots = r.alloc.slots(rseq, 0, L)
    got_k = np.stack([kp[sl // ps, :, sl % ps] for sl in slots])
    got_v = np.stack([vp[sl // ps, :, sl % ps] for sl in slots])
    assert np.array_equal(got_k, _bf16_bits(dk)) and np.array_equal(got_v, _bf16_bits(dv))
    assert np.isnan(host_f64(r.k_pool)).sum() == (r.desc.num_pages * ps - L) * hkv * D
    # attention over the restored sequence
    rng = np.random.default_rng(L)
    hq = hkv * 4
    q = synth.normal_values(rng, (1, hq, D), synth.BF16)
    out = host_f64(r.decode([rseq], dev_tensor(q, synth.BF16)))
    e = attend(synth.to_f64(q, synth.BF16), synth.bf16_bits_to_f32(_bf16_bits(dk)).astype(np.float64),
               synth.bf16_bits_to_f32(_bf16_bits(dv)).astype(np.float64), r.scale)
    err = np.abs(out - e)
    assert np.isfinite(out).all() and err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


@pytest.mark.parametrize("bits", [4, 8])
def test_encode_exact_ties_bit_exact(bits):
    """Groups whose elements are exact half-integer multiples of their scale:
    max 1.53125 gives the Q4 scale 7/32 exactly, and (2k + 1) * 7/64 is
    (k + 1/2) * scale, so the division lands on exact ties that go to even.
    Powers of two move the groups across binades without losing exactness.
    A per-group reciprocal would round some of these the other way; the
    kernel must match the division."""
    L, D, ps, hkv = 40, 128, 16, 8
    print(f"codec encode exact ties bits={bits}", flush=True)
    rng = np.random.default_rng(500 + bits)
    s, seq, k, v = _stored_sequence(L, D, ps, hkv, seed=11 + bits)
    ties = np.array([(2 * j + 1) * 7 / 64 for j in range(7)])
    for t in (k, v):
        for p in range(L):
            for h in range(hkv):
                g = np.concatenate([[1.53125], rng.choice(ties, 63) * rng.choice([-1.0, 1.0], 63)])
                t[p, h, :64] = synth.f32_to_bf16_bits((g * 2.0 ** rng.integers(-6, 7)).astype(np.float32))
    s.store(seq, 0, k, v, synth.BF16)
    n = pkv.codec_payload_bytes(L, hkv, D, bits)
    payload = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)
    pkv.codec_encode(s.desc, s.k_pool, s.v_pool, i32(s.alloc.block_table(seq)), L, bits, payload)
    torch.cuda.synchronize()
    kf, vf = synth.to_f64(k, synth.BF16), synth.to_f64(v, synth.BF16)
    expect = oracle_encode(kf, vf, bits)
    assert np.array_equal(payload.cpu().numpy(), expect)
    if bits == 4:    # the input does separate the two readings
        x = kf[:, :, :64].astype(np.float32)
        sc = (np.abs(x).max(-1, keepdims=True) / np.float32(7)).astype(np.float16).astype(np.float32)
        by_recip = np.clip(np.rint((x * (np.float32(1) / sc)).astype(np.float32)), -7, 7)
        by_div = np.clip(np.rint((x / sc).astype(np.float32)), -7, 7)
        assert (by_recip != by_div).sum() > 100


def test_table_entries_off_the_pool():
    """A block-table entry that is not a page of the pool (-1, num_pages)
    encodes its positions as zeros and is skipped by the restore: no other
    page is read in its place or written."""
    L, D, ps, hkv, bits = 48, 128, 16, 8, 8
    print("codec table entries off the pool", flush=True)
    s, seq, k, v = _stored_sequence(L, D, ps, hkv, seed=21)
    bt = s.alloc.block_table(seq).copy()
    bt[1] = -1                                       # positions 16..31
    payload = torch.empty((pkv.codec_payload_bytes(L, hkv, D, bits),), dtype=torch.uint8, device=DEV)
    pkv.codec_encode(s.desc, s.k_pool, s.v_pool, i32(bt), L, bits, payload)
    torch.cuda.synchronize()
    kf, vf = synth.to_f64(k, synth.BF16), synth.to_f64(v, synth.BF16)
    kf[16:32] = 0
    vf[16:32] = 0
    assert np.array_equal(payload.cpu().numpy(), oracle_encode(kf, vf, bits))
    # restore with entries -1 and num_pages: those positions stay NaN, the others are restored
    r = Session.open(_Pools(D, ps, hkv, 12, seed=5))
    rseq = r.alloc.seq_new()
    r.alloc.reserve(rseq, L)
    rbt = r.alloc.block_table(rseq).copy()
    rbt[0], rbt[2] = -1, r.desc.num_pages
    pkv.codec_decode(r.desc, r.k_pool, r.v_pool, i32(rbt), L, bits, payload)
    torch.cuda.synchronize()
    dk, _ = oracle_decode(payload.cpu().numpy(), (L, hkv, D), bits)
    kp = r.k_pool.view(torch.int16).cpu().numpy().view(np.uint16)
    page = int(rbt[1])
    assert np.array_equal(kp[page].transpose(1, 0, 2), _bf16_bits(dk[16:32]))
    others = [p for p in range(r.desc.num_pages) if p != page]
    assert np.isnan(host_f64(r.k_pool)[others]).all() and np.isnan(host_f64(r.v_pool)[others]).all()


def test_empty_prefix_is_a_no_op():
    s, seq, k, v = _stored_sequence(16, 128, 16, 8, seed=3)
    payload = torch.zeros((16,), dtype=torch.uint8, device=DEV)
    pkv.codec_encode(s.desc, s.k_pool, s.v_pool, i32(s.alloc.block_table(seq)), 0, 8, payload)
    torch.cuda.synchronize()
    assert not payload.any()
