"""pkv_decode_noalloc (decode with the library's static scratch, for callers
that cannot allocate) against pkv_decode with a caller workspace: the same
inputs give bit-identical outputs, on calls in a row of which the second is
smaller than the first (the scratch keeps the first call's contents) and the
third, on INT8 pages, larger.  A batch whose workspace exceeds the static
array is refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import pagedattention_pkv_store_amd as pkv
import synth
from conftest import ensure_library
from pagedattention_pkv_store_amd import _lib


@pytest.fixture(scope="module", autouse=True)
def _loaded():
    ensure_library()


def _decode_both(w, seed, kv_int8=False):
    """Store a decode batch, then run pkv_decode (workspace) and
    pkv_decode_noalloc on the same inputs; return both outputs."""
    from gpu_path import DEV, Session, dev_tensor, i32
    s = Session.open(w, kv_int8=kv_int8)
    seqs = [s.alloc.seq_new() for _ in w.lengths]
    items = []
    for b, seq in enumerate(seqs):
        L, lo = int(w.lengths[b]), int(w.offsets[b])
        s.alloc.reserve(seq, L)
        items.append((seq, 0, w.k[lo:lo + L], w.v[lo:lo + L]))
    s.store_many(items, w.dtype)
    q = dev_tensor(w.q, w.dtype)
    bt = i32(s.alloc.block_tables(seqs, max(s.alloc.num_blocks(x) for x in seqs)))
    lens = i32(np.array([s.alloc.seq_len(x) for x in seqs], np.int32))
    max_len = int(w.lengths.max())
    need = pkv.workspace_bytes(s.desc, len(seqs), w.num_q_heads, 1, max_len)
    assert 0 < need <= _lib.PKV_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref = torch.empty_like(q)
    pkv.decode(s.desc, s.k_pool, s.v_pool, q, bt, lens, max_len, s.scale, ref, ws)
    got = torch.full_like(q, float("nan"))
    pkv.decode_noalloc(s.desc, s.k_pool, s.v_pool, q, bt, lens, max_len, s.scale, got)
    torch.cuda.synchronize()
    return ref, got, need


@pytest.mark.gpu
def test_noalloc_decode_equals_decode_on_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    # first call: the 64-sequence GQA batch shape (lengths U{512..4096}, 32 / 8 heads of 128)
    w1 = synth.decode_batch(num_pages=16_384, seed=3)
    print("noalloc decode, call 1: 64 sequences", flush=True)
    ref1, got1, need1 = _decode_both(w1, 3)
    assert torch.isfinite(ref1.float()).all()
    assert torch.equal(got1, ref1), "call 1: pkv_decode_noalloc differs from pkv_decode"
    # second call, smaller: 9 sequences of 1..700 positions, 16 / 2 heads of 64
    w2 = synth.decode_batch(n_seqs=9, len_lo=1, len_hi=700, num_pages=200, num_q_heads=16, num_kv_heads=2,
                            head_dim=64, seed=4)
    print("noalloc decode, call 2: 9 sequences", flush=True)
    ref2, got2, need2 = _decode_both(w2, 4)
    assert need2 < need1
    assert torch.isfinite(ref2.float()).all()
    assert torch.equal(got2, ref2), "call 2: pkv_decode_noalloc differs from pkv_decode"
    # third call: the 64-sequence batch on INT8 pages (2048 waves: the largest workspace of the three)
    print("noalloc decode, call 3: 64 sequences on INT8 pages", flush=True)
    ref3, got3, need3 = _decode_both(w1, 5, kv_int8=True)
    assert need3 > need1
    assert torch.isfinite(ref3.float()).all()
    assert torch.equal(got3, ref3), "call 3: pkv_decode_noalloc differs from pkv_decode on INT8 pages"


def test_noalloc_decode_refuses_a_batch_beyond_the_scratch():
    """4,096 sequences x 8 KV heads need about 280 MB of partial states: the
    call fails with BUFFER_TOO_SMALL before touching any pointer or device."""
    L = _lib.lib()
    desc = _lib.PoolDescC(_lib.PKV_BF16, 300_000, 16, 8, 128)
    need = L.pkv_workspace_bytes(ctypes.byref(desc), 4096, 32, 1, 4096)
    assert need > _lib.PKV_NOALLOC_SCRATCH_BYTES
    rc = L.pkv_decode_noalloc(ctypes.byref(desc), None, None, None, 4096, 32, None, 256, None, 4096, 0.088,
                              None, None)
    assert rc == _lib.PKV_ERR_BUFFER_TOO_SMALL
    msg = _lib.last_error()
    assert "pkv_decode_noalloc" in msg and str(need) in msg and "pkv_decode" in msg
