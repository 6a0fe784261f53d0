"""The binding refuses tensors whose shapes do not match the call before it
takes a pointer or enqueues anything: a tensor smaller than a launch assumes
would let a kernel read or write past its allocation.  CPU tensors of the
wrong shape raise ValueError naming the argument; with the right shapes the
same CPU tensors get as far as the device check ("must be a device")."""

import numpy as np
import pytest
import torch

import pagedattention_pkv_store_amd as pkv
from conftest import ensure_library


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _desc(dtype=pkv.PKV_BF16):
    return pkv.PoolDesc(dtype, 10, 16, 2, 128)


def _pools(desc, pages=None):
    shape = list(desc.pool_shape)
    if pages is not None:
        shape[0] = pages
    return (torch.zeros(shape, dtype=desc.pool_torch_dtype()),
            torch.zeros(shape, dtype=desc.pool_torch_dtype()))


def _decode_args(n=3, hq=8, d=128):
    desc = _desc()
    kp, vp = _pools(desc)
    q = torch.zeros((n, hq, d), dtype=torch.bfloat16)
    return dict(desc=desc, k_pool=kp, v_pool=vp, q=q, block_tables=torch.zeros((n, 4), dtype=torch.int32),
                seq_lens=torch.ones(n, dtype=torch.int32), max_seq_len=64, scale=0.1, out=torch.empty_like(q),
                workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def test_decode_shapes_are_checked():
    with pytest.raises(ValueError, match="must be a device"):
        pkv.bind_decode(**_decode_args())
    a = _decode_args()
    a["out"] = torch.empty((3, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must have shape"):
        pkv.bind_decode(**a)
    with pytest.raises(ValueError, match="head_dim"):
        pkv.bind_decode(**_decode_args(d=64))
    with pytest.raises(ValueError, match="multiple"):
        pkv.bind_decode(**_decode_args(hq=3))
    a = _decode_args()
    a["block_tables"] = torch.zeros((2, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="block_tables must have at least 3 rows"):
        pkv.bind_decode(**a)
    a = _decode_args()
    a["block_tables"] = torch.zeros(12, dtype=torch.int32)
    with pytest.raises(ValueError, match="block_tables must have 2"):
        pkv.bind_decode(**a)
    a = _decode_args()
    a["seq_lens"] = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="seq_lens"):
        pkv.bind_decode(**a)
    a = _decode_args()
    a["k_pool"] = _pools(a["desc"], pages=9)[0]
    with pytest.raises(ValueError, match="k_pool holds"):
        pkv.bind_decode(**a)
    a = _decode_args()
    a["q"] = torch.zeros((3, 8 * 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be"):
        pkv.bind_decode(**a)


def _prefill_args(total=7, n=2):
    desc = _desc()
    kp, vp = _pools(desc)
    q = torch.zeros((total, 8, 128), dtype=torch.bfloat16)
    return dict(desc=desc, k_pool=kp, v_pool=vp, q=q, cu_q=torch.tensor([0, 3, total][: n + 1], dtype=torch.int32),
                block_tables=torch.zeros((n, 4), dtype=torch.int32), seq_lens=torch.full((n,), 8, dtype=torch.int32),
                max_q_per_seq=4, max_seq_len=64, scale=0.1, out=torch.empty_like(q),
                workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def test_prefill_shapes_are_checked():
    with pytest.raises(ValueError, match="must be a device"):
        pkv.bind_prefill_append(**_prefill_args())
    a = _prefill_args()
    a["out"] = torch.empty((6, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must have shape"):
        pkv.bind_prefill_append(**a)
    a = _prefill_args()
    a["seq_lens"] = torch.full((1,), 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="seq_lens"):
        pkv.bind_prefill_append(**a)
    a = _prefill_args()
    a["cu_q"] = torch.zeros((2, 2), dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_q"):
        pkv.bind_prefill_append(**a)
    a = _prefill_args()
    a["v_pool"] = torch.zeros(5, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="v_pool holds"):
        pkv.bind_prefill_append(**a)


def test_store_kv_row_counts_are_checked():
    desc = _desc()
    kp, vp = _pools(desc)
    slots = torch.arange(5, dtype=torch.int64)
    good = torch.zeros((5, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be a device"):
        pkv.bind_store_kv(desc, kp, vp, good, good, slots)
    short = torch.zeros((4, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_new must hold"):
        pkv.bind_store_kv(desc, kp, vp, short, good, slots)
    with pytest.raises(ValueError, match="v_new must hold"):
        pkv.bind_store_kv(desc, kp, vp, good, short, slots)


def test_codec_table_and_payload_sizes_are_checked():
    desc = _desc()
    kp, vp = _pools(desc)
    n = 40                                             # 3 pages of 16
    payload = torch.zeros(pkv.codec_payload_bytes(n, 2, 128, 8), dtype=torch.uint8)
    with pytest.raises(ValueError, match="must be a device"):
        pkv.codec_encode(desc, kp, vp, torch.zeros(3, dtype=torch.int32), n, 8, payload)
    for fn in (pkv.codec_encode, pkv.codec_decode):
        with pytest.raises(ValueError, match="block_table must hold"):
            fn(desc, kp, vp, torch.zeros(2, dtype=torch.int32), n, 8, payload)
        with pytest.raises(ValueError, match="payload must hold"):
            fn(desc, kp, vp, torch.zeros(3, dtype=torch.int32), n, 8, payload[:-1])
