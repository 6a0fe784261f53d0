"""Paged KV storage and paged attention for MI355X (gfx950).

A thin Python binding over libpkv.so (C ABI in include/pkv.h).  Every step of
the path runs in the library: the host page allocator and prefix planner in
C++, the KV scatter and the paged attention kernels in HIP.  This module only
marshals arguments -- NumPy arrays for host calls, PyTorch tensors (device
memory) and the current HIP stream for device calls -- and turns error codes
into exceptions.  Nothing here computes a slot, a plan or an attention value.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import PKV_BF16, PKV_F32, PKV_I8  # noqa: F401

__all__ = [
    "PkvError", "OutOfPagesError", "SharedPageError", "UnsupportedError",
    "PoolDesc", "Allocator", "plan_prefix", "store_kv", "copy_pages", "decode", "decode_noalloc", "prefill_append",
    "codec_payload_bytes", "codec_encode", "codec_decode",
    "workspace_bytes", "validate_tables", "PKV_F32", "PKV_BF16", "PKV_I8",
    "BoundCall", "bind_store_kv", "bind_decode", "bind_prefill_append",
]


class PkvError(RuntimeError):
    """A libpkv call returned an error code."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class OutOfPagesError(PkvError):
    pass


class SharedPageError(PkvError):
    pass


class UnsupportedError(PkvError):
    pass


class BufferTooSmallError(PkvError):
    pass


_ERRORS = {
    _lib.PKV_ERR_OUT_OF_PAGES: OutOfPagesError,
    _lib.PKV_ERR_SHARED_PAGE: SharedPageError,
    _lib.PKV_ERR_UNSUPPORTED: UnsupportedError,
    _lib.PKV_ERR_BUFFER_TOO_SMALL: BufferTooSmallError,
}


def _check(rc: int) -> None:
    if rc != _lib.PKV_OK:
        raise _ERRORS.get(rc, PkvError)(rc, _lib.last_error())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---------------------------------------------------------------------------
# host: allocator and planner
# ---------------------------------------------------------------------------
class Allocator:
    """Host page allocator (pkv_alloc_*): free stack, block tables, refcounts."""

    def __init__(self, num_pages: int, page_size: int, free_order: Optional[Sequence[int]] = None):
        L = _lib.lib()
        handle = ctypes.c_void_p()
        if free_order is None:
            _check(L.pkv_alloc_create(num_pages, page_size, None, ctypes.byref(handle)))
        else:
            order = _i32(free_order)
            if order.size != num_pages:
                raise PkvError(_lib.PKV_ERR_INVALID_ARG, "free_order must have num_pages entries")
            _check(L.pkv_alloc_create(num_pages, page_size, _ptr(order, ctypes.c_int32),
                                      ctypes.byref(handle)))
        self._h = handle
        self._L = L
        self.num_pages = num_pages
        self.page_size = page_size

    def close(self) -> None:
        if self._h:
            self._L.pkv_alloc_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_new(self) -> int:
        out = ctypes.c_int32()
        _check(self._L.pkv_seq_new(self._h, ctypes.byref(out)))
        return out.value

    def reserve(self, seq: int, n: int) -> None:
        _check(self._L.pkv_reserve(self._h, seq, n))

    def truncate(self, seq: int, n_keep: int) -> None:
        _check(self._L.pkv_truncate(self._h, seq, n_keep))

    def release(self, seq: int) -> None:
        _check(self._L.pkv_release(self._h, seq))

    def share_prefix(self, child: int, parent: int, n_tokens: int) -> None:
        _check(self._L.pkv_share_prefix(self._h, child, parent, n_tokens))

    def fork(self, child: int, parent: int) -> None:
        """Empty ``child`` references all of ``parent``'s pages (pkv_fork)."""
        _check(self._L.pkv_fork(self._h, child, parent))

    def reserve_cow(self, seq: int, n: int) -> Optional[Tuple[int, int]]:
        """pkv_reserve with copy-on-write: returns (shared page, fresh page)
        when the device must copy a page before the new positions are stored
        (copy_pages), else None."""
        cp = (ctypes.c_int32 * 2)()
        nc = ctypes.c_int32()
        _check(self._L.pkv_reserve_cow(self._h, seq, n, cp, ctypes.byref(nc)))
        return (cp[0], cp[1]) if nc.value else None

    # -- KV retention pool -------------------------------------------------
    def retention_add(self, seq: int, probability_of_reuse: float, recompute_seconds: float) -> None:
        _check(self._L.pkv_retention_add(self._h, seq, float(probability_of_reuse), float(recompute_seconds)))

    def retention_evict(self, limit_pages: int, max_evicted: Optional[int] = None) -> np.ndarray:
        """Release lowest-priority retained sequences until at most limit_pages
        remain retained; returns their ids in eviction order."""
        cap = self.retention_pages() if max_evicted is None else max_evicted
        out = np.empty(max(1, cap), np.int32)
        n = ctypes.c_int32()
        _check(self._L.pkv_retention_evict(self._h, int(limit_pages), _ptr(out, ctypes.c_int32), cap,
                                           ctypes.byref(n)))
        return out[: n.value]

    def retention_take(self, seq: int) -> bool:
        avail = ctypes.c_int32()
        _check(self._L.pkv_retention_take(self._h, seq, ctypes.byref(avail)))
        return bool(avail.value)

    def retention_pages(self) -> int:
        n = ctypes.c_int64()
        _check(self._L.pkv_retention_pages(self._h, ctypes.byref(n)))
        return n.value

    def seq_len(self, seq: int) -> int:
        out = ctypes.c_int32()
        _check(self._L.pkv_seq_len(self._h, seq, ctypes.byref(out)))
        return out.value

    def num_free(self) -> int:
        out = ctypes.c_int32()
        _check(self._L.pkv_num_free(self._h, ctypes.byref(out)))
        return out.value

    def refcount(self, page: int) -> int:
        out = ctypes.c_int32()
        _check(self._L.pkv_page_refcount(self._h, page, ctypes.byref(out)))
        return out.value

    def num_blocks(self, seq: int) -> int:
        out = ctypes.c_int32()
        _check(self._L.pkv_seq_num_blocks(self._h, seq, ctypes.byref(out)))
        return out.value

    def block_table(self, seq: int) -> np.ndarray:
        n = self.num_blocks(seq)
        return self.block_tables([seq], n)[0]

    def block_tables(self, seqs: Sequence[int], stride: int,
                     out: Optional[np.ndarray] = None) -> np.ndarray:
        seqs_a = _i32(seqs)
        if out is None:
            out = np.zeros((len(seqs_a), stride), dtype=np.int32)
        if out.dtype != np.int32 or not out.flags.c_contiguous or out.shape != (len(seqs_a), stride):
            raise PkvError(_lib.PKV_ERR_INVALID_ARG, "out must be a C-contiguous int32 [n][stride]")
        _check(self._L.pkv_block_tables(self._h, _ptr(seqs_a, ctypes.c_int32), len(seqs_a),
                                        stride, _ptr(out, ctypes.c_int32)))
        return out

    def prepare_step(self, seqs: Sequence[int], n_new: Sequence[int], bt_stride: int,
                     slots_out: Optional[np.ndarray] = None, bt_out: Optional[np.ndarray] = None,
                     lens_out: Optional[np.ndarray] = None):
        """Reserve n_new[b] positions for each seqs[b] and return (slots of the
        new positions packed in b order, block tables [n][bt_stride], new
        lengths).  Preallocated (e.g. pinned) output arrays may be passed.
        bt_stride 0 skips the block-table export."""
        seqs_a = _i32(seqs)
        n_a = _i32(n_new)
        n = seqs_a.size
        total = int(n_a.sum())
        if slots_out is None:
            slots_out = np.empty(total, np.int64)
        if bt_out is None:
            bt_out = np.empty((n, bt_stride), np.int32)
        if lens_out is None:
            lens_out = np.empty(n, np.int32)
        if (slots_out.dtype != np.int64 or slots_out.size < total or bt_out.dtype != np.int32
                or bt_out.size < n * bt_stride or lens_out.dtype != np.int32 or lens_out.size < n
                or not (slots_out.flags.c_contiguous and bt_out.flags.c_contiguous
                        and lens_out.flags.c_contiguous)):
            raise PkvError(_lib.PKV_ERR_INVALID_ARG, "prepare_step: output arrays too small or wrong dtype")
        bt_ptr = _ptr(bt_out, ctypes.c_int32) if bt_stride > 0 else None  # 0: no tables
        _check(self._L.pkv_prepare_step(self._h, _ptr(seqs_a, ctypes.c_int32), n,
                                        _ptr(n_a, ctypes.c_int32), bt_stride,
                                        _ptr(slots_out, ctypes.c_int64), bt_ptr,
                                        _ptr(lens_out, ctypes.c_int32)))
        return slots_out[:total], bt_out.reshape(-1)[: n * bt_stride].reshape(n, bt_stride), lens_out[:n]

    def bind_prepare_step(self, seqs: Sequence[int], n_new: Sequence[int], bt_stride: int,
                          slots_out: np.ndarray, bt_out: Optional[np.ndarray], lens_out: np.ndarray) -> "BoundCall":
        """pkv_prepare_step with its arguments marshalled once, for a serving
        loop that repeats it on fixed (e.g. pinned) output arrays: each call
        reserves n_new[b] more positions for seqs[b] and rewrites the outputs
        (see prepare_step).  bt_out may be None (no block tables)."""
        seqs_a = _i32(seqs)
        n_a = _i32(n_new)
        n = seqs_a.size
        total = int(n_a.sum())
        if (slots_out.dtype != np.int64 or slots_out.size < total or lens_out.dtype != np.int32
                or lens_out.size < n or not (slots_out.flags.c_contiguous and lens_out.flags.c_contiguous)
                or (bt_out is not None and (bt_out.dtype != np.int32 or bt_out.size < n * bt_stride
                                            or not bt_out.flags.c_contiguous))):
            raise PkvError(_lib.PKV_ERR_INVALID_ARG, "prepare_step: output arrays too small or wrong dtype")
        bt_ptr = _ptr(bt_out, ctypes.c_int32) if bt_out is not None and bt_stride > 0 else None
        args = (self._h, _ptr(seqs_a, ctypes.c_int32), n, _ptr(n_a, ctypes.c_int32),
                bt_stride if bt_ptr is not None else 0, _ptr(slots_out, ctypes.c_int64), bt_ptr,
                _ptr(lens_out, ctypes.c_int32))
        return BoundCall(self._L.pkv_prepare_step, args, (self, seqs_a, n_a, slots_out, bt_out, lens_out))

    def slots(self, seq: int, start: int, n: int, out: Optional[np.ndarray] = None) -> np.ndarray:
        if out is None:
            out = np.empty(n, dtype=np.int64)
        if out.dtype != np.int64 or not out.flags.c_contiguous or out.size < n:
            raise PkvError(_lib.PKV_ERR_INVALID_ARG, "out must be a C-contiguous int64 array")
        _check(self._L.pkv_slots(self._h, seq, start, n, _ptr(out, ctypes.c_int64)))
        return out[:n]


def plan_prefix(docs_tokens: Sequence[np.ndarray], page_size: int
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Sharing plan (order, parent, shared) of documents given as token arrays.

    parent[d] = -1 for a document that shares nothing.
    """
    n = len(docs_tokens)
    lens = np.array([len(d) for d in docs_tokens], dtype=np.int64)
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    tokens = (np.concatenate([np.asarray(d, dtype=np.int32) for d in docs_tokens])
              if n else np.zeros(0, np.int32))
    tokens = _i32(tokens)
    return plan_prefix_packed(tokens, offsets, page_size)


def plan_prefix_packed(tokens: np.ndarray, offsets: np.ndarray, page_size: int
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    tokens = _i32(tokens)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    n = offsets.size - 1
    order = np.empty(n, np.int32)
    parent = np.empty(n, np.int32)
    shared = np.empty(n, np.int32)
    tok_ptr = _ptr(tokens, ctypes.c_int32) if tokens.size else None
    _check(_lib.lib().pkv_plan_prefix(tok_ptr, _ptr(offsets, ctypes.c_int64), n, page_size,
                                      _ptr(order, ctypes.c_int32), _ptr(parent, ctypes.c_int32),
                                      _ptr(shared, ctypes.c_int32)))
    return order, parent, shared


# ---------------------------------------------------------------------------
# device: store_kv / decode / prefill_append on PyTorch tensors
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class PoolDesc:
    dtype: int          # PKV_F32, PKV_BF16 or PKV_I8
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int

    def c(self) -> _lib.PoolDescC:
        return _lib.PoolDescC(self.dtype, self.num_pages, self.page_size, self.num_kv_heads,
                              self.head_dim)

    @property
    def pool_shape(self) -> Tuple[int, ...]:
        """Shape of one pool tensor: [num_pages][Hkv][page_size][D] elements,
        or for PKV_I8 [num_pages][Hkv][block bytes] (codes, then scales)."""
        if self.dtype == PKV_I8:
            return (self.num_pages, self.num_kv_heads,
                    int(_lib.lib().pkv_i8_block_bytes(self.page_size, self.head_dim)))
        return (self.num_pages, self.num_kv_heads, self.page_size, self.head_dim)

    def pool_bytes(self) -> int:
        n = int(_lib.lib().pkv_pool_bytes(ctypes.byref(self.c())))
        if n == 0:
            _check(_lib.PKV_ERR_UNSUPPORTED)
        return n

    def torch_dtype(self):
        """dtype of new K/V, queries and outputs (bf16 for INT8 pools)."""
        import torch
        return torch.float32 if self.dtype == PKV_F32 else torch.bfloat16

    def pool_torch_dtype(self):
        import torch
        return torch.int8 if self.dtype == PKV_I8 else self.torch_dtype()

    def new_pools(self, device, fill=None):
        """A (K, V) pair of pool tensors on ``device``.  ``fill``: a value for
        every element (fp32 / bf16 pools) or byte (PKV_I8 pools), or None."""
        import torch
        pools = []
        for _ in range(2):
            t = torch.empty(self.pool_shape, dtype=self.pool_torch_dtype(), device=device)
            if fill is not None:
                if self.dtype == PKV_I8:
                    t.view(torch.uint8).fill_(int(fill))
                else:
                    t.fill_(fill)
            pools.append(t)
        return pools[0], pools[1]


def _dev(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# Shape checks run before any pointer is taken: a tensor smaller than the call
# assumes would make a kernel read or write past its allocation.
def _need_shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_rows(t, name, n, dims=None):
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimension(s), got {t.dim()}")
    rows = int(t.shape[0]) if t.dim() else 0
    if rows < n:
        raise ValueError(f"{name} must have at least {n} rows, got {rows}")


def _need_pools(desc: "PoolDesc", k_pool, v_pool):
    need = desc.pool_bytes()
    for t, name in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        have = t.numel() * t.element_size()
        if have < need:
            raise ValueError(f"{name} holds {have} bytes; the pool descriptor needs {need}")


def _need_heads(desc: "PoolDesc", hq: int, d: int, name: str):
    if d != desc.head_dim:
        raise ValueError(f"{name}: last dimension {d} differs from the pool's head_dim {desc.head_dim}")
    if desc.num_kv_heads <= 0 or hq % desc.num_kv_heads:
        raise ValueError(f"{name}: {hq} query heads are not a multiple of {desc.num_kv_heads} KV heads")


class BoundCall:
    """A device call whose arguments were checked and marshalled once.

    Calling it enqueues the same launch again, with the same pointers, sizes
    and stream, for loops that repeat a call on fixed buffers (the values in
    those buffers may change between calls).  It keeps the tensors it was
    bound to alive."""

    __slots__ = ("_fn", "_args", "_keep")

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != _lib.PKV_OK:
            _check(rc)


def bind_store_kv(desc: PoolDesc, k_pool, v_pool, k_new, v_new, slots, stream=None) -> BoundCall:
    """pkv_store_kv with its arguments bound (see store_kv)."""
    import torch
    dt = desc.torch_dtype()
    pdt = desc.pool_torch_dtype()
    n = int(slots.numel())
    _need_pools(desc, k_pool, v_pool)
    row = desc.num_kv_heads * desc.head_dim
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if t.numel() < n * row:
            raise ValueError(f"{name} must hold at least slots.numel() * num_kv_heads * head_dim = {n * row} "
                             f"elements, got {t.numel()}")
    c_desc = desc.c()
    args = (ctypes.byref(c_desc), _dev(k_pool, "k_pool", pdt), _dev(v_pool, "v_pool", pdt),
            _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt), _dev(slots, "slots", torch.int64),
            n, _stream(stream))
    return BoundCall(_lib.lib().pkv_store_kv, args, (c_desc, k_pool, v_pool, k_new, v_new, slots))


def store_kv(desc: PoolDesc, k_pool, v_pool, k_new, v_new, slots, stream=None) -> None:
    """Scatter new K/V rows [T][Hkv][D] into the pools at int64 ``slots``."""
    bind_store_kv(desc, k_pool, v_pool, k_new, v_new, slots, stream)()


def copy_pages(desc: PoolDesc, k_pool, v_pool, copies, stream=None) -> None:
    """Copy whole pages in both pools: ``copies`` is a device int32 tensor
    [n][2] of (source, destination) page ids (pkv_copy_pages)."""
    import torch
    pdt = desc.pool_torch_dtype()
    n = int(copies.shape[0]) if copies.dim() == 2 else 0
    if copies.dim() != 2 or copies.shape[1] != 2:
        raise ValueError("copies must be [n][2]")
    _need_pools(desc, k_pool, v_pool)
    c_desc = desc.c()
    _check(_lib.lib().pkv_copy_pages(ctypes.byref(c_desc), _dev(k_pool, "k_pool", pdt), _dev(v_pool, "v_pool", pdt),
                                     _dev(copies, "copies", torch.int32), n, _stream(stream)))


def bind_stream_read(buf, partial_sums, stream=None) -> BoundCall:
    """pkv_stream_read with its arguments bound: read every byte of the device
    tensor ``buf`` once; ``partial_sums`` (device int32/uint32 [n]) receives the
    per-workgroup sums modulo 2^32 of its 32-bit words."""
    nbytes = buf.numel() * buf.element_size()
    if partial_sums.element_size() != 4 or not partial_sums.is_contiguous():
        raise ValueError("partial_sums must be a contiguous 32-bit tensor")
    args = (_dev(buf, "buf"), nbytes, _dev(partial_sums, "partial_sums"), int(partial_sums.numel()), _stream(stream))
    return BoundCall(_lib.lib().pkv_stream_read, args, (buf, partial_sums))


def stream_read(buf, partial_sums, stream=None) -> None:
    """Streaming read of a device buffer (a bandwidth measurement aid)."""
    bind_stream_read(buf, partial_sums, stream)()


def codec_payload_bytes(n_positions: int, num_kv_heads: int, head_dim: int, bits: int) -> int:
    n = int(_lib.lib().pkv_codec_payload_bytes(n_positions, num_kv_heads, head_dim, bits))
    if n == 0 and n_positions > 0:
        _check(_lib.PKV_ERR_UNSUPPORTED)
    return n


def _need_codec(desc, k_pool, v_pool, block_table, n_positions, bits, payload):
    _need_pools(desc, k_pool, v_pool)
    if n_positions < 0:
        raise ValueError("n_positions must be >= 0")
    blocks = -(-n_positions // desc.page_size) if desc.page_size > 0 else 0
    if block_table.numel() < blocks:
        raise ValueError(f"block_table must hold ceil(n_positions / page_size) = {blocks} entries, "
                         f"got {block_table.numel()}")
    need = codec_payload_bytes(n_positions, desc.num_kv_heads, desc.head_dim, bits) if n_positions else 0
    if payload.numel() * payload.element_size() < need:
        raise ValueError(f"payload must hold {need} bytes, got {payload.numel() * payload.element_size()}")


def codec_encode(desc: PoolDesc, k_pool, v_pool, block_table, n_positions: int, bits: int, payload,
                 stream=None) -> None:
    """Quantize a sequence's first n_positions K/V (read through its device
    block table) into a device uint8 payload (pkv_codec_encode)."""
    import torch
    pdt = desc.pool_torch_dtype()
    _need_codec(desc, k_pool, v_pool, block_table, n_positions, bits, payload)
    _check(_lib.lib().pkv_codec_encode(ctypes.byref(desc.c()), _dev(k_pool, "k_pool", pdt),
                                       _dev(v_pool, "v_pool", pdt), _dev(block_table, "block_table", torch.int32),
                                       n_positions, bits, _dev(payload, "payload", torch.uint8), _stream(stream)))


def codec_decode(desc: PoolDesc, k_pool, v_pool, block_table, n_positions: int, bits: int, payload,
                 stream=None) -> None:
    """Restore a payload into a sequence's first n_positions (pkv_codec_decode)."""
    import torch
    pdt = desc.pool_torch_dtype()
    _need_codec(desc, k_pool, v_pool, block_table, n_positions, bits, payload)
    _check(_lib.lib().pkv_codec_decode(ctypes.byref(desc.c()), _dev(k_pool, "k_pool", pdt),
                                       _dev(v_pool, "v_pool", pdt), _dev(block_table, "block_table", torch.int32),
                                       n_positions, bits, _dev(payload, "payload", torch.uint8), _stream(stream)))


def workspace_bytes(desc: PoolDesc, n_seqs: int, num_q_heads: int, max_q_per_seq: int,
                    max_seq_len: int) -> int:
    return int(_lib.lib().pkv_workspace_bytes(ctypes.byref(desc.c()), n_seqs, num_q_heads,
                                              max_q_per_seq, max_seq_len))


def _workspace(ws, need):
    if need == 0:
        return ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), 0
    if ws is None:
        raise PkvError(_lib.PKV_ERR_BUFFER_TOO_SMALL, f"workspace of {need} bytes required")
    _dev(ws, "workspace")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def bind_decode(desc: PoolDesc, k_pool, v_pool, q, block_tables, seq_lens, max_seq_len: int,
                scale: float, out, workspace=None, stream=None) -> BoundCall:
    """pkv_decode with its arguments bound (see decode)."""
    import torch
    dt = desc.torch_dtype()
    if q.dim() != 3:
        raise ValueError(f"q must be [n_seqs][num_q_heads][head_dim], got {tuple(q.shape)}")
    n_seqs, hq, d = (int(x) for x in q.shape)
    _need_heads(desc, hq, d, "q")
    _need_shape(out, "out", q.shape)
    _need_rows(block_tables, "block_tables", n_seqs, dims=2)
    _need_rows(seq_lens, "seq_lens", n_seqs, dims=1)
    _need_pools(desc, k_pool, v_pool)
    pdt = desc.pool_torch_dtype()
    need = workspace_bytes(desc, n_seqs, hq, 1, max_seq_len)
    ws_ptr, ws_bytes = _workspace(workspace, need)
    c_desc = desc.c()
    args = (ctypes.byref(c_desc), _dev(k_pool, "k_pool", pdt), _dev(v_pool, "v_pool", pdt),
            _dev(q, "q", dt), n_seqs, hq, _dev(block_tables, "block_tables", torch.int32),
            int(block_tables.shape[1]), _dev(seq_lens, "seq_lens", torch.int32), max_seq_len,
            float(scale), _dev(out, "out", dt), ws_ptr, ws_bytes, _stream(stream))
    keep = (c_desc, k_pool, v_pool, q, block_tables, seq_lens, out, workspace)
    return BoundCall(_lib.lib().pkv_decode, args, keep)


def decode(desc: PoolDesc, k_pool, v_pool, q, block_tables, seq_lens, max_seq_len: int,
           scale: float, out, workspace=None, stream=None) -> None:
    """Paged decode: q [B][Hq][D] -> out [B][Hq][D] (one new query per sequence)."""
    bind_decode(desc, k_pool, v_pool, q, block_tables, seq_lens, max_seq_len, scale, out,
                workspace, stream)()


def decode_noalloc(desc: PoolDesc, k_pool, v_pool, q, block_tables, seq_lens, max_seq_len: int,
                   scale: float, out, stream=None) -> None:
    """pkv_decode_noalloc: decode with the library's static scratch instead of
    a workspace (allocates nothing); refused when the batch needs more than
    PKV_NOALLOC_SCRATCH_BYTES of scratch."""
    import torch
    dt = desc.torch_dtype()
    if q.dim() != 3:
        raise ValueError(f"q must be [n_seqs][num_q_heads][head_dim], got {tuple(q.shape)}")
    n_seqs, hq, d = (int(x) for x in q.shape)
    _need_heads(desc, hq, d, "q")
    _need_shape(out, "out", q.shape)
    _need_rows(block_tables, "block_tables", n_seqs, dims=2)
    _need_rows(seq_lens, "seq_lens", n_seqs, dims=1)
    _need_pools(desc, k_pool, v_pool)
    pdt = desc.pool_torch_dtype()
    c_desc = desc.c()
    _check(_lib.lib().pkv_decode_noalloc(
        ctypes.byref(c_desc), _dev(k_pool, "k_pool", pdt), _dev(v_pool, "v_pool", pdt), _dev(q, "q", dt), n_seqs, hq,
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(seq_lens, "seq_lens", torch.int32), max_seq_len, float(scale), _dev(out, "out", dt), _stream(stream)))


def bind_prefill_append(desc: PoolDesc, k_pool, v_pool, q, cu_q, block_tables, seq_lens,
                        max_q_per_seq: int, max_seq_len: int, scale: float, out, workspace=None,
                        stream=None) -> BoundCall:
    """pkv_prefill_append with its arguments bound (see prefill_append)."""
    import torch
    dt = desc.torch_dtype()
    if q.dim() != 3:
        raise ValueError(f"q must be [total_q][num_q_heads][head_dim], got {tuple(q.shape)}")
    total_q, hq, d = (int(x) for x in q.shape)
    _need_heads(desc, hq, d, "q")
    _need_shape(out, "out", q.shape)
    if cu_q.dim() != 1 or cu_q.numel() < 1:
        raise ValueError("cu_q must be a 1-D tensor of n_seqs + 1 offsets")
    n_seqs = int(cu_q.numel()) - 1
    _need_rows(block_tables, "block_tables", n_seqs, dims=2)
    _need_rows(seq_lens, "seq_lens", n_seqs, dims=1)
    _need_pools(desc, k_pool, v_pool)
    pdt = desc.pool_torch_dtype()
    need = workspace_bytes(desc, n_seqs, hq, max_q_per_seq, max_seq_len)
    ws_ptr, ws_bytes = _workspace(workspace, need)
    c_desc = desc.c()
    args = (ctypes.byref(c_desc), _dev(k_pool, "k_pool", pdt), _dev(v_pool, "v_pool", pdt),
            _dev(q, "q", dt), total_q, _dev(cu_q, "cu_q", torch.int32), n_seqs, hq,
            _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
            _dev(seq_lens, "seq_lens", torch.int32), max_q_per_seq, max_seq_len, float(scale),
            _dev(out, "out", dt), ws_ptr, ws_bytes, _stream(stream))
    keep = (c_desc, k_pool, v_pool, q, cu_q, block_tables, seq_lens, out, workspace)
    return BoundCall(_lib.lib().pkv_prefill_append, args, keep)


def prefill_append(desc: PoolDesc, k_pool, v_pool, q, cu_q, block_tables, seq_lens,
                   max_q_per_seq: int, max_seq_len: int, scale: float, out, workspace=None,
                   stream=None) -> None:
    """Paged prefill/append over packed queries q [Tq][Hq][D] -> out [Tq][Hq][D]."""
    bind_prefill_append(desc, k_pool, v_pool, q, cu_q, block_tables, seq_lens, max_q_per_seq,
                        max_seq_len, scale, out, workspace, stream)()


def validate_tables(desc: PoolDesc, block_tables: np.ndarray, seq_lens: np.ndarray,
                    cu_q: Optional[np.ndarray] = None, max_q_per_seq: int = 0) -> None:
    """Host check of block tables / lengths / cu_q before a device call."""
    bt = _i32(block_tables)
    sl = _i32(seq_lens)
    cq = _i32(cu_q) if cu_q is not None else None
    n_seqs = sl.size
    stride = bt.shape[1] if bt.ndim == 2 else 0
    _check(_lib.lib().pkv_validate_tables(
        ctypes.byref(desc.c()), _ptr(bt, ctypes.c_int32), n_seqs, stride, _ptr(sl, ctypes.c_int32),
        _ptr(cq, ctypes.c_int32) if cq is not None else None, max_q_per_seq))
