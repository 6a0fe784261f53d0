"""Softmax attention over a sequence's K/V gathered through its block table.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "KV Cache Management and PagedAttention", section "Compute attention
over scattered KV" (Figure 4).  The query of the input at position p uses the
keys and values of positions 0..p of its own request -- including its own,
just written -- read through the block table; other requests' pages and the
unused slots of the last page take no part; changing where the KV is stored
does not change the result.  So the paged method reaches exactly the result of
ordinary softmax attention over the request's logical K/V, and this oracle is
that definition: gather K/V into logical order through the block table, then
compute softmax attention in float64.

Readings (also listed in the design notes):
* The softmax scale is an argument (every caller passes 1/sqrt(head_dim)).
* Grouped-query attention maps query head h to KV head h // (Hq / Hkv).
* A sequence of length L with n new queries: query i sits at position
  L - n + i and sees positions 0..L-n+i (causal among the new block, full over
  everything stored before it -- shared-prefix pages or pages kept after a
  rewind).  Decode is the case n = 1.
* Inputs are upcast to float64 exactly (fp32 and bf16 are both exact in fp64).
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .paging import slot_of


def gather_kv(pool: np.ndarray, block_table: Sequence[int], length: int) -> np.ndarray:
    """Logical K (or V) of one sequence, [length][Hkv][D], from a pool.

    ``pool`` is laid out [num_pages][Hkv][page_size][D]; position p is read
    from page block_table[p // page_size] at offset p % page_size.
    """
    num_pages, hkv, page_size, d = pool.shape
    out = np.empty((length, hkv, d), dtype=np.float64)
    for p in range(length):
        slot = slot_of(block_table, p, page_size)
        out[p] = pool[slot // page_size, :, slot % page_size, :]
    return out


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Attention of n new queries over a sequence's logical K/V.

    q: [n][Hq][D]; k, v: [L][Hkv][D] with n <= L.  Returns [n][Hq][D] float64.
    Query i attends to positions 0 .. L - n + i.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    length, hkv, _ = k.shape
    if n > length:
        raise ValueError("more new queries than positions")
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    start = length - n
    visible = np.arange(length)[None, :] <= (start + np.arange(n))[:, None]  # [n][L]
    out = np.empty((n, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        z = scale * (q[:, h, :] @ k[:, g, :].T)          # [n][L]
        z = np.where(visible, z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        w = np.exp(z - m)                                # masked -> exp(-inf) = 0
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def attend_row(q_row: np.ndarray, k: np.ndarray, v: np.ndarray, position: int,
               scale: float) -> np.ndarray:
    """One query vector [D] at ``position`` over one KV head's k, v [L][D]."""
    q_row = np.asarray(q_row, dtype=np.float64)
    kk = np.asarray(k[: position + 1], dtype=np.float64)
    vv = np.asarray(v[: position + 1], dtype=np.float64)
    z = scale * (kk @ q_row)
    w = np.exp(z - z.max())
    return (w @ vv) / w.sum()


def paged_attention(q_packed: np.ndarray, cu_q: Sequence[int], seq_lens: Sequence[int],
                    block_tables: Sequence[Sequence[int]], k_pool: np.ndarray,
                    v_pool: np.ndarray, scale: float) -> np.ndarray:
    """Attention for a batch whose new queries are packed [Tq][Hq][D].

    Sequence b owns q_packed[cu_q[b] : cu_q[b+1]]; its K/V are the first
    seq_lens[b] positions read from the pools through block_tables[b].
    """
    out = np.zeros(q_packed.shape, dtype=np.float64)
    for b in range(len(seq_lens)):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        if hi == lo:
            continue
        length = int(seq_lens[b])
        k = gather_kv(k_pool, block_tables[b], length)
        v = gather_kv(v_pool, block_tables[b], length)
        out[lo:hi] = attend(q_packed[lo:hi], k, v, scale)
    return out
