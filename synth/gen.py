"""Seeded generators for the five paged-attention workloads.

No method arithmetic lives here (see ``synth/__init__.py``).  Value arrays are
float32 for ``F32`` workloads and raw bfloat16 bit patterns (uint16) for
``BF16`` workloads; ``to_f64`` widens either exactly.

Workload ids (used in the seed's spawn key):
  1  tiny fp32 paged attention (page_size 4, 6-page pool, lengths 7 and 6)
  2  paged decode batch (64 sequences, lengths U{512..4096}, page_size 16)
  3  prefix-shared prefill over agent-trace rows (256 rows, 32 traces)
  4  KV rewind (1,000 documents of 300 tokens, two 50-token questions)
  5  long-context decode with speculative rollback (8 sequences, 32K-128K)
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

F32 = "f32"
BF16 = "bf16"

_STREAMS = {
    "pages": 0, "lengths": 1, "tokens": 2, "q": 3, "k": 4, "v": 5,
    "keep": 6, "trace_of": 7, "draft_q": 8, "draft_k": 9, "draft_v": 10,
    "q1": 11, "k1": 12, "v1": 13, "q2": 14, "k2": 15, "v2": 16,
}


def generator(workload: int, stream: str, seed: int = 0, instance: int = 0) -> np.random.Generator:
    """Independent NumPy generator for one quantity of one workload instance."""
    return np.random.default_rng(
        np.random.SeedSequence(seed, spawn_key=(workload, _STREAMS[stream], instance)))


# ---------------------------------------------------------------------------
# value encoding
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite N(0,1) draws, so no NaN/Inf handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(values: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 image of generated values (f32 array or bf16 bit array)."""
    if dtype == F32:
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f32(values).astype(np.float64)
    raise ValueError(dtype)


def normal_values(gen: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) drawn in float32; bf16 workloads get the rounded bit patterns."""
    x = gen.standard_normal(size=shape, dtype=np.float32)
    if dtype == F32:
        return x
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def _offsets(lengths: Sequence[int]) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


# ---------------------------------------------------------------------------
# workload 1: tiny fp32
# ---------------------------------------------------------------------------
@dataclass
class TinyBatch:
    """Two sequences B (7 positions) and C (6) in a 6-page pool of 4-slot pages.

    ``k``/``v``/``q`` are packed over all positions of both sequences
    (offsets ``offsets``); every position has a query, so a causal prefill of
    all positions and a decode of the last position can both be formed.
    """
    dtype: str
    page_size: int
    num_pages: int
    free_order: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lengths: np.ndarray
    offsets: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray


def tiny_batch(seed: int = 0, free_order: Optional[Sequence[int]] = None) -> TinyBatch:
    wl = 1
    ps, num_pages, hq, hkv, d = 4, 6, 2, 1, 64
    lengths = np.array([7, 6], dtype=np.int64)
    if free_order is None:
        free_order = generator(wl, "pages", seed).permutation(num_pages)
    total = int(lengths.sum())
    return TinyBatch(
        dtype=F32, page_size=ps, num_pages=num_pages,
        free_order=np.asarray(free_order, dtype=np.int32),
        num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        lengths=lengths, offsets=_offsets(lengths),
        q=normal_values(generator(wl, "q", seed), (total, hq, d), F32),
        k=normal_values(generator(wl, "k", seed), (total, hkv, d), F32),
        v=normal_values(generator(wl, "v", seed), (total, hkv, d), F32),
    )


# ---------------------------------------------------------------------------
# workload 2: paged decode batch
# ---------------------------------------------------------------------------
@dataclass
class DecodeBatch:
    """B sequences; ``lengths[b]`` counts the new token (stored, then attended).

    ``k``/``v`` hold every position of every sequence, packed by ``offsets``;
    ``q`` is the one new query per sequence, [B][Hq][D].
    """
    dtype: str
    page_size: int
    num_pages: int
    free_order: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lengths: np.ndarray
    offsets: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray


def decode_batch(n_seqs: int = 64, len_lo: int = 512, len_hi: int = 4096,
                 num_pages: int = 300_000, page_size: int = 16,
                 num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                 dtype: str = BF16, seed: int = 0, instance: int = 0,
                 workload: int = 2) -> DecodeBatch:
    g = lambda s: generator(workload, s, seed, instance)  # noqa: E731
    lengths = g("lengths").integers(len_lo, len_hi, size=n_seqs, endpoint=True).astype(np.int64)
    total = int(lengths.sum())
    return DecodeBatch(
        dtype=dtype, page_size=page_size, num_pages=num_pages,
        free_order=g("pages").permutation(num_pages).astype(np.int32),
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        lengths=lengths, offsets=_offsets(lengths),
        q=normal_values(g("q"), (n_seqs, num_q_heads, head_dim), dtype),
        k=normal_values(g("k"), (total, num_kv_heads, head_dim), dtype),
        v=normal_values(g("v"), (total, num_kv_heads, head_dim), dtype),
    )


# ---------------------------------------------------------------------------
# workload 3: prefix-shared prefill over agent traces
# ---------------------------------------------------------------------------
@dataclass
class PrefixTraces:
    """Rows that are prefixes of agent traces.

    Trace t has ``trace_len`` random token ids and per-position Q/K/V
    (``q[t]`` [trace_len][Hq][D], ``k[t]``/``v[t]`` [trace_len][Hkv][D]).  Row
    r is the first ``row_len[r]`` tokens of trace ``row_trace[r]``; its Q/K/V
    at position p are its trace's at p, so equal prefixes carry equal KV.
    Rows 0-2 are the first 1,000 / 1,400 / 1,900 tokens of trace 0.
    """
    dtype: str
    page_size: int
    num_pages: int
    free_order: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    trace_tokens: np.ndarray   # [n_traces][trace_len] int32
    row_trace: np.ndarray      # [n_rows] int64
    row_len: np.ndarray        # [n_rows] int64
    q: Optional[np.ndarray]    # None when drawn without values
    k: Optional[np.ndarray]
    v: Optional[np.ndarray]

    def row_tokens(self, r: int) -> np.ndarray:
        return self.trace_tokens[self.row_trace[r], : self.row_len[r]]


def prefix_traces(n_rows: int = 256, n_traces: int = 32,
                  first_rows: Sequence[int] = (1000, 1400, 1900),
                  len_lo: int = 1000, len_hi: int = 8000, trace_len: int = 8000,
                  num_pages: int = 100_000, page_size: int = 16,
                  num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                  dtype: str = BF16, seed: int = 0, instance: int = 0,
                  workload: int = 3, values: bool = True) -> PrefixTraces:
    """``values=False`` draws only the structure (tokens, lengths, pages)."""
    g = lambda s: generator(workload, s, seed, instance)  # noqa: E731
    n_rest = n_rows - len(first_rows)
    rest_trace = g("trace_of").integers(1, n_traces - 1, size=n_rest, endpoint=True)
    rest_len = g("lengths").integers(len_lo, len_hi, size=n_rest, endpoint=True)
    row_trace = np.concatenate([np.zeros(len(first_rows), np.int64), rest_trace]).astype(np.int64)
    row_len = np.concatenate([np.asarray(first_rows, np.int64), rest_len]).astype(np.int64)
    tokens = g("tokens").integers(0, 2**31 - 1, size=(n_traces, trace_len)).astype(np.int32)
    return PrefixTraces(
        dtype=dtype, page_size=page_size, num_pages=num_pages,
        free_order=g("pages").permutation(num_pages).astype(np.int32),
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        trace_tokens=tokens, row_trace=row_trace, row_len=row_len,
        q=normal_values(g("q"), (n_traces, trace_len, num_q_heads, head_dim), dtype) if values else None,
        k=normal_values(g("k"), (n_traces, trace_len, num_kv_heads, head_dim), dtype) if values else None,
        v=normal_values(g("v"), (n_traces, trace_len, num_kv_heads, head_dim), dtype) if values else None,
    )


# ---------------------------------------------------------------------------
# workload 4: KV rewind
# ---------------------------------------------------------------------------
@dataclass
class RewindDocs:
    """Documents of ``doc_len`` positions and two questions of ``q_len`` each.

    ``doc_k``/``doc_v`` [n_docs][doc_len][Hkv][D]; question j (1 or 2) has
    ``qj_q`` [n_docs][q_len][Hq][D] and ``qj_k``/``qj_v`` [n_docs][q_len][Hkv][D].
    """
    dtype: str
    page_size: int
    num_pages: int
    free_order: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    doc_len: int
    q_len: int
    doc_k: np.ndarray
    doc_v: np.ndarray
    q1_q: np.ndarray
    q1_k: np.ndarray
    q1_v: np.ndarray
    q2_q: np.ndarray
    q2_k: np.ndarray
    q2_v: np.ndarray


def rewind_docs(n_docs: int = 1000, doc_len: int = 300, q_len: int = 50,
                num_pages: int = 32_768, page_size: int = 16,
                num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                dtype: str = BF16, seed: int = 0, instance: int = 0,
                workload: int = 4) -> RewindDocs:
    g = lambda s: generator(workload, s, seed, instance)  # noqa: E731
    kv_doc = (n_docs, doc_len, num_kv_heads, head_dim)
    kv_q = (n_docs, q_len, num_kv_heads, head_dim)
    qq = (n_docs, q_len, num_q_heads, head_dim)
    return RewindDocs(
        dtype=dtype, page_size=page_size, num_pages=num_pages,
        free_order=g("pages").permutation(num_pages).astype(np.int32),
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        doc_len=doc_len, q_len=q_len,
        doc_k=normal_values(g("k"), kv_doc, dtype),
        doc_v=normal_values(g("v"), kv_doc, dtype),
        q1_q=normal_values(g("q1"), qq, dtype),
        q1_k=normal_values(g("k1"), kv_q, dtype),
        q1_v=normal_values(g("v1"), kv_q, dtype),
        q2_q=normal_values(g("q2"), qq, dtype),
        q2_k=normal_values(g("k2"), kv_q, dtype),
        q2_v=normal_values(g("v2"), kv_q, dtype),
    )


# ---------------------------------------------------------------------------
# workload 5: long-context decode with speculative rollback
# ---------------------------------------------------------------------------
@dataclass
class SpecDecode:
    """Long sequences that repeatedly take ``drafts`` draft tokens and keep some.

    ``ctx_k``/``ctx_v`` hold each sequence's initial ``ctx_len[b]`` positions,
    packed by ``ctx_offsets``.  Step s drafts ``draft_q[s]`` [B][drafts][Hq][D]
    and ``draft_k[s]``/``draft_v[s]`` [B][drafts][Hkv][D]; after verifying, a
    sequence keeps the first ``keep[s][b]`` drafts (0..drafts).
    """
    dtype: str
    page_size: int
    num_pages: int
    free_order: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    drafts: int
    ctx_len: np.ndarray
    ctx_offsets: np.ndarray
    ctx_k: np.ndarray
    ctx_v: np.ndarray
    draft_q: np.ndarray
    draft_k: np.ndarray
    draft_v: np.ndarray
    keep: np.ndarray


def spec_decode(n_seqs: int = 8, len_lo: int = 32_768, len_hi: int = 131_072,
                steps: int = 16, drafts: int = 5, page_size: int = 64,
                num_q_heads: int = 64, num_kv_heads: int = 8, head_dim: int = 128,
                num_pages: Optional[int] = None, dtype: str = BF16, seed: int = 0,
                instance: int = 0, workload: int = 5) -> SpecDecode:
    g = lambda s: generator(workload, s, seed, instance)  # noqa: E731
    ctx_len = g("lengths").integers(len_lo, len_hi, size=n_seqs, endpoint=True).astype(np.int64)
    if num_pages is None:
        # Room for every sequence at its longest (all drafts of all steps kept),
        # doubled so pages scatter over a pool twice the live size.
        longest = ctx_len + steps * drafts
        num_pages = int(2 * sum(-(-int(x) // page_size) for x in longest))
    total = int(ctx_len.sum())
    return SpecDecode(
        dtype=dtype, page_size=page_size, num_pages=num_pages,
        free_order=g("pages").permutation(num_pages).astype(np.int32),
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        drafts=drafts, ctx_len=ctx_len, ctx_offsets=_offsets(ctx_len),
        ctx_k=normal_values(g("k"), (total, num_kv_heads, head_dim), dtype),
        ctx_v=normal_values(g("v"), (total, num_kv_heads, head_dim), dtype),
        draft_q=normal_values(g("draft_q"), (steps, n_seqs, drafts, num_q_heads, head_dim), dtype),
        draft_k=normal_values(g("draft_k"), (steps, n_seqs, drafts, num_kv_heads, head_dim), dtype),
        draft_v=normal_values(g("draft_v"), (steps, n_seqs, drafts, num_kv_heads, head_dim), dtype),
        keep=g("keep").integers(0, drafts, size=(steps, n_seqs), endpoint=True).astype(np.int64),
    )
