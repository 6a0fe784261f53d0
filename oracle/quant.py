"""INT8 KV pages: one symmetric scale per cached vector, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: TileInfer.jl docs, "KV cache", section "INT8 cache".  In this mode
each cached vector (the keys or values of one KV head at one position) is
stored as Int8 codes plus a single Float32 scale, and x is approximated by
scale * code, symmetrically, with the scale set from the vector's largest
magnitude divided by 127.  Quantization happens at write time only, so no
scale is ever revised.  The attention kernels work on the codes directly and
apply the scales as factors: per key on its scores, per value on its
probability ahead of the PV product.  Storage per 128-element vector drops
from 256 bytes (BFloat16) to 132 (codes plus the 4-byte scale).

Readings where the page leaves a choice open (each is listed in the design
notes):
* Arithmetic of the code: the page fixes the scale's type (Float32) but not
  how a code is rounded.  Here both steps are IEEE float32 operations on the
  vector's values (exact for bf16 and fp32 inputs): scale = max|x| / 127, then
  code = x / scale rounded to the nearest integer, ties to even (the default
  rounding of the page's language and of IEEE arithmetic), kept in
  [-127, 127].  For a normal float32 scale |x / scale| exceeds 127 by at most
  a rounding step, so the bound only acts when max|x| is so small that the
  scale is subnormal.
* A vector of zeros has scale 0; its codes are 0 (x / scale is undefined).
* Attention over an INT8 pool is attention over the values scale * code.
  Folding the scales into the scores and the probabilities, as the page
  describes, computes the same products in another order, so the oracle
  dequantizes (exactly, in float64) and applies the attention definition of
  ``oracle.attention``.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .attention import attend, paged_attention

CODE_MAX = 127


def quantize(x) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize vectors along the last axis.

    x: float array [..., D] (its values must be exact in float32).  Returns
    (codes int8 [..., D], scales float32 [...]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("input values must be exact in float32")
    amax = np.max(np.abs(x32), axis=-1)                       # exact
    scales = (amax / np.float32(CODE_MAX)).astype(np.float32)  # one float32 division
    safe = np.where(scales > 0, scales, np.float32(1))[..., None]
    ratio = (x32 / safe).astype(np.float32)                    # one float32 division
    codes = np.rint(ratio)                                     # nearest, ties to even
    codes = np.clip(codes, -CODE_MAX, CODE_MAX)
    codes = np.where(scales[..., None] > 0, codes, 0.0)
    return codes.astype(np.int8), scales


def dequantize(codes, scales) -> np.ndarray:
    """scale * code in float64 (exact: a float32 times an 8-bit integer)."""
    return np.asarray(scales, dtype=np.float64)[..., None] * np.asarray(codes, dtype=np.float64)


def store_rows_int8(code_pool: np.ndarray, scale_pool: np.ndarray, slots: Sequence[int], rows) -> None:
    """store_kv into an INT8 pool: quantize each new row ([Hkv][D] per token)
    once, then write codes and scales at the token's slot.

    code_pool: int8 [num_pages][Hkv][ps][D]; scale_pool: float32
    [num_pages][Hkv][ps].  Slots outside the pool are skipped.
    """
    page_size = code_pool.shape[2]
    limit = code_pool.shape[0] * page_size
    for t, slot in enumerate(slots):
        slot = int(slot)
        if 0 <= slot < limit:
            codes, scales = quantize(rows[t])
            code_pool[slot // page_size, :, slot % page_size, :] = codes
            scale_pool[slot // page_size, :, slot % page_size] = scales


def attend_int8(q, k, v, scale: float) -> np.ndarray:
    """Attention of n new queries over a sequence's logical K/V held in INT8.

    q: [n][Hq][D]; k, v: (codes [L][Hkv][D], scales [L][Hkv]).  Query i sits
    at position L - n + i, as in ``oracle.attention.attend``.
    """
    return attend(q, dequantize(*k), dequantize(*v), scale)


def paged_attention_int8(q_packed, cu_q, seq_lens, block_tables, k_pools, v_pools,
                         scale: float) -> np.ndarray:
    """``oracle.attention.paged_attention`` over INT8 pools: k_pools, v_pools =
    (codes [num_pages][Hkv][ps][D], scales [num_pages][Hkv][ps]) read through
    the block tables, dequantized, then the attention definition."""
    return paged_attention(q_packed, cu_q, seq_lens, block_tables, dequantize(*k_pools),
                           dequantize(*v_pools), scale)


def quantize_then_attend(q, k_values, v_values, scale: float) -> np.ndarray:
    """What a query sees when the K/V it attends to were written to an INT8
    cache: each vector quantized at store time, then attention over the
    stored values."""
    return attend_int8(q, quantize(k_values), quantize(v_values), scale)
