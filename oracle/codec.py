"""Group-wise low-bit KV codec (the quantize / restore half of a KV handoff),
written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: ReKV, section 2.2.  The prefix KV tensors are quantized in groups of
G = 64 elements along the last dimension and sent as packed payloads with
one FP16 scale per group; the receiver dequantizes them.  With b in {4, 8}
bits per element the payload of E elements is E * (b/8 + 2/G) bytes
(eq. (7), without the boundary tensor).

Readings (also listed in the design notes):
* Symmetric groups (one scale, no zero point, as the two bytes per group in
  eq. (7) allow): scale = max|x| / q_max with q_max = 2^(b-1) - 1 (127 for
  Q8, 7 for Q4), computed in fp32 and rounded to fp16 (nearest, ties to
  even).  Codes use the stored scale: code = x / scale16, one IEEE fp32
  division per element (correctly rounded), rounded to the nearest integer
  (ties to even), clamped to [-q_max, q_max]; a zero scale gives zero codes.
  Restoring computes scale16 * code in fp32 (exact) and rounds it to the
  pool's bf16.
* Payload order: K, then V; within each, position-major, then KV head, then
  element, the same order as the logical KV; codes of all elements first,
  then the scales of all groups in the same order.  Q8 codes are bytes; Q4
  codes are 4-bit two's complement, element 2i in the low nibble of byte i
  and element 2i + 1 in the high nibble.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

GROUP = 64


def q_max(bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    return (1 << (bits - 1)) - 1


def payload_bytes(n_elements: int, bits: int) -> int:
    """eq. (7) for one tensor set: codes b/8 bytes per element plus a 2-byte
    scale per group of 64."""
    if n_elements % GROUP:
        raise ValueError("the element count must be whole groups")
    return n_elements * bits // 8 + 2 * (n_elements // GROUP)


def quantize_groups(x, bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """x: values exact in fp32, last axis a multiple of 64.  Returns (codes
    int8 with the shape of x, scales float16 [..., D/64])."""
    qm = np.float32(q_max(bits))
    x32 = np.asarray(x, dtype=np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("input values must be exact in float32")
    if x32.shape[-1] % GROUP:
        raise ValueError("last axis must be whole groups of 64")
    g = x32.reshape(x32.shape[:-1] + (x32.shape[-1] // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)
    scale16 = (amax / qm).astype(np.float32).astype(np.float16)
    sf = scale16.astype(np.float32)[..., None]
    safe = np.where(sf > 0, sf, np.float32(1))
    codes = np.rint((g / safe).astype(np.float32))
    codes = np.clip(codes, -qm, qm)
    codes = np.where(sf > 0, codes, 0.0)
    return codes.astype(np.int8).reshape(x32.shape), scale16


def dequantize_groups(codes, scales16) -> np.ndarray:
    """scale16 * code per element, float64 (exact)."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales16, dtype=np.float16).astype(np.float64)
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // GROUP, GROUP))
    return (g * s[..., None]).reshape(c.shape)


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes (int8, any shape, flattened in C order) -> payload code bytes."""
    flat = np.asarray(codes, dtype=np.int8).reshape(-1)
    if bits == 8:
        return flat.view(np.uint8).copy()
    if flat.size % 2:
        raise ValueError("Q4 packs pairs")
    nib = (flat.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def unpack(code_bytes: np.ndarray, bits: int, n: int) -> np.ndarray:
    b = np.asarray(code_bytes, dtype=np.uint8)
    if bits == 8:
        return b[:n].view(np.int8).copy()
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    out = np.empty(2 * b.size, np.int16)
    out[0::2], out[1::2] = lo, hi
    out = np.where(out >= 8, out - 16, out)
    return out[:n].astype(np.int8)


def encode(k, v, bits: int) -> np.ndarray:
    """A prefix's K and V ([L][Hkv][D] each, logical order) -> payload bytes."""
    ck, sk = quantize_groups(k, bits)
    cv, sv = quantize_groups(v, bits)
    codes = np.concatenate([pack(ck, bits), pack(cv, bits)])
    scales = np.concatenate([sk.reshape(-1), sv.reshape(-1)]).astype(np.float16)
    return np.concatenate([codes, scales.view(np.uint8)])


def decode(payload, shape, bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Payload bytes -> (K, V) as float64 values scale16 * code, each of
    ``shape`` = (L, Hkv, D)."""
    n = int(np.prod(shape))
    p = np.asarray(payload, dtype=np.uint8)
    code_bytes = n * bits // 8
    ck = unpack(p[:code_bytes], bits, n).reshape(shape)
    cv = unpack(p[code_bytes:2 * code_bytes], bits, n).reshape(shape)
    ng = n // GROUP
    sc = p[2 * code_bytes:2 * code_bytes + 4 * ng].view(np.float16)
    sk = sc[:ng].reshape(shape[:-1] + (shape[-1] // GROUP,))
    sv = sc[ng:].reshape(shape[:-1] + (shape[-1] // GROUP,))
    return dequantize_groups(ck, sk), dequantize_groups(cv, sv)
