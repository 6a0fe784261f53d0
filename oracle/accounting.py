"""Closed forms for KV bytes, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources
-------
* TileInfer.jl docs, "KV cache" -- "Sizing": the cache holds
  2 x layers x kv_heads x head_dim elements per position (keys and values of
  every layer and KV head); the sizing table lists per-position bytes for
  BFloat16 and INT8 and totals at 4,096 and 32,768 positions.  "INT8 cache":
  an INT8 vector of 128 values takes 132 bytes (128 one-byte codes plus one
  Float32 scale) instead of 256.
* ReKV, section 2.1, eqs. (1)-(2): a boundary hidden tensor holds S*d*e bytes
  and one layer's KV state 2*S*n_kv*d_h*e bytes.  Section 2.2, eq. (7): a
  b-bit prefix of c layers with groups of G elements and a two-byte scale per
  group takes c*E*(b/8 + 2/G) + 2*S*d bytes, E = 2*S*n_kv*d_h.
"""

from __future__ import annotations


def kv_elements_per_position(layers: int, kv_heads: int, head_dim: int) -> int:
    return 2 * layers * kv_heads * head_dim


def kv_bytes_per_position(layers: int, kv_heads: int, head_dim: int,
                          elem_bytes: int) -> int:
    return kv_elements_per_position(layers, kv_heads, head_dim) * elem_bytes


def int8_vector_bytes(head_dim: int) -> int:
    """One cached INT8 vector: head_dim one-byte codes and a 4-byte fp32 scale."""
    return head_dim + 4


def int8_kv_bytes_per_position(layers: int, kv_heads: int, head_dim: int) -> int:
    return 2 * layers * kv_heads * int8_vector_bytes(head_dim)


def boundary_bytes(seq: int, hidden: int, elem_bytes: int) -> int:
    """ReKV eq. (1): B_H = S d e."""
    return seq * hidden * elem_bytes


def layer_kv_bytes(seq: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """ReKV eq. (2): B_KV = 2 S n_kv d_h e."""
    return 2 * seq * kv_heads * head_dim * elem_bytes


def lowbit_payload_bytes(layers_sent: int, seq: int, kv_heads: int, head_dim: int,
                         bits: int, group: int, hidden: int) -> float:
    """ReKV eq. (7): c E (b/8 + 2/G) + 2 S d, with E = 2 S n_kv d_h."""
    elements = 2 * seq * kv_heads * head_dim
    return layers_sent * elements * (bits / 8 + 2 / group) + 2 * seq * hidden
