"""Pins for the oracle's byte accounting against the printed figures.

TileInfer.jl "KV cache", sections "Sizing" and "INT8 cache"
(tests/golden/tileinfer_sizing.json); ReKV sections 2.1-2.2 and 4.2
(tests/golden/rekv_bytes.json).
"""

from oracle.accounting import (boundary_bytes, int8_kv_bytes_per_position, int8_vector_bytes,
                               kv_bytes_per_position, layer_kv_bytes, lowbit_payload_bytes)

KIB = 1024
MIB = 1024 * 1024


def test_tileinfer_sizing_table(golden):
    ex = golden("tileinfer_sizing.json")
    assert int8_vector_bytes(128) == ex["int8_vector_bytes"]
    assert 128 * 2 == ex["bf16_vector_bytes"]
    for row in ex["rows"]:
        bf16 = kv_bytes_per_position(row["layers"], row["kv_heads"], row["head_dim"], 2)
        assert bf16 == row["per_position_bf16_kib"] * KIB           # exact
        i8 = int8_kv_bytes_per_position(row["layers"], row["kv_heads"], row["head_dim"])
        assert round(i8 / KIB) == row["per_position_int8_kib"]      # 57.75, 74.25
        assert round(4096 * bf16 / 1e9, 2) == row["gb_4096_bf16"]
        assert round(32768 * bf16 / 1e9, 1) == row["gb_32768_bf16"]


def test_rekv_byte_model(golden):
    ex = golden("rekv_bytes.json")
    S, d, nkv, dh = ex["seq"], ex["hidden"], ex["kv_heads"], ex["head_dim"]
    assert boundary_bytes(S, d, 2) == ex["boundary_mib"] * MIB
    assert layer_kv_bytes(S, nkv, dh, 2) == ex["bf16_layer_mib"] * MIB
    assert boundary_bytes(S, d, 2) / layer_kv_bytes(S, nkv, dh, 2) == ex["ratio_hidden_to_kv"]
    q8_layer = lowbit_payload_bytes(1, S, nkv, dh, 8, ex["group"], 0)
    assert q8_layer == ex["q8_layer_mib"] * MIB
    assert lowbit_payload_bytes(ex["q8_prefix_layers"], S, nkv, dh, 8, ex["group"], d) \
        == ex["q8_prefix_plus_boundary_mib"] * MIB
    assert lowbit_payload_bytes(ex["layers"], S, nkv, dh, 8, ex["group"], 0) \
        == ex["full_q8_mib"] * MIB
    assert ex["layers"] * layer_kv_bytes(S, nkv, dh, 2) == ex["full_bf16_mib"] * MIB
