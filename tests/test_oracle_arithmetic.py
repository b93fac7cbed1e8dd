"""Pins the oracle's memory arithmetic to the numbers the pages print."""

import math

from oracle import block_bytes, kv_bytes_per_token, kv_cache_bytes


def test_kv_cache_13b(golden):
    g = golden("memory_formulas.json")
    for key in ("kv_cache_13b_1000_tokens", "kv_cache_13b_4096_tokens"):
        c = g[key]
        assert kv_cache_bytes(c["layers"], c["heads"], c["head_dim"], c["seq_len"],
                              c["bytes"]) == c["expect"]
    c = g["kv_cache_13b_4096_tokens"]
    # printed "≈ 3.13 GB" is GiB: 3.125 rounded half-up to 2 places
    assert math.floor(c["expect"] / 2**30 * 100 + 0.5) / 100 == c["printed_gb"]
    ten = g["ten_requests_gb"]
    assert round(10 * c["printed_gb"], 1) == ten["expect"]
    assert round(100 * ten["expect"] / 80) == ten["a100_fraction_percent"]


def test_block_bytes_13b(golden):
    c = golden("memory_formulas.json")["block_13b"]
    b = block_bytes(c["layers"], c["heads"], c["head_dim"], c["bytes"], c["block_size"])
    assert b == c["expect"]
    assert b / 2**20 == c["printed_mb"]
    # One block over all layers = per-token bytes x 16.
    assert b == kv_bytes_per_token(40, 40, 128, 2) * 16


def test_script_7b(golden):
    c = golden("memory_formulas.json")["script_7b_128x4096"]
    total = kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["bytes"]) * c["tokens"]
    assert f"{total / 2**30:.1f}" == c["expect_gib_1dp"]
    # The 7B-shape block used by the mixed-length workload: 8 MiB over 32 layers.
    assert block_bytes(32, 32, 128, 2) == 8 * 2**20
    assert math.isclose(kv_cache_bytes(32, 32, 128, 4096, 2), 2 * 2**30)
