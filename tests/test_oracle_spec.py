"""Pins of the oracle's layout constants against the figures the pages print."""

import json
import math
import os

import pytest

from oracle import spec

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_block_densities_match_printed_values():
    d = GOLD["densities_bytes_per_element"]
    assert spec.bytes_per_element(spec.Q4_0, 128) == d["q4_0"]
    assert spec.bytes_per_element(spec.Q6_0, 256) == d["q6_0"]
    assert spec.bytes_per_element(spec.Q8_0, 128) == d["q8_0"]
    # density is a per-block property: the same for every multiple of 32
    for D in (32, 64, 96, 128, 256, 512):
        assert spec.bytes_per_element(spec.Q4_0, D) == d["q4_0"]
        assert spec.bytes_per_element(spec.Q6_0, D) == d["q6_0"]
        assert spec.bytes_per_element(spec.Q8_0, D) == d["q8_0"]


def test_bytes_per_token_table_is_density_over_bf16():
    t = GOLD["bytes_per_token_table"]
    d = GOLD["densities_bytes_per_element"]
    elems = t["bf16"] / d["bf16"]            # elements per token of that model
    assert elems * spec.bytes_per_element(spec.Q4_0, 128) == t["q4_0"]
    assert elems * spec.bytes_per_element(spec.Q6_0, 128) == t["q6_0"]
    assert elems * d["q8_0"] == t["q8_0"]
    assert elems * spec.bytes_per_element(spec.Q8_0, 128) == t["q8_0"]
    for n_tok, gib in GOLD["gib_at_context"]["q4_0"]:
        assert round(n_tok * t["q4_0"] / 2**30, 2) == gib


def test_asym_g32_compression_ratio():
    a = GOLD["asym_g32_compression_vs_fp16"]
    bpe = spec.bytes_per_element(spec.ASYM_G32, 128)
    assert bpe == 0.625
    assert 2.0 / bpe == a["ratio"]


def test_had_int4_per_head_memory_table():
    h = GOLD["had_int4_per_head_kb"]
    D = h["head_dim"]
    row = spec.payload_bytes(spec.HAD_INT4, D) + spec.scale_bytes(spec.HAD_INT4, D)
    assert row == 68  # 64 nibble bytes + one f32 scale
    for T, f16kb, i4kb in zip(h["T"], h["f16_kb"], h["int4_kb"]):
        assert 2 * T * row == i4kb * 1024          # K and V
        assert 2 * T * D * 2 == f16kb * 1024


def test_had_int4_per_token_model_figure():
    m = GOLD["had_int4_per_token_model"]
    f16 = m["layers"] * 2 * m["kv_heads"] * m["head_dim"] * 2
    assert f16 == m["f16_bytes_per_token"]
    nibbles = m["layers"] * 2 * m["kv_heads"] * spec.payload_bytes(spec.HAD_INT4, m["head_dim"])
    assert nibbles * 4 == f16
    assert nibbles == m["int4_kb_per_token"] * 1024


def test_code_ranges_and_magnitudes():
    r = GOLD["q4_0_symmetric_range"]
    assert spec.code_range(spec.Q4_0) == (r["lo"], r["hi"])
    assert spec.max_magnitude(spec.Q4_0) == r["max_magnitude"]
    assert spec.code_range(spec.HAD_INT4) == (-8, 7)
    assert spec.code_range(spec.Q6_0) == (-32, 31)
    assert spec.max_magnitude(spec.Q6_0) == 32
    assert spec.code_range(spec.ASYM_G32) == (0, 15)
    # q8_0: 2^(bits-1) by the same rule as q6_0
    assert spec.code_range(spec.Q8_0) == (-128, 127)
    assert spec.max_magnitude(spec.Q8_0) == 128


def test_group_counts_and_head_dim_checks():
    assert spec.n_groups(spec.HAD_INT4, 128) == 1
    assert spec.n_groups(spec.Q4_0, 128) == 4
    assert spec.n_groups(spec.Q6_0, 256) == 8
    assert spec.scale_bytes(spec.ASYM_G32, 128) == 16
    assert spec.n_groups(spec.Q8_0, 128) == 4
    assert spec.payload_bytes(spec.Q8_0, 128) == 128 and spec.scale_bytes(spec.Q8_0, 128) == 8
    with pytest.raises(ValueError):
        spec.payload_bytes(spec.Q4_0, 48)
    with pytest.raises(ValueError):
        spec.payload_bytes(spec.HAD_INT4, 96)       # not a power of two
    assert spec.payload_bytes(spec.Q4_0, 96) == 48
    assert math.isclose(spec.bytes_per_element(spec.HAD_INT4, 128), 0.53125)
