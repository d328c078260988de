"""Pins for the oracle's memory arithmetic against the numbers printed on the pages (CPU only)."""
import json
import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GIB = 1 << 30


def test_kv_memory_worked_example():
    """Textbook 10.4.1: L=32, B=1, Hkv=8, S=32768, dh=128 -> 4 GiB fp16/bf16,
    about 2 GiB INT8/FP8, about 0.5 GiB ideal 2-bit."""
    gold = json.load(open(os.path.join(GOLDEN, "kv_memory_worked_example.json")))
    s = gold["shape"]
    for key, gib in gold["payload_gib"].items():
        bits = gold["bits_per_element"][key]
        got = oracle.kv_cache_bytes(s["L"], s["B"], s["Hkv"], s["S"], s["dh"], bits)
        assert got == gib * GIB, key


def test_kv_memory_uses_kv_heads_not_query_heads():
    """Textbook 10.4.1: under GQA the cache scales with Hkv; using the 32 query
    heads of the same model would overstate it four-fold."""
    kv = oracle.kv_cache_bytes(32, 1, 8, 32768, 128, 8)
    wrong = oracle.kv_cache_bytes(32, 1, 32, 32768, 128, 8)
    assert wrong == 4 * kv and kv == 2 * GIB


def test_fp8_halves_the_cache():
    """Guide, introduction: FP8 roughly halves the KV cache against bf16/fp16."""
    for shape in [(1, 1, 1, 1, 1), (32, 32, 8, 4352, 128), (80, 4, 8, 131072, 128)]:
        assert 2 * oracle.kv_cache_bytes(*shape, 8) == oracle.kv_cache_bytes(*shape, 16)


def test_per_token_head_metadata_ratio():
    """Textbook 10.4.3: dh=128 with one fp16 scale each for K and V per
    (token, head): fp16 payload 512 B, INT8 payload 256 B, scales 4 B, ratio 512/260 ~ 1.97."""
    gold = json.load(open(os.path.join(GOLDEN, "per_token_head_metadata.json")))
    dh = gold["dh"]
    hi = oracle.token_head_bytes(dh, 16, 0)
    lo = oracle.token_head_bytes(dh, 8, 2)
    assert hi == gold["fp16_payload_bytes"]
    assert oracle.token_head_bytes(dh, 8, 0) == gold["int8_payload_bytes"]
    assert lo - gold["int8_payload_bytes"] == gold["scale_bytes_total"]
    assert hi / lo == pytest.approx(512 / 260, rel=0, abs=1e-15)
    assert round(hi / lo, 2) == gold["ratio_printed"]
