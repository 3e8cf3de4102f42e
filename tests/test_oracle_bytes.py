"""Oracle byte accounting against the byte figures the pages print."""

import json
import os

import pytest

from oracle import cache_bytes as cb

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "byte_examples.json")))
UNIT = {"GB": 1e9, "MB": 1e6, "GiB": 2.0 ** 30, "MiB": 2.0 ** 20}


def _label_matches(value, printed, unit):
    # the page rounds to the digits it prints: compare at that resolution
    digits = len(str(printed).split(".")[1]) if "." in str(printed) else 0
    return round(value / UNIT[unit], digits) == printed


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: c["name"])
def test_printed_cache_bytes(case):
    got = cb.kv_cache_bytes(**case["args"])
    if case["exact"] is not None:
        assert got == case["exact"]
    assert _label_matches(got, case["printed"], case["unit"]), (got, case["printed"], case["unit"])


@pytest.mark.parametrize("case", GOLDEN["per_token"], ids=lambda c: c["name"])
def test_printed_per_token_bytes(case):
    got = cb.kv_bytes_per_token(**case["args"])
    assert got == case["exact"]
    assert _label_matches(got, case["printed"], case["unit"])


def test_reference_table_ratios():
    """Only the ratios of the DantinoX table are consistent with its formula."""
    t = GOLDEN["table_ratios"]
    base = cb.kv_cache_bytes(12, 8, 32, 512, 1, 2)
    for hkv, mb in t["kv_mb_512"].items():
        want = mb / t["kv_mb_512"]["8"]
        got = cb.kv_cache_bytes(12, int(hkv), 32, 512, 1, 2) / base
        assert abs(got - want) <= t["rel_tol"] * want + 0.003
    for ctx, mb in t["mha_by_ctx"].items():
        want = mb / t["mha_by_ctx"]["512"]
        got = cb.kv_cache_bytes(12, 8, 32, int(ctx), 1, 2) / base
        assert abs(got - want) <= t["rel_tol"] * want


def test_long_context_cache_equals_llama2_example():
    """80 layers x 8 KV heads x 128 x 32768 tokens in bf16 is the same integer as
    the Llama-2-70B example (64 heads x 4096 tokens), since 64*4096 = 8*32768."""
    assert cb.kv_cache_bytes(80, 8, 128, 32768, 1, 2) == 10737418240


def test_payload_and_growth_consistent():
    """Lesson record: M_KV(T) = T * per-token growth per sequence, times B."""
    for (B, L, T, Hkv, Dh, s) in [(1, 2, 3, 4, 5, 2), (8, 32, 4096, 8, 128, 2), (3, 12, 205, 8, 32, 4)]:
        assert cb.kv_cache_bytes(L, Hkv, Dh, T, B, s) == B * T * cb.kv_bytes_per_token(L, Hkv, Dh, s)


def test_mla_formula_special_cases():
    """Latent cache: one tensor of width d_c. A latent as wide as 2*H_kv*d_h holds
    exactly the K+V bytes; the decoupled rotary key adds d_R per row."""
    assert cb.mla_cache_bytes(32, 2 * 8 * 128, 4096, 16, 2) == cb.kv_cache_bytes(32, 8, 128, 4096, 16, 2)
    assert cb.mla_cache_bytes(1, 512, 4096, 32, 2, rope_dim=64) == 1 * 576 * 4096 * 32 * 2
    assert cb.mla_cache_bytes(1, 512, 4096, 32, 2, rope_dim=64) == 150994944


def test_quantised_widths():
    """Section 4.4 of the textbook page: p = 1 (int8) halves, p = 0.5 (int4) quarters the fp16 bytes."""
    fp16 = cb.kv_cache_bytes(80, 8, 128, 8192, 32, 2)
    assert cb.kv_cache_bytes(80, 8, 128, 8192, 32, 1) * 2 == fp16
    assert cb.kv_cache_bytes(80, 8, 128, 8192, 32, 0.5) * 4 == fp16


def test_logical_bytes():
    assert cb.logical_kv_bytes(12, 8, 32, [205], 4) == 5038080
    assert cb.logical_kv_bytes(1, 2, 4, [0, 3, 5], 2) == 2 * 1 * 2 * 4 * 8 * 2
