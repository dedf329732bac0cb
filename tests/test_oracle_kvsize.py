"""Pins for oracle.kvsize: the pages' printed KV-size and waste numbers (tests/golden)."""
import pytest

from oracle import kvsize
from tests.golden.load import load

KV = load("kv_size.txt")
WASTE = load("waste.txt")
MiB = 1 << 20


def test_llama31_8b_bytes_per_token():
    assert kvsize.kv_bytes_per_token(32, 8, 128, 2) == KV["llama31_8b_bytes_per_token"]
    assert KV["llama31_8b_bytes_per_token"] == 128 * 1024


@pytest.mark.parametrize("tokens,key", [(1024, "llama31_8b_ctx_1k"), (8192, "llama31_8b_ctx_8k"),
                                        (32768, "llama31_8b_ctx_32k"),
                                        (131072, "llama31_8b_ctx_128k")])
def test_context_table(tokens, key):
    assert tokens * kvsize.kv_bytes_per_token(32, 8, 128, 2) == KV[key]


def test_context_table_units():
    assert KV["llama31_8b_ctx_1k"] == 128 * MiB
    assert KV["llama31_8b_ctx_128k"] == 16 * 1024 * MiB


def test_gqa_factor():
    r = kvsize.kv_bytes_per_token(32, 32, 128, 2) / kvsize.kv_bytes_per_token(32, 8, 128, 2)
    assert r == KV["gqa_32_vs_8_ratio"]


def test_walkthrough_formula_is_mha_case():
    # d_model = n_head * d_head; with one KV head per query head the two formulas agree
    for B, S, L, nh, dh, p in [(1, 1, 1, 1, 1, 2), (3, 100, 40, 40, 128, 2), (64, 4096, 32, 32, 128, 1)]:
        assert kvsize.kv_bytes_total(B, S, L, nh * dh, p) == B * S * kvsize.kv_bytes_per_token(L, nh, dh, p)


def test_llama13b_upper_bound():
    # assumptions not on the page: 40 layers, d_model 5120, fp16, 2048 tokens
    b = kvsize.kv_bytes_total(1, 2048, 40, 5120, 2)
    assert b == 1_677_721_600
    assert b <= KV["llama13b_seq_upper_bound"]


def test_waste_figures():
    assert kvsize.naive_waste(100, 2048) == WASTE["naive_maxlen2048_S100"]
    assert kvsize.paged_waste(100, 16) == WASTE["paged_bs16_S100"]
    assert kvsize.paged_waste(32, 16) == WASTE["paged_bs16_S32"]
    assert kvsize.paged_waste(1, 16) == WASTE["paged_bs16_S1"]
    assert kvsize.naive_waste(1, 2048) == WASTE["naive_maxlen2048_S1"]


def test_paged_waste_bound():
    ws = [kvsize.paged_waste(s, 16) for s in range(1, 5000)]
    assert max(ws) == WASTE["paged_bs16_max"]
    assert min(ws) == 0
    assert all(kvsize.paged_waste(16 * k, 16) == 0 for k in range(1, 100))
