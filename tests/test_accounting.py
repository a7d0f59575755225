"""Host-side accounting against the numbers the pages print (golden file)."""
import json
import os

import pytest

from kv_cache_eviction_lse_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_kv_cache_bytes_pages():
    g = _golden()["kv_cache_bytes"]
    a, b = g
    assert acc.kv_cache_bytes(a["layers"], a["tokens"], a["kv_heads"], a["head_dim"], a["bytes_per_elem"]) == a["bytes"]
    nb = acc.kv_cache_bytes(b["layers"], b["tokens"], b["kv_heads"], b["head_dim"], b["bytes_per_elem"])
    assert nb == 335_544_320_000 and nb // 10**9 == b["bytes_rounded_gb"]  # printed truncated
    # the page's "23GiB" label is a unit slip: 23.59e9 B is 21.97 GiB
    assert abs(a["bytes"] / 2**30 - 21.97) < 0.01


def test_compression_factor_table():
    for row in _golden()["compression_ratio_to_factor"]["rows"]:
        f = acc.compression_factor(row["ratio"])
        assert int(f * 10) / 10 == row["factor_printed"]


def test_pair_counts_small_cases():
    # repeat: 3 queries in chunks of 2 -> self pairs 1+2 + 1 = 4, ctx 3*5
    assert acc.lse_pairs(1, 5, 3, "repeat", 2) == 15 + 4
    assert acc.lse_pairs(2, 7, 7, "causal") == 2 * 28
    assert acc.sum_pairs(1, 5, 2) == 3 + 2 + 1
    assert acc.sum_pairs(1, 5, 9) == 0
    assert acc.max_pairs(3, 4, 5) == 60


def test_evict_bytes_qwen25_14b_120k():
    # 8 KV heads, 120000 keys, top 25% (30000) + 128 window kept per head
    kept = 8 * (30000 + 128)
    assert acc.evict_bytes(8, 120000, kept, 128) == 251_612_672
    assert kept * 128 * 2 * 2 == 123_404_288
