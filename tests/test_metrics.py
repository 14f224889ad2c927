"""Work counters used for throughput and roofline figures."""
import json
import os

from dynamic_block_sparse_head_amd import configs, metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pair_counts.json")


def test_dense_pair_counts_match_the_pages():
    for case in json.load(open(GOLDEN))["cases"]:
        assert metrics.dense_pairs(case["n"]) == case["pairs"], case["source"]
    assert metrics.dense_pairs(2000) == 4 * metrics.dense_pairs(1000)


def test_causal_pairs_and_selected_blocks():
    assert metrics.dense_pairs(4, causal=True) == 10
    c = configs.PREFILL_16K
    sel = metrics.prefill_selected_blocks(c.n_blocks, c.topk, c.n_local)
    # rows 0..23 hold i+1 blocks, the remaining 232 rows hold 24
    assert sel == sum(range(1, 25)) + (256 - 24) * 24 == 5868
    flops = metrics.prefill_effective_flops(c.Hq, c.D, c.block, sel)
    assert abs(flops - 3.94e11) / 3.94e11 < 1e-3


def test_decode_selected_bytes():
    c = configs.DECODE_128K
    assert c.topk == 102
    assert metrics.decode_selected_bytes(c.B, c.Hkv, c.topk, c.page, c.D) == 427_819_008
