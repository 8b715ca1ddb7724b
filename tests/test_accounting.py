"""The accounting helpers reproduce the figures the P3 page prints (tests/golden/accounting.json)."""
import json
import math
import os

from prefill_slot_mapping_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accounting.json")))


def test_kv_bytes_per_token_matches_the_page():
    for row in GOLD["kv_bytes_per_token"]:
        assert acc.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"],
                                      row["elem_bytes"], row["tp"]) == row["bytes"], row["cite"]


def test_decode_kv_time_model_matches_the_page():
    g = GOLD["kv_ms_model"]
    for row, dec in zip(g["rows"], g["decimals"]):
        ms = acc.kv_read_time_ms(row["batch"], row["ctx"], g["bytes_per_token"],
                                 g["hbm_bytes_per_s"])
        assert round(ms, dec) == row["ms"]
        # the same bytes through decode_kv_bytes (per layer x 36 layers / tp 4)
        per_layer = acc.decode_kv_bytes([row["ctx"]] * row["batch"], 2, 128, 2)
        assert per_layer * 36 == row["batch"] * row["ctx"] * g["bytes_per_token"]


def test_padded_transient_matches_the_page():
    g = GOLD["padded_decode_transient"]
    b = acc.decode_kv_bytes([g["tokens"]] * g["seqs"], g["kv_heads"], g["head_dim"],
                            g["elem_bytes"])
    assert round(b / 2 ** 30, 2) == g["gib"]


def test_tp4_pool_token_count():
    g = GOLD["tp4_pool_tokens"]
    tokens = g["gib"] * 2 ** 30 / g["bytes_per_token"]
    assert str(int(tokens)).startswith(str(g["tokens_prefix"]))


def test_pool_guard_example():
    g = GOLD["pool_guard"]
    cached = g["prompt"] + g["new_tokens"] - 1          # the last sampled token is never fed back
    assert cached == g["cached_tokens"]
    assert math.ceil(cached / g["block_size"]) == g["blocks"]


def test_visible_pairs_and_flops():
    # a 3-row chunk on a 2-token prior: rows see 3, 4, 5 keys
    assert acc.visible_pairs(5, 3) == 12
    assert acc.visible_pairs(7, 1) == 7
    assert acc.attention_flops([5, 7], [3, 1], 2, 4) == 4 * 4 * 2 * 19
    assert acc.append_bytes(10, 8, 128, 2) == 4 * 10 * 8 * 128 * 2
