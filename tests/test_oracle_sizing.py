"""Pins for oracle.sizing: figures printed on the pages (tests/golden)."""

import json
import os

import pytest

from oracle import sizing

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


SIZES = _load("kv_sizes.json")
TABLES = _load("block_tables.json")


@pytest.mark.parametrize("key", [k for k in SIZES if "num_layers" in SIZES[k]])
def test_kv_bytes_closed_form(key):
    e = SIZES[key]
    got = sizing.kv_cache_bytes(e["num_layers"], e["num_kv_heads"], e["head_dim"],
                                e["seq_len"], e["batch"], e["dtype_bytes"])
    assert got == e["bytes"]
    if "bytes_at_1_byte" in e:
        got1 = sizing.kv_cache_bytes(e["num_layers"], e["num_kv_heads"],
                                     e["head_dim"], e["seq_len"], e["batch"], 1)
        assert got1 == e["bytes_at_1_byte"]


def test_7b_example_reads_4_gib():
    e = SIZES["llama2_7b_2048x4"]
    got = sizing.kv_cache_bytes(32, 32, 128, 2048, 4)
    assert got / 2 ** 30 == 4.0 and e["readable"] == "4.00 GiB"


def test_tensor_parallel_divides():
    full = sizing.kv_cache_bytes(32, 32, 128, 2048, 4)
    assert sizing.kv_cache_bytes(32, 32, 128, 2048, 4, tp_ways=8) * 8 == full


def test_score_matrix_figures():
    e = SIZES["score_matrix_8192"]
    assert 8192 * 8192 * 4 == e["bytes_per_head"]
    assert e["bytes_per_head"] * 32 == e["bytes_per_layer"]
    assert e["bytes_per_layer"] * 32 == e["bytes_total"]


def test_68_token_table():
    e = TABLES["table_68_tokens"]
    assert sizing.blocks_needed(e["num_tokens"], e["block_size"]) == e["blocks_needed"]
    ranges = sizing.block_ranges(e["num_tokens"], e["block_size"])
    assert [[a, b - 1] for a, b in ranges] == e["block_contents_first_last"]
    assert sizing.tokens_in_last_block(e["num_tokens"], e["block_size"]) == e["last_block_tokens"]


@pytest.mark.parametrize("key", ["dynamic_growth", "utilisation_example"])
def test_block_counts(key):
    e = TABLES[key]
    for n, blocks in e["tokens_to_blocks"].items():
        assert sizing.blocks_needed(int(n), e["block_size"]) == blocks
    for n, blocks in e.get("tokens_to_blocks_corrected", {}).items():
        assert sizing.blocks_needed(int(n), e["block_size"]) == blocks


def test_prealloc_utilisation_percentages():
    e = TABLES["utilisation_example"]
    for n, pct in e["prealloc_used_percent"].items():
        assert round(100 * int(n) / e["max_seq_len_prealloc"], 1 if pct < 10 else 0) == pct


def test_question8_partial_block():
    e = TABLES["question8_partial_block"]
    assert sizing.blocks_needed(e["num_tokens"], e["block_size"]) == e["blocks_needed"]
    assert sizing.tokens_in_last_block(e["num_tokens"], e["block_size"]) == e["last_block_tokens"]
