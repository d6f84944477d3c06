"""Pins of the oracle's cache accounting and model constants against the pages.

Fixtures under tests/golden/ hold the numbers as the pages print them:
kv_ledger_page1.json ("256K 长上下文真能本地用", §二), model_config_page1.json
(same page, §一) and mla_fields_page5.json ("mHC+MLA+MTP 是什么", MLA section).
"""
import json
import math
import os

import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _round1_half_up(x):
    return math.floor(x * 10 + 0.5) / 10


def test_per_token_bytes_latent_plus_v_convention():
    g = _load("kv_ledger_page1.json")
    elems = O.cache_elems_per_token("latent+v")
    assert elems == g["elems_latent"] + g["elems_v"] == g["elems_per_token_per_layer"]
    assert O.mla_cache_bytes(1, "latent+v", layers=1) == g["bytes_per_token_per_layer"]
    assert O.mla_cache_bytes(1, "latent+v") == g["bytes_per_token_all_layers"]
    assert O.mla_cache_bytes(1, "latent+v") / 1024 == g["kib_per_token_all_layers"]


def test_mla_column_of_the_ledger_table():
    # MLA column: tokens = k * 1024, GiB, one decimal, half up.
    g = _load("kv_ledger_page1.json")
    for row in g["table"]:
        tokens = row["tokens_k"] * 1024
        gib = O.mla_cache_bytes(tokens, "latent+v") / 2 ** 30
        assert _round1_half_up(gib) == row["mla_gb"], row


def test_mha_column_of_the_ledger_table_and_its_garble():
    # The MHA rows 4K..128K only reproduce with K = 1000 tokens; the 256K row
    # uses K = 1024.  Both readings of the printed formula are asserted.
    g = _load("kv_ledger_page1.json")
    f = g["mha_formula"]
    per_token = f["kv_heads"] * f["qk_dim"] * f["k_and_v"] * f["layers"] * f["bytes"]
    assert O.mha_cache_bytes(1) == per_token == 983040
    assert f["qk_dim"] == f["qk_nope_head_dim"] + f["qk_rope_head_dim"]
    for row in g["table"]:
        k = 1024 if row["tokens_k"] == 256 else 1000
        gib = O.mha_cache_bytes(row["tokens_k"] * k) / 2 ** 30
        printed = row["mha_gb"]
        got = round(gib) if printed >= 100 else _round1_half_up(gib)
        assert got == printed, (row, gib)
    # with K = 1024 the 4K row would print 3.8, not the page's 3.7
    assert _round1_half_up(O.mha_cache_bytes(4096) / 2 ** 30) == 3.8


def test_compression_about_19x():
    g = _load("kv_ledger_page1.json")
    ratio = O.mha_cache_bytes(262144) / O.mla_cache_bytes(262144, "latent+v")
    assert ratio == pytest.approx(19.2)
    assert round(ratio) == g["compression_about"]


def test_cache_row_conventions_of_the_mla_page():
    g = _load("mla_fields_page5.json")
    assert O.cache_elems_per_token("latent+rope") == g["kv_lora_rank"] + g["qk_rope_head_dim"] == 576
    assert O.cache_elems_per_token("latent+per-head-rope") == 512 + 32 * 64
    # the 576-element row used by the cache: 1152 B/token/layer, 45 KiB over 40 layers
    assert O.mla_cache_bytes(1, layers=1) == 1152
    assert O.mla_cache_bytes(1) == 46080 == 45 * 1024
    assert O.mla_cache_bytes(262144) == 12_079_595_520
    assert O.mla_cache_bytes(262144) / 2 ** 30 == 11.25
    assert O.mla_cache_bytes(32768) == 1_509_949_440


def test_model_constants_match_the_printed_config():
    c = _load("model_config_page1.json")
    f = _load("mla_fields_page5.json")
    assert O.MAX_POSITIONS == c["max_position_embeddings"]
    assert O.MAX_POSITIONS == c["rope_scaling"]["original_max_position_embeddings"] * c["rope_scaling"]["factor"]
    for k, v in c["rope_scaling"].items():
        assert O.ROPE_SCALING[k] == v, k
    assert O.KV_LORA_RANK == c["kv_lora_rank"] == f["kv_lora_rank"]
    assert O.V_HEAD_DIM == c["v_head_dim"] == f["v_head_dim"]
    assert O.NUM_LAYERS == c["num_hidden_layers"]
    assert O.NUM_HEADS == c["num_attention_heads"] == c["num_key_value_heads"]
    assert O.QK_NOPE_HEAD_DIM == f["qk_nope_head_dim"]
    assert O.QK_ROPE_HEAD_DIM == f["qk_rope_head_dim"]
    assert c["attention_bias"] is False
