"""Pins of the oracle's KV-size closed forms against figures printed on the pages.

Fixtures: tests/golden/kv_sizes.json (each entry names its page and section).
"""
import json
import os

import numpy as np

from oracle import kv_bytes, bytes_per_block, blocks_in_pool, blocks_for_tokens

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_sizes.json")))
KIB, MIB, GIB = 1024, 1024 ** 2, 1024 ** 3


def test_per_token_llama3_8b():
    g = GOLD["per_token_llama3_8b"]
    b = kv_bytes(g["num_layers"], g["num_kv_heads"], g["head_size"], 1, g["elem_bytes"])
    assert b == g["bytes"]
    assert f"{b / KIB:.0f} KiB" in g["printed"]


def test_formula_is_linear_in_every_factor():
    # A dropped or squared factor anywhere in 2*L*H_kv*d_h*S*b breaks one of these.
    base = kv_bytes(3, 5, 7, 11, 2)
    assert base == 2 * 3 * 5 * 7 * 11 * 2
    assert kv_bytes(6, 5, 7, 11, 2) == 2 * base
    assert kv_bytes(3, 10, 7, 11, 2) == 2 * base
    assert kv_bytes(3, 5, 14, 11, 2) == 2 * base
    assert kv_bytes(3, 5, 7, 22, 2) == 2 * base
    assert kv_bytes(3, 5, 7, 11, 4) == 2 * base


def test_naive_reservation():
    g = GOLD["naive_reservation_40_requests"]
    per_tok = kv_bytes(32, 8, 128, 1, 2)
    reserved = g["num_requests"] * g["max_len"] * per_tok
    assert f"{reserved / GIB:5.2f}".strip() == g["gib_2dp"]


def test_conversation_2000_tokens():
    g = GOLD["conversation_2000_tokens"]
    assert kv_bytes(32, 8, 128, g["tokens"], 2) == g["mib"] * MIB


def test_worked_example_pool():
    g = GOLD["worked_example_60gib_pool"]
    blk = bytes_per_block(g["block_size"], 32, 8, 128, 2)
    assert blk == g["block_mib"] * MIB
    pool = blocks_in_pool(g["pool_gib"] * GIB, blk)
    assert pool == g["blocks"]
    assert blocks_for_tokens(g["short_request_tokens"], 16) == g["short_request_blocks"]
    assert pool // g["short_request_blocks"] == g["short_requests_fit"]
    assert blocks_for_tokens(g["reserved_tokens"], 16) == g["reserved_blocks"]
    assert pool // g["reserved_blocks"] == g["reserved_requests_fit"]
    assert blocks_for_tokens(g["long_chat_tokens"], 16) == g["long_chat_blocks"]
    assert pool // g["long_chat_blocks"] == g["long_chats_fit"]
    whole = g["shared_prompt_tokens"] // 16
    assert whole == g["shared_whole_blocks"] and whole * 16 == g["shared_whole_block_tokens"]
    own = g["long_chat_tokens"] - whole * 16
    assert own == g["own_tokens"]
    assert blocks_for_tokens(own, 16) == g["own_blocks"]
    assert (pool - whole) // g["own_blocks"] == g["chats_with_sharing_fit"]


def test_exercise_block_budget():
    g = GOLD["exercise_block_budget"]
    blk = bytes_per_block(g["block_size"], g["num_layers"], g["num_kv_heads"], g["head_size"],
                          g["elem_bytes"])
    blocks = blocks_in_pool(g["pool_gib"] * GIB, blk)
    assert blocks * g["block_size"] == g["token_slots"]


def test_startup_log_concurrency():
    g = GOLD["startup_log_concurrency"]
    assert f"{g['kv_tokens'] / g['tokens_per_request']:.2f}" == g["concurrency_2dp"]


def test_startup_sketch_blocks_computed():
    # llm-stack-book 7.3, "How many blocks exist?": 80 GiB GPU, utilisation 0.9,
    # 14 GiB weights, 4 GiB activations, 16-token blocks of the 8B shape in bf16.
    # The page prints no output for this sketch; the value is computed here.
    usable = int(80 * GIB * 0.90)
    kv_cache = usable - 14 * GIB - 4 * GIB
    blk = bytes_per_block(16, 32, 8, 128, 2)
    assert blocks_in_pool(kv_cache, blk) == 27648


def test_pool_nbytes_identity():
    # key_cache + value_cache of one layer equal kv_bytes(1, H_kv, d_h, NB*bs, b).
    NB, bs, Hkv, d = 37, 16, 2, 64
    kc = np.zeros((NB, bs, Hkv, d), np.uint16)
    vc = np.zeros_like(kc)
    assert kc.nbytes + vc.nbytes == kv_bytes(1, Hkv, d, NB * bs, 2)
