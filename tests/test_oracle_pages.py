"""Pins of the oracle's bookkeeping and address translation to numbers the pages print.

Each fixture under tests/golden/ names the page and section it comes from.

Citation keys ([HRL], [TSS], [VIBE], ...): the page titles listed in oracle/__init__.py.
"""

import json
import os

import pytest

from oracle import accounting as acc
from oracle import alloc
from oracle import paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example (ainew)


def test_worked_example_accounting():
    g = load("ainew_worked_example.json")
    B = g["block_size"]
    assert [acc.blocks_needed(n, B) for n in g["lengths"]] == g["blocks_per_request"]
    assert [acc.blocks_needed(n, B) * B - n for n in g["lengths"]] == g["padding_per_request"]
    assert acc.slots_paged(g["lengths"], B) == g["slots_used"]
    assert sum(g["lengths"]) == g["tokens"]
    assert acc.waste_paged(g["lengths"], B) == g["waste_slots"]
    assert acc.slots_contiguous(len(g["lengths"]), g["max_context"]) == g["contiguous_slots"]
    assert g["contiguous_slots"] // g["slots_used"] == g["contiguous_to_paged_ratio"]
    waste_pct = 100.0 * acc.waste_contiguous(g["lengths"], g["max_context"]) / g["contiguous_slots"]
    assert round(waste_pct, 1) == g["contiguous_waste_percent"]
    assert acc.blocks_needed(g["single_request_tokens"], B) == g["single_request_blocks"]
    assert acc.slots_paged([g["single_request_tokens"]], B) == g["single_request_slots"]


def test_worked_example_allocation_and_growth():
    g = load("ainew_worked_example.json")
    B = g["block_size"]
    order = g["free_order"] + [b for b in range(g["pool_blocks"]) if b not in g["free_order"]]
    pool = alloc.BlockPool(g["pool_blocks"], B, free_order=order)
    seqs = []
    for n in g["lengths"]:
        s = alloc.Sequence()
        alloc.allocate_prompt(pool, s, n)
        seqs.append(s)
    assert [s.block_table for s in seqs] == g["tables"]
    assert pool.num_free == g["free_after"]
    # request B keeps decoding; its 49th token (index 48) is the first to need a 4th block
    r = seqs[g["growth_request"]]
    for t in range(g["lengths"][g["growth_request"]], 48):
        assert alloc.ensure_capacity(pool, r, t) == []
    assert alloc.ensure_capacity(pool, r, 48) == [11]
    assert r.block_table == g["growth_table"]


def test_block_size_tradeoff():
    g = load("ainew_block_sizes.json")
    for c in g["cases"]:
        B = c["block_size"]
        assert acc.table_lookups(g["tokens"], B) == c["lookups"]
        assert acc.waste_paged([g["tokens"]], B) == c["wasted_slots"]
        if "wasted_percent_of_block" in c:
            # 17 of 64 slots is 26.6 %; the page prints the truncated percentage
            assert int(100 * c["wasted_slots"] / B) == c["wasted_percent_of_block"]


def test_waste_bound_per_request():
    # waste never exceeds block_size - 1 for any length ([HRL] section 7)
    for B in (1, 4, 16, 32, 64):
        for n in range(0, 300):
            w = acc.waste_paged([n], B)
            assert 0 <= w <= B - 1


# ---------------------------------------------------------------- copy-on-write (ainew)


def test_cow_clones_only_the_written_block():
    g = load("ainew_cow.json")
    B = g["block_size"]
    pool = alloc.BlockPool(g["pool_blocks"], B)
    a = alloc.Sequence()
    alloc.allocate_prompt(pool, a, g["prompt_tokens"])
    assert a.block_table == g["shared_table"]
    b = alloc.fork(pool, a)
    # B generates its next token, which lands in the block it still shares with A
    slot, cow = alloc.prepare_write(pool, b, g["prompt_tokens"])
    assert list(cow) == g["cow_pair"]
    assert a.block_table == g["table_a_after"]
    assert b.block_table == g["table_b_after"]
    assert {str(k): pool.refcount[k] for k in (0, 1, 2)} == g["refcounts_after"]
    assert slot == g["cow_pair"][1] * B + g["prompt_tokens"] % B
    # A now writes into its own block in place: no copy
    slot_a, cow_a = alloc.prepare_write(pool, a, g["prompt_tokens"])
    assert cow_a is None and slot_a == 1 * B + g["prompt_tokens"] % B


def test_cow_last_holder_writes_in_place():
    pool = alloc.BlockPool(8, 4)
    a = alloc.Sequence()
    alloc.allocate_prompt(pool, a, 6)
    b = alloc.fork(pool, a)
    c = alloc.fork(pool, a)
    assert pool.refcount[1] == 3
    _, cow_b = alloc.prepare_write(pool, b, 6)
    _, cow_c = alloc.prepare_write(pool, c, 6)
    _, cow_a = alloc.prepare_write(pool, a, 6)
    assert cow_b == (1, 2) and cow_c == (1, 3) and cow_a is None
    assert pool.refcount[1] == 1 and pool.refcount[0] == 3


# ---------------------------------------------------------------- walkthrough (hrl)


def test_hrl_walkthrough_growth_and_release():
    g = load("hrl_walkthrough.json")["walkthrough"]
    B = g["block_size"]
    pool = alloc.BlockPool(17, B, free_order=g["free_blocks"])
    r = alloc.Sequence()
    for t in range(g["prompt_tokens"]):
        alloc.ensure_capacity(pool, r, t)
    assert acc.blocks_needed(g["prompt_tokens"], B) == g["prompt_blocks"]
    assert r.block_table == g["table_after_prefill"]
    for t in (6, 7):
        alloc.ensure_capacity(pool, r, t)
    assert r.block_table == g["table_after_tokens_6_and_7"]
    alloc.ensure_capacity(pool, r, 8)
    assert r.block_table == g["table_after_token_8"]
    free_before = set(pool.free_queue)
    alloc.release_sequence(pool, r)
    assert set(pool.free_queue) - free_before == set(g["released_on_finish"])


def test_hrl_translation():
    g = load("hrl_walkthrough.json")["section5"]
    B = g["block_size"]
    assert acc.blocks_needed(g["tokens"], B) == g["blocks"]
    assert paged.logical_block_and_offset(g["lookup_token"], B)[0] == g["lookup_logical_block"]
    assert paged.translate(g["table"], g["lookup_token"], B)[0] == g["lookup_physical_block"]
    for j, (lo, hi) in enumerate(g["logical_block_token_ranges"]):
        for t in range(lo, hi + 1):
            assert paged.logical_block_and_offset(t, B) == (j, t - lo)
    # every token of a 3-entry table resolves into the listed physical blocks in order
    t4 = load("hrl_walkthrough.json")["section4"]["table"]
    seen = [paged.translate(t4, t, 4)[0] for t in range(12)]
    assert seen == [17] * 4 + [3] * 4 + [91] * 4


def test_hrl_pseudocode_round_trip():
    # write_kv / read_kv of the section-17 pseudocode, on the oracle's pool bookkeeping
    g = load("hrl_walkthrough.json")["walkthrough"]
    pool = alloc.BlockPool(17, g["block_size"], free_order=g["free_blocks"])
    r = alloc.Sequence()
    store = {}
    for t in range(9):
        slot, cow = alloc.prepare_write(pool, r, t)
        assert cow is None
        store[slot] = t
    for t in range(9):
        assert store[paged.slot_id(r.block_table, t, g["block_size"])] == t
    assert r.block_table == g["table_after_token_8"]


def test_hrl_last_block_and_static_reservation():
    g = load("hrl_walkthrough.json")
    s7 = g["section7"]
    B = s7["block_size"]
    assert acc.blocks_needed(s7["tokens"], B) == s7["blocks"]
    assert (s7["blocks"] - 1) * B == s7["tokens_in_full_blocks"]
    assert s7["tokens"] - s7["tokens_in_full_blocks"] == s7["last_block_used"]
    assert acc.waste_paged([s7["tokens"]], B) == s7["last_block_empty"]
    assert max(acc.waste_paged([n], B) for n in range(1, 5000)) == s7["max_waste_per_request"]
    s13 = g["section13"]
    n = s13["requests"]
    assert acc.slots_contiguous(n, s13["max_tokens"]) == s13["static_reserved"]
    assert n * s13["avg_tokens"] == s13["used"]
    assert acc.blocks_needed(s13["avg_tokens"], s13["block_size"]) == s13["blocks_per_request"]
    assert acc.slots_paged([s13["avg_tokens"]], s13["block_size"]) == s13["slots_per_request"]
    assert acc.slots_paged([s13["avg_tokens"]] * n, s13["block_size"]) == s13["paged_reserved"]


# ---------------------------------------------------------------- vibe / tss numbers


def test_vibe_numbers():
    g = load("vibe_numbers.json")
    r = g["short_request"]
    w = acc.waste_contiguous([r["tokens"]], r["max_len"])
    assert w == r["contiguous_waste"]
    assert round(100 * w / r["max_len"]) == r["contiguous_waste_percent"]
    assert acc.waste_paged([r["tokens"]], r["block_size"]) == r["paged_waste"]
    o = g["opt13b"]
    # per-token KV of a model whose K/V rows are the full hidden size (no GQA)
    per_token = acc.kv_cache_bytes(1, 1, o["layers"], 1, o["hidden"], o["bytes_per_elem"])
    assert per_token / 1024 == o["bytes_per_token_kb"]
    seq = acc.kv_cache_bytes(1, o["sequence_tokens"], o["layers"], 1, o["hidden"], o["bytes_per_elem"])
    assert round(seq / 1e9, 1) == pytest.approx(o["sequence_gb"], abs=0.1)


def test_tss_capacity_and_sharing():
    g = load("tss_numbers.json")
    B = g["block_size"]
    assert g["cache_tokens"] // B == g["cache_blocks"] and g["cache_tokens"] % B == 0
    assert round(g["cache_tokens"] / g["max_len"], 2) == g["max_concurrency"]
    m = g["qwen3_8b"]
    assert acc.kv_cache_bytes(1, 1, m["layers"], m["kv_heads"], m["head_dim"], m["bytes_per_elem"]) == \
        g["kv_bytes_per_token"] == 144 * 1024
    assert g["prompt_tokens"] + g["answer_tokens"] == g["request_tokens"]
    assert acc.blocks_needed(g["request_tokens"], B) == g["blocks_per_request"]
    n = g["requests_in_flight"]
    assert round(100 * n * g["blocks_per_request"] / g["cache_blocks"], 1) == g["unshared_percent"]
    # sharing modelled with the oracle's pool: one prefix, sixteen forks, private tails
    pool = alloc.BlockPool(g["cache_blocks"], B, reserve_null_block=True)
    prefix = alloc.Sequence()
    alloc.allocate_prompt(pool, prefix, g["shared_prefix_tokens"])
    assert len(prefix.block_table) == g["shared_prefix_blocks"]
    reqs = []
    for _ in range(n):
        r = alloc.fork(pool, prefix)
        for t in range(g["shared_prefix_tokens"], g["request_tokens"]):
            _, cow = alloc.prepare_write(pool, r, t)
            assert cow is None  # the prefix is whole blocks: nothing shared is written
        reqs.append(r)
    alloc.release_sequence(pool, prefix, reusable=True)  # requests keep the prefix alive
    assert all(len(r.block_table) - g["shared_prefix_blocks"] == g["private_blocks_per_request"] for r in reqs)
    assert pool.num_in_use == g["shared_total_blocks"]
    assert round(100 * pool.num_in_use / g["cache_blocks"], 1) == g["shared_percent"]


def test_tss_finding_a_token():
    # token 53 with 16-token blocks: logical block 3, offset 5, and the slot is the physical
    # block times the block size plus the offset, through whatever the table holds there
    g = load("tss_numbers.json")["finding_a_token"]
    B, t = g["block_size"], g["token"]
    assert paged.logical_block_and_offset(t, B) == (g["logical_block"], g["offset"])
    table = [40, 7, 1234, 88, 3]
    assert paged.translate(table, t, B) == (88, g["offset"])
    assert paged.slot_id(table, t, B) == 88 * B + g["offset"] == 1413
    assert paged.slot_mapping_ref([table], [0], [t], B).tolist() == [1413]


# ---------------------------------------------------------------- pool bookkeeping


def test_null_block_is_never_allocated_and_free_ordering():
    pool = alloc.BlockPool(6, 4, reserve_null_block=True)
    got = [pool.allocate() for _ in range(5)]
    assert 0 not in got and sorted(got) == [1, 2, 3, 4, 5]
    with pytest.raises(alloc.OutOfBlocks):
        pool.allocate()
    pool.release(3, reusable=True)   # back of the queue
    pool.release(4, reusable=False)  # front of the queue
    assert list(pool.free_queue) == [4, 3]
    assert pool.allocate() == 4


def test_out_of_blocks_keeps_state_consistent():
    pool = alloc.BlockPool(4, 16)
    s = alloc.Sequence()
    alloc.allocate_prompt(pool, s, 64)
    with pytest.raises(alloc.OutOfBlocks):
        alloc.ensure_capacity(pool, s, 64)
    assert s.block_table == [0, 1, 2, 3] and pool.num_free == 0 and pool.refcount == [1, 1, 1, 1]


def test_slot_mapping_ref_matches_translation():
    tables = [[3, 7], [0, 5, 9], [4]]
    seq_ids = [0, 0, 1, 1, 2, 1]
    pos = [0, 24, 46, 16, 11, -1]
    slots = paged.slot_mapping_ref(tables, seq_ids, pos, 16)
    assert slots.tolist() == [48, 7 * 16 + 8, 9 * 16 + 14, 5 * 16 + 0, 4 * 16 + 11, -1]
    with pytest.raises(IndexError):
        paged.slot_mapping_ref(tables, [2], [16], 16)
