"""Pins of the oracle prefix cache (oracle/prefix.py) to the pages and to invariants.

[TSS] "Sharing a prefix: one copy for many requests": chained block hashes,
only full blocks shared, a hit capped at the prompt minus one token, cached
blocks kept after free; "Measured: the same prompt, sixteen at a time": the
peak block counts and the computed-token count of the prefix-repetition run.

Citation keys ([HRL], [TSS], [VIBE], ...): the page titles listed in oracle/__init__.py.
"""

import hashlib
import json
import pathlib

import numpy as np
import pytest

from oracle import alloc, prefix

GOLDEN = pathlib.Path(__file__).parent / "golden"


def tokens(rng, n):
    return [int(t) for t in rng.integers(0, 1 << 17, size=n)]


# ---------------------------------------------------------------- the hash chain


def test_hash_is_sha256_of_parent_then_int32_le_ids():
    # the encoding reading, spelled out in bytes (ids 1, 2 and -1)
    want = hashlib.sha256(bytes(32) + bytes([1, 0, 0, 0, 2, 0, 0, 0, 255, 255, 255, 255])).digest()
    assert prefix.hash_block(prefix.ROOT, [1, 2, -1]) == want
    # FIPS 180-4 example value for "abc": the primitive is SHA-256
    assert hashlib.sha256(b"abc").hexdigest().startswith("ba7816bf")


def test_block_hash_names_the_whole_prefix():
    rng = np.random.default_rng(0)
    B = 16
    a = tokens(rng, 5 * B + 7)
    ha = prefix.block_hashes(a, B)
    assert len(ha) == 5  # the partial tail has no hash
    # same first 3 blocks, different 4th: first 3 hashes agree, the rest differ
    b = a[:3 * B] + tokens(rng, 2 * B)
    hb = prefix.block_hashes(b, B)
    assert hb[:3] == ha[:3] and hb[3] != ha[3] and hb[4] != ha[4]
    # one token changed in block 1 changes blocks 1.. even where block 4's own tokens are equal
    c = list(a)
    c[B + 3] ^= 1
    hc = prefix.block_hashes(c, B)
    assert hc[0] == ha[0] and all(hc[j] != ha[j] for j in range(1, 5))
    # the order of the ids inside a block matters
    d = list(a)
    d[0], d[1] = d[1], d[0]
    assert prefix.block_hashes(d, B)[0] != ha[0]
    # the same block after a different parent is a different block
    assert prefix.hash_block(ha[0], a[B:2 * B]) == ha[1]
    assert prefix.hash_block(prefix.ROOT, a[B:2 * B]) != ha[1]
    # chaining from a parent equals hashing the concatenation
    assert prefix.block_hashes(a[2 * B:], B, parent=ha[1]) == ha[2:]


# ---------------------------------------------------------------- the page's rules


def new_seq(pool, toks):
    s = prefix.CachedSequence()
    cached = prefix.allocate_prompt_cached(pool, s, toks)
    return s, cached


def test_second_request_with_same_prefix_points_at_the_same_blocks():
    rng = np.random.default_rng(1)
    pool = prefix.PrefixCachingPool(64, 16, reserve_null_block=True)
    shared = tokens(rng, 48)
    a, ca = new_seq(pool, shared + tokens(rng, 10))
    b, cb = new_seq(pool, shared + tokens(rng, 20))
    assert ca == 0 and cb == 48
    assert b.block_table[:3] == a.block_table[:3]
    assert all(pool.refcount[x] == 2 for x in a.block_table[:3])
    assert not set(b.block_table[3:]) & set(a.block_table)
    assert 0 not in a.block_table + b.block_table


def test_only_full_blocks_are_shared():
    rng = np.random.default_rng(2)
    pool = prefix.PrefixCachingPool(32, 16)
    p = tokens(rng, 20)
    a, _ = new_seq(pool, p)
    b, cb = new_seq(pool, p + tokens(rng, 5))
    assert cb == 16                      # the 4-token tail block of `a` is a's own
    assert b.block_table[1] != a.block_table[1]
    assert a.block_table[1] not in pool.hash_of


def test_full_hit_still_computes_one_token():
    rng = np.random.default_rng(3)
    pool = prefix.PrefixCachingPool(32, 16)
    p = tokens(rng, 32)
    a, _ = new_seq(pool, p)
    b, cb = new_seq(pool, p)             # the whole prompt is cached, yet
    assert cb == 16                      # the hit stops at prompt - 1 = 31: the last block is recomputed
    assert b.block_table[0] == a.block_table[0] and b.block_table[1] != a.block_table[1]
    assert a.block_table[1] in pool.hash_of and b.block_table[1] not in pool.hash_of  # the first copy stays cached
    c, cc = new_seq(pool, p + [7])       # one more token: both blocks hit
    assert cc == 32 and c.block_table[:2] == a.block_table[:2]
    d, cd = new_seq(pool, p[:1])         # a one-token prompt computes its token
    assert cd == 0


def test_blocks_stay_cached_after_free_until_reused():
    rng = np.random.default_rng(4)
    B = 16
    pool = prefix.PrefixCachingPool(10, B)
    p = tokens(rng, 3 * B + 5)
    a, _ = new_seq(pool, p)
    full = a.block_table[:3]
    tail = a.block_table[3]
    alloc.release_sequence(pool, a)
    # hashed blocks to the back, last block of the chain released first; the private tail to the front
    assert list(pool.free_queue)[0] == tail
    assert list(pool.free_queue)[-3:] == full[::-1]
    b, cb = new_seq(pool, p)
    assert cb == 3 * B and b.block_table[:3] == full
    alloc.release_sequence(pool, b)
    # memory pressure: a request that needs every block evicts them all
    c, cc = new_seq(pool, tokens(rng, 10 * B))
    assert cc == 0 and not set(prefix.block_hashes(p, B)) & set(pool.cached)
    alloc.release_sequence(pool, c)
    d, cd = new_seq(pool, p)
    assert cd == 0


def test_eviction_takes_the_chain_from_its_end():
    rng = np.random.default_rng(5)
    B = 16
    pool = prefix.PrefixCachingPool(8, B)
    p = tokens(rng, 4 * B + 1)               # 4 full blocks + a 1-token tail
    a, _ = new_seq(pool, p)
    alloc.release_sequence(pool, a)
    x, _ = new_seq(pool, tokens(rng, 4 * B + 1))  # the tail block, 3 never-used blocks, then one cached block
    hp = prefix.block_hashes(p, B)
    assert [h in pool.cached for h in hp] == [True, True, True, False]  # the chain's last block went first
    alloc.release_sequence(pool, x)
    b, cb = new_seq(pool, p)
    assert cb == 3 * B


def test_write_into_a_cached_block_evicts_it_and_committed_tokens_are_fixed():
    rng = np.random.default_rng(6)
    B = 16
    pool = prefix.PrefixCachingPool(16, B)
    a, _ = new_seq(pool, tokens(rng, 20))
    child = prefix.fork_cached(pool, a)
    assert child.tokens == a.tokens and child.num_tokens == 20
    with pytest.raises(ValueError):
        prefix.prepare_write_cached(pool, child, 19)   # committed position
    # the parent fills the shared tail block: copy-on-write, then the copy gets the hash
    for pos in range(20, 32):
        prefix.prepare_write_cached(pool, a, pos)
    prefix.commit_tokens(pool, a, tokens(rng, 12))
    assert a.block_table[1] != child.block_table[1] and a.block_table[1] in pool.hash_of
    with pytest.raises(ValueError):
        prefix.commit_tokens(pool, a, [1])              # past the written positions


def test_out_of_blocks_changes_nothing():
    rng = np.random.default_rng(7)
    pool = prefix.PrefixCachingPool(5, 16)
    p = tokens(rng, 40)
    a, _ = new_seq(pool, p)
    alloc.release_sequence(pool, a)
    b, _ = new_seq(pool, tokens(rng, 16))        # holds one block
    queue, cached, refs = list(pool.free_queue), dict(pool.cached), list(pool.refcount)
    s = prefix.CachedSequence()
    with pytest.raises(alloc.OutOfBlocks):
        prefix.allocate_prompt_cached(pool, s, p + tokens(rng, 40))  # 2 idle hits + 3 fresh > 4 free
    assert list(pool.free_queue) == queue and pool.cached == cached and pool.refcount == refs
    assert s.block_table == [] and s.num_tokens == 0


# ---------------------------------------------------------------- the page's measured run


def replay_prefix_repetition(g, num_prefixes, seed=0):
    """64 prompts of prefix + suffix, 16 at a time, each answering output_len tokens.

    The 16 requests in flight advance together, so they are admitted, decode
    and finish in waves.  Returns (peak blocks in use, prompt tokens, tokens
    computed, i.e. not found in the cache).
    """
    rng = np.random.default_rng(seed)
    B = g["block_size"]
    pool = prefix.PrefixCachingPool(g["cache_blocks"], B, reserve_null_block=True)
    prefixes = [tokens(rng, g["prefix_len"]) for _ in range(num_prefixes)]
    peak = total = missed = 0
    for wave in range(g["num_prompts"] // g["max_concurrency"]):
        running = []
        for i in range(g["max_concurrency"]):
            r = wave * g["max_concurrency"] + i
            p = prefixes[r % num_prefixes] + tokens(rng, g["suffix_len"])
            s = prefix.CachedSequence()
            cached = prefix.allocate_prompt_cached(pool, s, p)
            total += len(p)
            missed += len(p) - cached
            running.append(s)
        peak = max(peak, pool.num_in_use)
        for _ in range(g["output_len"]):
            for s in running:
                prefix.prepare_write_cached(pool, s, s.num_tokens)
                prefix.commit_tokens(pool, s, tokens(rng, 1))
            peak = max(peak, pool.num_in_use)
        for s in running:
            alloc.release_sequence(pool, s)
    return peak, total, missed


def test_measured_run_one_prefix():
    g = json.loads((GOLDEN / "tss_prefix_caching.json").read_text())
    peak, total, missed = replay_prefix_repetition(g, 1)
    assert peak == g["one_prefix"]["peak_blocks"] == 426
    assert round(100 * peak / g["cache_blocks"], 1) == g["one_prefix"]["peak_percent"]
    assert total == g["num_prompts"] * (g["prefix_len"] + g["suffix_len"])
    assert abs(total - g["printed_prompt_tokens"]) < 10
    # one copy of the prefix plus the private suffixes
    assert missed == g["prefix_len"] + g["num_prompts"] * g["suffix_len"]
    assert abs(missed - g["printed_miss_tokens"]) < 25


def test_measured_run_distinct_prefixes_behave_like_no_caching():
    g = json.loads((GOLDEN / "tss_prefix_caching.json").read_text())
    peak, total, missed = replay_prefix_repetition(g, g["distinct_prefixes"]["num_prefixes"])
    assert peak == g["distinct_prefixes"]["peak_blocks"] == g["max_concurrency"] * 261
    assert round(100 * peak / g["cache_blocks"], 1) == g["distinct_prefixes"]["peak_percent"]
    assert missed == total
