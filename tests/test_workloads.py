"""Structure of the seeded workloads, checked with the oracle's own bookkeeping."""

import numpy as np
import pytest

from oracle import accounting as acc
from oracle import alloc
from oracle import paged
from workloads import make_config


def live_blocks(w, step=0):
    B = w.block_size
    out = []
    for s in range(w.num_seqs):
        n = acc.blocks_needed(int(w.steps[step].context_lens[s]), B)
        out.append([int(b) for b in w.block_tables[s, :n]])
    return out


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_small_workloads_are_valid(k):
    w = make_config(k, small=True)
    B = w.block_size
    last = len(w.steps) - 1
    rows = live_blocks(w, last)
    flat = [b for r in rows for b in r]
    assert all(0 <= b < w.num_blocks for b in flat)
    if w.null_block is not None:
        assert w.null_block not in flat
    if not w.meta["prefix_tokens"]:
        assert len(flat) == len(set(flat)), "unshared workloads never reuse a block"
    for st in w.steps:
        assert (st.write_pos == st.context_lens - 1).all()
        assert st.q.shape == (w.num_seqs, w.num_q_heads, w.head_dim)
        assert st.k_new.shape == (len(st.write_seq), w.num_kv_heads, w.head_dim)
    # every resident token (all positions before step 0's write) holds finite data once
    # the step's copy-on-write copies are done (the tables already point at the copies)
    st0 = w.steps[0]
    pool64 = paged.to_f64(paged.block_copy_ref(w.pool, st0.cow_src, st0.cow_dst)[:, 0, 0, :, 0])
    for s in range(w.num_seqs):
        for t in range(int(st0.context_lens[s]) - 1):
            blk, off = paged.translate(w.block_tables[s], t, B)
            assert np.isfinite(pool64[blk, off])
    # blocks no sequence ever uses are poisoned
    used = set(flat) | set(st0.cow_src.tolist()) | set(st0.cow_dst.tolist())
    for b in range(w.num_blocks):
        if b not in used:
            assert np.isnan(pool64[b]).all()


def test_worked_example_shape():
    w = make_config(1)
    assert w.steps[0].context_lens.tolist() == [25, 47, 12]
    assert w.num_blocks == 16 and w.block_size == 16 and w.dtype == "f32"
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim) == (4, 4, 64)
    rows = live_blocks(w)
    assert [len(r) for r in rows] == [2, 3, 1]
    assert len(set(sum(rows, []))) == 6
    assert w.scale == np.float32(0.125)


def test_prefix_sharing_follows_the_oracle_cow_rule():
    """Replay workload 3's sharing with the oracle's pool: same tables, same copies."""
    for small in (True,):
        w = make_config(3, small=small)
        B, P = w.block_size, w.meta["prefix_tokens"] // w.block_size
        st = w.steps[0]
        lens = st.context_lens
        pool = alloc.BlockPool(w.num_blocks, B)
        cows = []
        tables = {}
        for g0 in range(0, w.num_seqs, w.meta["group"]):
            members = list(range(g0, min(w.num_seqs, g0 + w.meta["group"])))
            need = [acc.blocks_needed(int(lens[s]), B) for s in members]
            prefix = alloc.Sequence()
            # the group's prefix blocks are the first shared entries of the workload's tables
            owner = members[int(np.argmax(need))]
            shared_ids = [int(b) for b in w.block_tables[owner, :min(P, max(need))]]
            for b in shared_ids:
                if b in st.cow_dst.tolist():  # the owner itself may have copied one; find the source
                    b = int(st.cow_src[st.cow_dst.tolist().index(b)])
                pool.free_queue.remove(b)
                pool.refcount[b] = 1
                prefix.block_table.append(b)
            prefix.num_tokens = len(prefix.block_table) * B
            seqs = []
            for s, n in zip(members, need):
                seq = alloc.fork(pool, prefix, min(P, n))
                for j in range(min(P, n), n):  # private tail blocks
                    b = int(w.block_tables[s, j])
                    pool.free_queue.remove(b)
                    pool.refcount[b] = 1
                    seq.block_table.append(b)
                seqs.append(seq)
            alloc.release_sequence(pool, prefix)  # only the sequences hold the prefix now
            for s, seq in zip(members, seqs):
                fresh = [d for d in st.cow_dst.tolist() if d in w.block_tables[s].tolist()]
                if fresh:  # hand the oracle the same fresh block the workload used
                    pool.free_queue.remove(fresh[0])
                    pool.free_queue.appendleft(fresh[0])
                _, cow = alloc.prepare_write(pool, seq, int(lens[s]) - 1)
                if cow is not None:
                    cows.append(cow)
                tables[s] = seq.block_table
        assert cows == list(zip(st.cow_src.tolist(), st.cow_dst.tolist()))
        for s in range(w.num_seqs):
            n = acc.blocks_needed(int(lens[s]), B)
            assert tables[s] == w.block_tables[s, :n].tolist()
        assert len(cows) > 0


def test_growth_takes_a_block_exactly_when_a_write_starts_one():
    w = make_config(5, small=True)
    B = w.block_size
    for k, st in enumerate(w.steps):
        for s in range(w.num_seqs):
            have = acc.blocks_needed(int(st.context_lens[s]) - 1, B) if k else None
            need = acc.blocks_needed(int(st.context_lens[s]), B)
            if k:
                grew = [e for e in st.new_blocks if e[0] == s]
                assert (need > have) == bool(grew)
                if grew:
                    assert grew[0][1] == need - 1 and w.block_tables[s, need - 1] == grew[0][2]


def test_seeds_are_deterministic():
    a = make_config(3, small=True)
    b = make_config(3, small=True)
    assert np.array_equal(a.pool, b.pool) and np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.steps[0].q, b.steps[0].q)


def test_full_size_workload_structure():
    """Lengths, pool fit and distributions of the full workloads (no K/V materialised twice)."""
    w2 = make_config(2)
    lens = w2.steps[0].context_lens
    assert w2.num_seqs == 64 and lens.min() >= 4100 and lens.max() <= 4164
    assert w2.num_blocks == 38348 and w2.pool.dtype == np.uint16
    assert abs(w2.kv_bytes() - 1.083e9) < 0.01e9
    del w2


def test_tensor_parallel_share_keeps_the_sequences():
    """One GPU's share of the 70B-shaped workload at 8-way tensor parallelism: one KV head
    serving eight query heads, with workload 4's sequences, lengths, block size and pool size."""
    from workloads import make_tp_share
    w = make_tp_share(8)
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size) == (8, 1, 128, 32)
    assert w.pool.shape == (8192, 2, 1, 32, 128)
    assert list(w.steps[0].context_lens) == [32768] * 8
    # a permutation of the whole pool, as in workload 4
    assert sorted(w.block_tables.ravel().tolist()) == list(range(8192))
    assert w.kv_bytes(0) == 8 * 32768 * 2 * 1 * 128 * 2
