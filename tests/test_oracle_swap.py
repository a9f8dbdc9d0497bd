"""Pins of the oracle swap (oracle/swap.py) to the pages and to invariants.

[VIBE] "The vLLM procedure" steps 7-8: all of a sequence's blocks leave at
once, sequences sharing blocks leave together, and evicted blocks come back
from CPU memory later; [HRL] §12: blocks of lower-priority requests move to
CPU memory.  The data tests move real block contents with the pairs a swap
returns and check that every sequence reads back exactly what it held.

Citation keys ([HRL], [TSS], [VIBE], ...): the page titles listed in oracle/__init__.py.
"""

import numpy as np
import pytest

from oracle import alloc, paged, swap


def pools(rng, n_gpu, n_host, B=4, H=2, D=8):
    gpu = rng.standard_normal((n_gpu, 2, H, B, D))
    host = np.full((n_host, 2, H, B, D), np.nan)
    return gpu, host


def seq_with(pool, n_tokens):
    s = alloc.Sequence()
    alloc.allocate_prompt(pool, s, n_tokens)
    return s


def gather(data, seq, B, L):
    return [paged.gather_ref(data, np.asarray(seq.block_table), L, h) for h in range(data.shape[2])]


def test_round_trip_restores_every_sequence_exactly():
    rng = np.random.default_rng(0)
    B = 4
    gpu_pool = alloc.BlockPool(24, B, reserve_null_block=True)
    host_pool = alloc.BlockPool(16, B)
    gpu, host = pools(rng, 24, 16, B)
    a, b = seq_with(gpu_pool, 10), seq_with(gpu_pool, 7)
    before = {id(s): gather(gpu, s, B, s.num_tokens) for s in (a, b)}
    q = rng.standard_normal((2, 2, 8))

    def decode():
        tables = np.zeros((2, 3), dtype=np.int32)
        tables[0, :3], tables[1, :2] = a.block_table, b.block_table
        return paged.decode_ref(gpu, q, tables, [10, 7], 0.35)

    out_before = decode()
    pairs = swap.swap_out(gpu_pool, host_pool, [a, b])
    assert len(pairs) == 3 + 2 and a.on_host and b.on_host
    for g, h in pairs:
        host[h] = gpu[g]
    # memory pressure: another request takes the freed GPU blocks and overwrites them
    other = seq_with(gpu_pool, gpu_pool.num_free * B)
    gpu[other.block_table] = rng.standard_normal(gpu[other.block_table].shape)
    alloc.release_sequence(gpu_pool, other)
    back = swap.swap_in(gpu_pool, host_pool, [a, b])
    assert len(back) == 5 and host_pool.num_free == 16
    for h, g in back:
        gpu[g] = host[h]
    for s in (a, b):
        after = gather(gpu, s, B, s.num_tokens)
        for k0, k1 in zip(before[id(s)], after):
            assert all(np.array_equal(x, y) for x, y in zip(k0, k1))
    # attention over the restored blocks is unchanged, bit for bit (identical inputs)
    assert np.array_equal(decode(), out_before)


def test_all_blocks_leave_at_once_and_shared_blocks_are_copied_once():
    rng = np.random.default_rng(1)
    B = 4
    gpu_pool = alloc.BlockPool(32, B, reserve_null_block=True)
    host_pool = alloc.BlockPool(32, B)
    parent = seq_with(gpu_pool, 12)                  # 3 blocks
    beam1 = alloc.fork(gpu_pool, parent)             # shares all 3
    beam2 = alloc.fork(gpu_pool, parent, 2)          # shares the first 2
    alloc.prepare_write(gpu_pool, beam2, 8)          # and grows its own third block
    outsider = alloc.fork(gpu_pool, parent, 1)       # holds block 0 and is not swapped
    old = list(parent.block_table)
    own = beam2.block_table[2]
    free_before = gpu_pool.num_free
    pairs = swap.swap_out(gpu_pool, host_pool, [parent, beam1, beam2])
    # distinct blocks of the group: parent's 3 + beam2's own one, each copied once
    assert len(pairs) == 4 and sorted(g for g, _ in pairs) == sorted(old + [own])
    assert beam1.block_table == parent.block_table and beam2.block_table[:2] == parent.block_table[:2]
    hb = parent.block_table
    assert [host_pool.refcount[h] for h in hb] == [3, 3, 2]
    # the group holds no GPU block; block 0 stays on the GPU for the outsider
    assert gpu_pool.refcount[old[0]] == 1 and gpu_pool.refcount[old[1]] == 0 and gpu_pool.refcount[old[2]] == 0
    assert gpu_pool.refcount[own] == 0 and gpu_pool.num_free == free_before + 3
    assert outsider.block_table == [old[0]]
    # swap-in: one GPU block per host block, shared again by the same holders
    back = swap.swap_in(gpu_pool, host_pool, [parent, beam1, beam2])
    assert len(back) == 4 and host_pool.num_free == 32
    assert beam1.block_table == parent.block_table and beam2.block_table[:2] == parent.block_table[:2]
    assert [gpu_pool.refcount[b] for b in parent.block_table] == [3, 3, 2]


def test_swap_is_all_or_nothing():
    rng = np.random.default_rng(2)
    gpu_pool = alloc.BlockPool(16, 4)
    host_pool = alloc.BlockPool(2, 4)
    a = seq_with(gpu_pool, 12)
    state = (list(gpu_pool.free_queue), list(gpu_pool.refcount), list(a.block_table))
    with pytest.raises(alloc.OutOfBlocks):
        swap.swap_out(gpu_pool, host_pool, [a])
    assert (list(gpu_pool.free_queue), list(gpu_pool.refcount), list(a.block_table)) == state
    assert host_pool.num_free == 2 and not getattr(a, "on_host", False)
    # and back in: a full GPU pool refuses the swap-in
    host_pool = alloc.BlockPool(8, 4)
    swap.swap_out(gpu_pool, host_pool, [a])
    hog = seq_with(gpu_pool, gpu_pool.num_free * 4 - 4)   # leaves 1 free block, a needs 3
    with pytest.raises(alloc.OutOfBlocks):
        swap.swap_in(gpu_pool, host_pool, [a])
    assert a.on_host and host_pool.num_free == 5
    with pytest.raises(ValueError):
        swap.swap_out(gpu_pool, host_pool, [a])              # already out
    with pytest.raises(ValueError):
        swap.swap_in(gpu_pool, host_pool, [hog])             # not out
    swap.release_swapped(host_pool, a)
    assert host_pool.num_free == 8 and list(host_pool.free_queue)[:3] == sorted(list(host_pool.free_queue)[:3])
