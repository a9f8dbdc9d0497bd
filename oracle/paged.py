"""Oracle for the paged KV-cache hot path: translation, writes, copies, decode.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``, which also lists the page
titles behind the citation keys).  Plain numpy; floating
point in float64.  The product HIP path never imports this module.

Storage conventions (inputs arrive exactly as the GPU stores them):

* A pool is a numpy array of shape ``[num_blocks][2][num_kv_heads][block_size]
  [head_dim]``: index 0 of the second axis is K, index 1 is V.  A physical
  block is therefore one contiguous chunk holding K and V of ``block_size``
  consecutive positions of one sequence ([AINEW] "PagedAttention in one
  picture": a block carries K and V for a run of consecutive positions; the
  axis order inside a block is this project's choice).
* fp32 data is held as ``np.float32``; bf16 data as ``np.uint16`` bit patterns
  (the upper half of the fp32 encoding).  Writes and copies move these bits
  unchanged; attention first widens them exactly to float64.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# exact widening of the stored element types
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly.

    A bf16 value is, by definition, the upper 16 bits of an IEEE binary32
    value; shifting the pattern into the upper half of a 32-bit word and
    reinterpreting it as float32 reproduces the value exactly, and float32 to
    float64 is exact.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray) -> np.ndarray:
    """Widen a stored array (float32, or uint16 holding bf16) to float64."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        return bf16_bits_to_f64(arr)
    if arr.dtype == np.float32 or arr.dtype == np.float64:
        return arr.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {arr.dtype}")


# ---------------------------------------------------------------------------
# address translation
# ---------------------------------------------------------------------------


def logical_block_and_offset(token_index: int, block_size: int) -> tuple[int, int]:
    """Token position -> (logical block index, offset inside the block).

    [HRL] §5 "What the Block Table Does" and §17 "A Minimal Pseudocode
    Walkthrough": the logical block is the position divided by the block size
    (rounded down) and the offset is the remainder.
    """
    if token_index < 0:
        raise ValueError("token index must be non-negative")
    return token_index // block_size, token_index % block_size


def translate(table_row, token_index: int, block_size: int) -> tuple[int, int]:
    """Token position -> (physical block id, offset), through one block table row.

    [HRL] §5: look the logical block up in the request's block table to find
    the physical block, then use the offset inside that block.
    """
    logical, offset = logical_block_and_offset(token_index, block_size)
    if logical >= len(table_row):
        raise IndexError(f"token {token_index} lies beyond the block table ({len(table_row)} blocks)")
    return int(table_row[logical]), offset


def slot_id(table_row, token_index: int, block_size: int) -> int:
    """Flat slot id of a token: physical block times block size plus offset.

    [TSS] "Finding a token: position, block, slot": the slot of a token is its
    block number multiplied by the block size, plus its offset in the block.
    """
    physical, offset = translate(table_row, token_index, block_size)
    return physical * block_size + offset


def slot_mapping_ref(block_tables, seq_ids, positions, block_size: int) -> np.ndarray:
    """Slots for a list of (sequence, position) tokens; a negative position gives -1.

    [TSS] "Finding a token": the slot of every token written in a step, one
    token at a time.  The -1 marker for padding entries is this project's
    convention (the cache write skips negative slots).
    """
    seq_ids = np.asarray(seq_ids)
    positions = np.asarray(positions)
    out = np.empty(len(positions), dtype=np.int64)
    for i in range(len(positions)):
        pos = int(positions[i])
        if pos < 0:
            out[i] = -1
        else:
            out[i] = slot_id(block_tables[int(seq_ids[i])], pos, block_size)
    return out


# ---------------------------------------------------------------------------
# cache write and block copy (bit copies)
# ---------------------------------------------------------------------------


def cache_write_ref(pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, slots) -> np.ndarray:
    """Scatter each new token's K and V into its slot; returns the updated pool.

    [VIBE] vLLM procedure step 4 (a generated token's key and value go into the
    next free slot of the last block) and [HRL] §17 ``write_kv`` (slot = block
    and offset found through the table).  The slot is split back into (block,
    offset) by the inverse of [TSS] "Finding a token".  Every head's K row and
    V row of token ``i`` is copied bit for bit; a negative slot is skipped.

    ``k_new`` and ``v_new`` have shape ``[T][num_kv_heads][head_dim]`` and the
    pool's storage dtype.
    """
    pool = pool.copy()
    num_blocks, two, num_kv_heads, block_size, head_dim = pool.shape
    assert two == 2
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    assert k_new.dtype == pool.dtype and v_new.dtype == pool.dtype
    assert k_new.shape == (len(slots), num_kv_heads, head_dim) == v_new.shape
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = slot // block_size, slot % block_size
        if block >= num_blocks:
            raise IndexError(f"slot {slot} lies outside the pool")
        for h in range(num_kv_heads):
            pool[block, 0, h, offset, :] = k_new[i, h, :]
            pool[block, 1, h, offset, :] = v_new[i, h, :]
    return pool


def block_copy_ref(pool: np.ndarray, src_blocks, dst_blocks) -> np.ndarray:
    """Copy whole physical blocks (K and V, every head, every slot); returns the pool.

    [AINEW] copy-on-write passage, [SALIV] "Advanced Memory Sharing and
    Copy-on-Write", [VIBE] step 6: the writer gets a fresh block holding a
    copy of the shared one.  Every copy reads the pool as it was before the
    call, so the result does not depend on the order of the pairs.
    """
    before = pool
    pool = pool.copy()
    src_blocks = np.asarray(src_blocks)
    dst_blocks = np.asarray(dst_blocks)
    assert src_blocks.shape == dst_blocks.shape
    for s, d in zip(src_blocks.tolist(), dst_blocks.tolist()):
        pool[d] = before[s]
    return pool


# ---------------------------------------------------------------------------
# table walk, attention, decode
# ---------------------------------------------------------------------------


def gather_ref(pool: np.ndarray, table_row, context_len: int, kv_head: int):
    """Rebuild one sequence's contiguous K and V (float64) for one KV head.

    [HRL] §14 "Why a Dedicated Kernel Is Needed" (per token: find its logical
    block, translate to the physical block, take the offset, read K and V)
    and §17 ``read_kv``.  Returns two arrays of shape ``[context_len][head_dim]``.
    """
    block_size = pool.shape[3]
    head_dim = pool.shape[4]
    keys = np.empty((context_len, head_dim), dtype=np.float64)
    values = np.empty((context_len, head_dim), dtype=np.float64)
    for t in range(context_len):
        physical, offset = translate(table_row, t, block_size)
        keys[t] = to_f64(pool[physical, 0, kv_head, offset, :])
        values[t] = to_f64(pool[physical, 1, kv_head, offset, :])
    return keys, values


def attention_ref(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Textbook softmax attention of one query over ``L`` keys and values.

    [HRL] §8 "Does PagedAttention Change the Attention Computation Itself?":
    the output is softmax(q K^T * scale) V with the ordinary formula; paging
    changes only where K and V live.  The maximum score is subtracted before
    the exponential (it cancels in the ratio).
    """
    q = np.asarray(q, dtype=np.float64)
    scores = (keys @ q) * float(scale)
    m = scores.max()
    p = np.exp(scores - m)
    return (p @ values) / p.sum()


def decode_ref(pool: np.ndarray, q: np.ndarray, block_tables, context_lens, scale: float) -> np.ndarray:
    """One decode step of paged attention for every (sequence, query head).

    For sequence ``s`` and query head ``hq`` the query attends over all
    ``context_lens[s]`` cached positions (the position written this step
    included), found by walking the sequence's block table ([VIBE] step 5;
    [HRL] §9: a decode query attends over every key and value cached so far).
    Query heads map to KV heads in contiguous groups: ``h = hq // (Hq / Hkv)``
    ([VIBE] "Across GPUs": query heads share KV heads; the grouping order is
    this project's reading).  A zero context gives a zero output (convention).

    ``q`` has shape ``[S][Hq][head_dim]`` in the pool's storage dtype; the
    result is float64 ``[S][Hq][head_dim]``.
    """
    num_kv_heads = pool.shape[2]
    head_dim = pool.shape[4]
    q = np.asarray(q)
    num_seqs, num_q_heads, qd = q.shape
    assert qd == head_dim and num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    q64 = to_f64(q)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        length = int(context_lens[s])
        if length == 0:
            continue
        for h in range(num_kv_heads):
            keys, values = gather_ref(pool, block_tables[s], length, h)
            for g in range(group):
                hq = h * group + g
                out[s, hq] = attention_ref(q64[s, hq], keys, values, scale)
    return out


def decode_one_ref(pool: np.ndarray, q: np.ndarray, block_tables, context_lens, scale: float,
                   seq: int, q_head: int) -> np.ndarray:
    """``decode_ref`` restricted to a single (sequence, query head) output row.

    Same steps as ``decode_ref``; lets tests sample outputs of full-size
    workloads one by one.
    """
    num_kv_heads = pool.shape[2]
    num_q_heads = q.shape[1]
    group = num_q_heads // num_kv_heads
    length = int(context_lens[seq])
    if length == 0:
        return np.zeros(pool.shape[4], dtype=np.float64)
    keys, values = gather_ref(pool, block_tables[seq], length, q_head // group)
    return attention_ref(to_f64(q[seq, q_head]), keys, values, scale)


def prefill_ref(pool: np.ndarray, q: np.ndarray, query_start_loc, context_lens, block_tables,
                scale: float) -> np.ndarray:
    """Prefill (or chunked prefill) attention of many queries per sequence, causal.

    [HRL] §9 "How PagedAttention Appears in Prefill and Decode": prefill runs
    the prompt's tokens together and fills their K/V into the blocks;
    [TSS] "Next": chunked prefill processes a prompt a piece at a time.
    Sequence ``s`` owns query rows ``query_start_loc[s] .. query_start_loc[s+1]-1``;
    they are its last ``n_s`` positions, so row ``i`` sits at position
    ``p = context_lens[s] - n_s + i`` and attends, as ordinary causal attention
    does, over cached positions ``0 .. p`` found through the block table
    ([HRL] §8 formula; §14 table walk).  ``q`` is ``[T][Hq][D]`` in the pool's
    storage dtype; the result is float64 ``[T][Hq][D]``.
    """
    num_kv_heads = pool.shape[2]
    head_dim = pool.shape[4]
    q = np.asarray(q)
    total, num_q_heads, qd = q.shape
    assert qd == head_dim and num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    q64 = to_f64(q)
    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    starts = np.asarray(query_start_loc, dtype=np.int64)
    for s in range(len(starts) - 1):
        n = int(starts[s + 1] - starts[s])
        ctx = int(context_lens[s])
        if n == 0:
            continue
        assert 0 < n <= ctx
        for h in range(num_kv_heads):
            keys, values = gather_ref(pool, block_tables[s], ctx, h)
            for i in range(n):
                pos = ctx - n + i
                row = int(starts[s]) + i
                for g in range(group):
                    hq = h * group + g
                    out[row, hq] = attention_ref(q64[row, hq], keys[:pos + 1], values[:pos + 1], scale)
    return out
