"""Oracle bookkeeping: block counts, slot usage, waste and KV byte sizes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``, which also lists the page
titles behind the citation keys).  Integers only.
"""

from __future__ import annotations


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Number of blocks that hold ``num_tokens`` tokens: the ceiling of the ratio.

    [TSS] "Paging: blocks handed out as tokens arrive" (a request takes the
    rounded-up quotient of its token count by the block size); [VIBE] step 3
    (prefill allocates that many blocks); [AINEW] "A small worked example".
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("need num_tokens >= 0 and block_size > 0")
    q, r = divmod(num_tokens, block_size)
    return q + (1 if r else 0)


def table_lookups(num_tokens: int, block_size: int) -> int:
    """Block-table lookups a kernel makes to read ``num_tokens`` tokens: one per block.

    [AINEW] "Why the attention kernel works at all" (the 47-token request at
    three block sizes).
    """
    return blocks_needed(num_tokens, block_size)


def slots_paged(lengths, block_size: int) -> int:
    """Slots reserved under paging: every request rounded up to whole blocks.

    [AINEW] "A small worked example"; [HRL] §13 "A Simple Numerical Comparison".
    """
    return sum(blocks_needed(int(n), block_size) * block_size for n in lengths)


def slots_contiguous(num_requests: int, max_len: int) -> int:
    """Slots reserved when every request holds its maximum length up front.

    [AINEW] "Fragmented memory, wasted GPU"; [HRL] §13.
    """
    return num_requests * max_len


def waste_paged(lengths, block_size: int) -> int:
    """Reserved-but-empty slots under paging (only each request's last block).

    [HRL] §7 "Why Waste Is Confined to the Last Block": at most
    ``block_size - 1`` per request.
    """
    return slots_paged(lengths, block_size) - sum(int(n) for n in lengths)


def waste_contiguous(lengths, max_len: int) -> int:
    """Reserved-but-empty slots when each request reserves ``max_len`` slots.

    [VIBE] opening example: the unused part of the reservation is the maximum
    length minus the tokens actually held.
    """
    return sum(max_len - int(n) for n in lengths)


def kv_cache_bytes(num_requests: int, num_tokens: int, num_layers: int, num_kv_heads: int,
                   head_dim: int, bytes_per_elem: int) -> int:
    """KV cache size as the product of its factors, times two for K and V.

    [HRL] §2 "Why the KV Cache Is So Large" (requests x tokens x layers x KV
    heads x head size x 2 x element size); [VIBE] "Start with the number"
    (per-token size of OPT-13B).
    """
    return num_requests * num_tokens * num_layers * num_kv_heads * head_dim * 2 * bytes_per_elem
