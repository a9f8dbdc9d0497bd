"""Oracle swap-out / swap-in of sequences between the GPU block pool and a host pool.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``, which also lists the page
titles behind the citation keys).  Pure Python.  It
follows [VIBE] "The vLLM procedure" steps 7 and 8 (when blocks run out, all
of a sequence's blocks are evicted at once, sequences sharing blocks are
evicted together, and evicted blocks are copied to CPU memory and copied back
later) and [HRL] §12 "Understanding Swap and Eviction" (moving lower-priority
requests' blocks to CPU memory).  It moves no data: a swap returns the
(source block, destination block) pairs that a cross-pool block copy performs.

Readings where the pages leave steps open:

* One call swaps a list of sequences as a group.  Their tables are walked in
  list order, each table first to last; the first time a block is met it gets
  a fresh block in the other pool (one copy pair), and every later holder in
  the group shares that copy (one reference each), so a block shared inside
  the group is copied once.
* Each listed sequence then drops its references in the pool it left, its
  blocks last to first (as a finished sequence does); a block still held by a
  sequence outside the group keeps its copy there.
* All or nothing: when the destination pool has fewer free blocks than the
  group has distinct blocks, nothing changes.
* Host blocks are numbered 0..H-1 in a pool of their own; a host block whose
  count reaches zero goes to the front of the host free queue.
* A swapped-out sequence can be swapped in or freed; nothing else.
"""

from __future__ import annotations

from . import alloc


def _move(src: alloc.BlockPool, dst: alloc.BlockPool, seqs) -> list[tuple[int, int]]:
    distinct = []
    seen = set()
    for s in seqs:
        for b in s.block_table:
            if b not in seen:
                seen.add(b)
                distinct.append(b)
    if len(distinct) > dst.num_free:
        raise alloc.OutOfBlocks("destination pool has too few free blocks for the group")
    mapping: dict[int, int] = {}
    pairs = []
    new_tables = []
    for s in seqs:
        table = []
        for b in s.block_table:
            if b in mapping:
                dst.share(mapping[b])
            else:
                mapping[b] = dst.allocate()
                pairs.append((b, mapping[b]))
            table.append(mapping[b])
        new_tables.append(table)
    for s, table in zip(seqs, new_tables):
        for b in reversed(s.block_table):
            src.release(b)
        s.block_table = table
    return pairs


def swap_out(gpu: alloc.BlockPool, host: alloc.BlockPool, seqs) -> list[tuple[int, int]]:
    """Move the group's blocks to the host pool; returns (GPU block, host block) copy pairs."""
    if len({id(s) for s in seqs}) != len(seqs) or any(getattr(s, "on_host", False) for s in seqs):
        raise ValueError("each sequence once, and only sequences on the GPU")
    pairs = _move(gpu, host, seqs)
    for s in seqs:
        s.on_host = True
    return pairs


def swap_in(gpu: alloc.BlockPool, host: alloc.BlockPool, seqs) -> list[tuple[int, int]]:
    """Bring the group's blocks back; returns (host block, GPU block) copy pairs."""
    if len({id(s) for s in seqs}) != len(seqs) or not all(getattr(s, "on_host", False) for s in seqs):
        raise ValueError("each sequence once, and only swapped-out sequences")
    pairs = _move(host, gpu, seqs)
    for s in seqs:
        s.on_host = False
    return pairs


def release_swapped(host: alloc.BlockPool, seq) -> None:
    """Free a swapped-out sequence: its host blocks, last to first."""
    for b in reversed(seq.block_table):
        host.release(b)
    seq.block_table = []
    seq.num_tokens = 0
    seq.on_host = False
