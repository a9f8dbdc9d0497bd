"""Oracle prefix cache: chained block hashes over the block pool.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``, which also lists the page
titles behind the citation keys).  Pure Python, slow and
direct.  It follows [TSS] "Sharing a prefix: one copy for many requests": each
full block is named by a hash of its own tokens and of the previous block's
hash, so the hash of block j stands for the whole prompt up to the end of
block j; a new prompt is hashed block by block and every hash found in the
table of cached blocks is a block the request points at instead of computing
it (``touch`` adds a reference); only full blocks are shared; a hit covers at
most the prompt minus one token; freed blocks keep their hash and wait at the
back of the free queue until a later allocation takes them.

Where the page leaves a step open, these readings are taken:

* The hash is SHA-256 (FIPS 180-4) of the parent block's 32-byte digest
  followed by the block's token ids as little-endian int32; the first block's
  parent is 32 zero bytes.  The page fixes only the inputs of the hash.
* The hit is the longest run of leading blocks whose hashes are cached,
  limited to floor((n - 1) / B) blocks for an n-token prompt, so at least one
  prompt token is always computed (a block-aligned prompt recomputes its last
  block).
* A prompt's full blocks are entered into the table when the prompt is
  allocated (they are computed in that same step); blocks filled later are
  entered when the id of their last token is committed.  A block that already
  carries a hash keeps it, and a hash already in the table keeps its block.
* Taking a block that carries a hash from the free queue removes the hash
  (eviction).  A write into a block that carries a hash removes the hash
  first, since its contents change; committed tokens cannot be rewritten.
* A released block that carries a hash goes to the back of the free queue
  ("reusable"), any other block to the front unless the caller marks it
  reusable.
"""

from __future__ import annotations

import hashlib
import struct

from . import alloc
from .accounting import blocks_needed

ROOT = bytes(32)


def hash_block(parent: bytes, tokens) -> bytes:
    """Hash of one full block: SHA-256 over parent digest || int32 LE token ids."""
    data = bytes(parent) + b"".join(struct.pack("<i", int(t)) for t in tokens)
    return hashlib.sha256(data).digest()


def block_hashes(tokens, block_size: int, parent: bytes = ROOT) -> list[bytes]:
    """Chained hashes of every full block of ``tokens`` (the partial tail has none)."""
    out = []
    h = parent
    for j in range(len(tokens) // block_size):
        h = hash_block(h, tokens[j * block_size:(j + 1) * block_size])
        out.append(h)
    return out


class PrefixCachingPool(alloc.BlockPool):
    """A block pool with a table of cached blocks: hash -> block and back."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None, reserve_null_block: bool = False):
        super().__init__(num_blocks, block_size, free_order=free_order, reserve_null_block=reserve_null_block)
        self.cached: dict[bytes, int] = {}
        self.hash_of: dict[int, bytes] = {}

    def forget(self, block: int) -> None:
        """Drop the block's hash from the table, if it has one."""
        h = self.hash_of.pop(block, None)
        if h is not None:
            del self.cached[h]

    def register(self, block: int, h: bytes) -> bool:
        """Enter ``block`` under ``h`` unless either is already in the table."""
        if block in self.hash_of or h in self.cached:
            return False
        self.cached[h] = block
        self.hash_of[block] = h
        return True

    def allocate(self) -> int:
        block = super().allocate()
        self.forget(block)  # a cached block taken for new contents is evicted
        return block

    def touch(self, block: int) -> None:
        """One more reference to a cached block, taking it off the free queue if idle."""
        if self.refcount[block] == 0:
            self.free_queue.remove(block)
            self.refcount[block] = 1
        else:
            self.refcount[block] += 1

    def release(self, block: int, reusable: bool = False) -> None:
        super().release(block, reusable=reusable or block in self.hash_of)


class CachedSequence(alloc.Sequence):
    """A sequence that also records the ids of its committed tokens."""

    def __init__(self):
        super().__init__()
        self.tokens: list[int] = []


def commit_tokens(pool: PrefixCachingPool, seq: CachedSequence, ids) -> None:
    """Record the ids of the next tokens; enter every block they complete."""
    ids = [int(t) for t in ids]
    if len(seq.tokens) + len(ids) > seq.num_tokens:
        raise ValueError("committing tokens past the sequence's written positions")
    B = pool.block_size
    full_before = len(seq.tokens) // B
    seq.tokens.extend(ids)
    full_after = len(seq.tokens) // B
    if full_after > full_before:
        hashes = block_hashes(seq.tokens, B)
        for j in range(full_before, full_after):
            pool.register(seq.block_table[j], hashes[j])


def cached_prefix_blocks(pool: PrefixCachingPool, tokens) -> list[int]:
    """Blocks of the longest cached leading run of ``tokens``, capped at floor((n-1)/B)."""
    n = len(tokens)
    limit = (n - 1) // pool.block_size if n > 0 else 0
    hits = []
    for h in block_hashes(tokens, pool.block_size)[:limit]:
        block = pool.cached.get(h)
        if block is None:
            break
        hits.append(block)
    return hits


def allocate_prompt_cached(pool: PrefixCachingPool, seq: CachedSequence, tokens) -> int:
    """Prefill allocation with prefix caching; returns the number of cached tokens.

    The hit blocks are touched and put first in the table, the rest of
    ``blocks_needed(n)`` come from the free queue, and the prompt's ids are
    committed (entering its full blocks).  All or nothing: without enough
    free blocks (idle hit blocks leave the queue too) nothing changes.
    """
    if seq.block_table or seq.num_tokens:
        raise ValueError("prefix-cached allocation needs an empty sequence")
    n = len(tokens)
    hits = cached_prefix_blocks(pool, tokens)
    fresh = blocks_needed(n, pool.block_size) - len(hits)
    idle_hits = sum(1 for b in hits if pool.refcount[b] == 0)
    if fresh + idle_hits > pool.num_free:
        raise alloc.OutOfBlocks("not enough free blocks for the prompt")
    for b in hits:
        pool.touch(b)
        seq.block_table.append(b)
    for _ in range(fresh):
        seq.block_table.append(pool.allocate())
    seq.num_tokens = n
    commit_tokens(pool, seq, tokens)
    return len(hits) * pool.block_size


def prepare_write_cached(pool: PrefixCachingPool, seq: CachedSequence, token_index: int):
    """``alloc.prepare_write`` plus the cache rules: no rewrite of committed
    tokens, and the written block loses its hash (its contents change)."""
    if token_index < len(seq.tokens):
        raise ValueError("position already committed")
    slot, cow = alloc.prepare_write(pool, seq, token_index)
    pool.forget(seq.block_table[token_index // pool.block_size])
    return slot, cow


def fork_cached(pool: PrefixCachingPool, parent: CachedSequence, num_shared_blocks: int | None = None):
    """``alloc.fork`` that also carries the parent's committed ids over the shared span."""
    base = alloc.fork(pool, parent, num_shared_blocks)
    child = CachedSequence()
    child.block_table, child.num_tokens = base.block_table, base.num_tokens
    child.tokens = parent.tokens[:child.num_tokens]
    return child
