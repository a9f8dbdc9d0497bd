"""Oracle block pool: free list, reference counts, growth and copy-on-write.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``, which also lists the page
titles behind the citation keys).  Pure Python.  This is
the bookkeeping the pages describe around the kernels; it pins the pages'
worked examples and checks the structure of generated workloads.  It moves no
data: a copy-on-write returns the (source, destination) pair that a block copy
must perform.
"""

from __future__ import annotations

from collections import deque

from .accounting import blocks_needed


class OutOfBlocks(RuntimeError):
    """No free physical block is left ([VIBE] step 7: the point where vLLM preempts)."""


class BlockPool:
    """Physical block pool with a free queue and per-block reference counts.

    [TSS] "Inside vLLM: the block pool": every block exists from the start;
    free blocks wait in a queue; allocation takes the front; each allocated
    block carries a reference count; a block whose count reaches zero returns
    to the back of the queue when its contents may be reused, else to the
    front.  Block 0 can be held back as the never-allocated null block that
    pads table entries.  [HRL] §17 ``allocate_block`` also pops the front.

    ``free_order`` fixes the initial queue (default: ascending ids).
    """

    def __init__(self, num_blocks: int, block_size: int, free_order=None, reserve_null_block: bool = False):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.refcount = [0] * self.num_blocks
        order = list(range(self.num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != sorted(set(order)) or any(b < 0 or b >= self.num_blocks for b in order):
            raise ValueError("free_order must list distinct block ids inside the pool")
        self.null_block = None
        if reserve_null_block:
            self.null_block = 0
            order = [b for b in order if b != 0]
        self.free_queue = deque(order)

    @property
    def num_free(self) -> int:
        return len(self.free_queue)

    @property
    def num_in_use(self) -> int:
        return sum(1 for c in self.refcount if c > 0)

    def allocate(self) -> int:
        """Pop the front of the free queue; the block starts with one reference."""
        if not self.free_queue:
            raise OutOfBlocks("free queue is empty")
        block = self.free_queue.popleft()
        assert self.refcount[block] == 0
        self.refcount[block] = 1
        return block

    def share(self, block: int) -> None:
        """Add one more logical reference to an allocated block ([TSS] ``touch``)."""
        if self.refcount[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self.refcount[block] += 1

    def release(self, block: int, reusable: bool = False) -> None:
        """Drop one reference; at zero the block re-enters the free queue.

        Back of the queue if its contents may be reused (so it is taken
        last), front otherwise ([TSS] ``free_blocks`` ordering).
        """
        if self.refcount[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            if reusable:
                self.free_queue.append(block)
            else:
                self.free_queue.appendleft(block)


class Sequence:
    """A request's state: its token count and its block table ([HRL] §17 ``RequestState``)."""

    def __init__(self):
        self.num_tokens = 0
        self.block_table: list[int] = []


def ensure_capacity(pool: BlockPool, seq: Sequence, token_index: int) -> list[int]:
    """Append freshly allocated blocks until the table covers ``token_index``.

    [HRL] §17 ``ensure_capacity``: the logical block of the position is
    computed and blocks are popped from the free queue while the table is too
    short.  [VIBE] step 4: a new block is taken only when the last one is
    full.  Returns the blocks appended.
    """
    logical = token_index // pool.block_size
    added = []
    while len(seq.block_table) <= logical:
        block = pool.allocate()
        seq.block_table.append(block)
        added.append(block)
    return added


def allocate_prompt(pool: BlockPool, seq: Sequence, num_tokens: int) -> list[int]:
    """Prefill allocation: ``blocks_needed(num_tokens)`` blocks ([VIBE] step 3)."""
    added = []
    for _ in range(blocks_needed(num_tokens, pool.block_size) - len(seq.block_table)):
        block = pool.allocate()
        seq.block_table.append(block)
        added.append(block)
    seq.num_tokens = max(seq.num_tokens, num_tokens)
    return added


def fork(pool: BlockPool, parent: Sequence, num_shared_blocks: int | None = None) -> Sequence:
    """A new sequence whose table points at the parent's first blocks, shared.

    [AINEW] copy-on-write passage and [VIBE] step 6: several tables may point
    at one physical block; each extra pointer adds one reference.
    """
    n = len(parent.block_table) if num_shared_blocks is None else num_shared_blocks
    child = Sequence()
    for block in parent.block_table[:n]:
        pool.share(block)
        child.block_table.append(block)
    child.num_tokens = min(parent.num_tokens, n * pool.block_size)
    return child


def prepare_write(pool: BlockPool, seq: Sequence, token_index: int):
    """Make the slot of ``token_index`` writable; return ``(slot, cow_pair)``.

    Growth first ([HRL] §17 ``ensure_capacity``).  Then copy-on-write
    ([AINEW] copy-on-write passage; [SALIV] "Advanced Memory Sharing and
    Copy-on-Write"; [VIBE] step 6): when the block receiving the write has more
    than one reference, a fresh block is allocated, the shared block loses one
    reference, and only the writer's table is repointed to the fresh block;
    the caller copies the block contents (the returned ``(src, dst)`` pair)
    before writing.  With one reference the write goes in place and the pair
    is ``None``.  The slot is the physical block times the block size plus the
    offset ([TSS] "Finding a token").
    """
    ensure_capacity(pool, seq, token_index)
    logical, offset = token_index // pool.block_size, token_index % pool.block_size
    block = seq.block_table[logical]
    cow = None
    if pool.refcount[block] > 1:
        fresh = pool.allocate()
        pool.release(block)
        seq.block_table[logical] = fresh
        cow = (block, fresh)
        block = fresh
    seq.num_tokens = max(seq.num_tokens, token_index + 1)
    return block * pool.block_size + offset, cow


def release_sequence(pool: BlockPool, seq: Sequence, reusable: bool = False) -> None:
    """Return every block of a finished request ([HRL] §18 step 8; [TSS] "Paging").

    The pages leave the order open; the blocks are released last to first,
    so that of a request's reusable blocks (back of the queue) the tail is
    taken first and a cached chain of blocks is lost from its end.
    """
    for block in reversed(seq.block_table):
        pool.release(block, reusable=reusable)
    seq.block_table = []
    seq.num_tokens = 0
