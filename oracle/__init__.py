"""Plain CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
links anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path: no kernels, helpers, tables or constants.

Everything is numpy, in float64 for floating point, and follows the pages it
cites step by step with no blocking, fusion or reordering:

* ``paged``      -- address translation, slot mapping, cache write, block copy,
                    table-walk gather, textbook softmax attention, decode.
* ``alloc``      -- the block pool bookkeeping the pages describe (free list,
                    null block, reference counts, on-demand growth,
                    copy-on-write decision).
* ``accounting`` -- block counts, slot usage and waste, KV byte sizes.
* ``prefix``     -- prefix caching: chained block hashes, the table of
                    cached blocks, hits capped at the prompt minus one.
* ``swap``       -- swap-out / swap-in of sequence groups between the GPU
                    pool and a host pool (the copy pairs a swap needs).
* ``parallel``   -- the decode oracle run per sequence in spawned worker
                    processes (no arithmetic of its own; for full-size checks
                    and the all-cores CPU baseline).

Citation keys used in docstrings (page title, then section):

* [AINEW]  "PagedAttention: KV-cache virtual memory technique improves
           inference efficiency" (news.ainew.jp, Arc 6 post)
* [SALIV]  "How PagedAttention Eliminates KV-Cache Fragmentation"
           (salivity.github.io)
* [VIBE]   "PagedAttention, explained." (vibeengines.com)
* [HRL]    "What Does PagedAttention Actually Optimize?" (hrletsgo.me)
* [TSS]    "Paged Attention: Virtual Memory for the KV Cache"
           (theservingstack.com)

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against values the pages print, brute force, closed forms or invariants,
except where a docstring says "parity unpinned".
"""

from . import accounting, alloc, paged, parallel, prefix, swap  # noqa: F401
