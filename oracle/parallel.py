"""The oracle's decode over many sequences, in worker processes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  No arithmetic of its
own: sequences of a decode step are independent ([HRL] section 8: each
query attends over its own sequence's keys and values), so each worker runs
``paged.decode_ref`` -- and, where a task carries writes, ``paged.cache_write_ref``
first -- on one sequence's blocks, copied out of the pool in table order and
addressed through the identity table.  That is the same walk as over the whole
pool, since a table only names where each logical block lives.

Workers are started with the ``spawn`` method (fresh interpreters that import
numpy and this package only), so a caller that holds a GPU context never
forks it.
"""

from __future__ import annotations

import concurrent.futures
import multiprocessing
import os

import numpy as np

from . import accounting, paged


def host_cores() -> int:
    """CPU cores this process may run on."""
    return len(os.sched_getaffinity(0))


def sequence_task(pool: np.ndarray, table_row, length: int, q_row: np.ndarray, scale: float,
                  writes=None) -> tuple:
    """One sequence's work: its first ceil(length / B) blocks (copies, in table order), its
    query rows ``[Hq][D]``, its length and scale, and optionally this sequence's writes
    ``(positions, k rows, v rows)`` to replay on those blocks before attending."""
    B = pool.shape[3]
    nb = accounting.blocks_needed(length, B)
    blocks = pool[np.asarray(table_row[:nb], dtype=np.int64)]
    return blocks, np.asarray(q_row), int(length), float(scale), writes


def run_task(task) -> np.ndarray:
    """Oracle output ``[Hq][D]`` (float64) of one ``sequence_task``."""
    blocks, q_row, length, scale, writes = task
    nb = blocks.shape[0]
    table = np.arange(nb, dtype=np.int32)[None, :]
    if writes is not None and len(writes[0]):
        pos, k_new, v_new = writes
        slots = paged.slot_mapping_ref(table, np.zeros(len(pos), dtype=np.int32), pos, blocks.shape[3])
        blocks = paged.cache_write_ref(blocks, k_new, v_new, slots)
    return paged.decode_ref(blocks, q_row[None], table, [length], scale)[0]


def _one_blas_thread() -> None:
    """Worker start-up: one BLAS thread per process (the workers already use every core)."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def worker_pool(workers: int | None = None) -> concurrent.futures.ProcessPoolExecutor:
    """A pool of ``workers`` spawned processes (default: every core this process may use, at
    most 16), one BLAS thread each, to pass to several ``run_tasks`` calls."""
    if workers is None:
        workers = min(host_cores(), 16)
    return concurrent.futures.ProcessPoolExecutor(max_workers=max(1, workers),
                                                  mp_context=multiprocessing.get_context("spawn"),
                                                  initializer=_one_blas_thread)


def run_tasks(tasks, pool: concurrent.futures.Executor | None = None, workers: int | None = None,
              timeout: float = 900.0) -> list:
    """``run_task`` over ``tasks``, results in task order: in ``pool`` if given, else in a
    pool of ``workers`` processes made for this call (``workers=1``: in this process).
    Raises ``TimeoutError`` if the results take longer than ``timeout`` seconds (a worker
    that failed to start never answers)."""
    tasks = list(tasks)
    if pool is not None:
        return list(pool.map(run_task, tasks, chunksize=1, timeout=timeout))
    if workers is None:
        workers = min(host_cores(), 16)
    workers = max(1, min(workers, len(tasks)))
    if workers == 1:
        return [run_task(t) for t in tasks]
    with worker_pool(workers) as ex:
        return list(ex.map(run_task, tasks, chunksize=1, timeout=timeout))
