"""Helpers shared by the GPU tests: move seeded workloads to the device and back,
and run one decode step through the C ABI (via the thin binding)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_cache_121_amd as pa

DEV = "cuda:0"


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_dev(arr: np.ndarray, dtype: str):
    """numpy storage array (float32, or uint16 bf16 bits) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def to_host(t) -> np.ndarray:
    """device tensor -> numpy storage array (uint16 bits for bf16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def device_pool(w) -> pa.PagedKVPool:
    return pa.PagedKVPool(to_dev(w.pool, w.dtype))


def run_step(w, pool: pa.PagedKVPool, tables_dev, k: int, partition_size: int = 0, max_context_len=None,
             keep_cached=None):
    """One step of workload ``w`` on the GPU: COW copies, slot mapping, cache write, decode."""
    st = w.steps[k]
    if len(st.cow_src):
        pa.pa_block_copy(pool, i32(st.cow_src), i32(st.cow_dst))
    slots = pa.pa_slot_mapping(pool, tables_dev, i32(st.write_seq), i32(st.write_pos))
    pa.pa_cache_write(pool, to_dev(st.k_new, w.dtype), to_dev(st.v_new, w.dtype), slots)
    lens = i32(st.context_lens)
    mcl = int(st.context_lens.max()) if max_context_len is None else max_context_len
    if keep_cached is None:  # workloads that share blocks keep K/V cached, the others stream
        keep_cached = bool(w.meta.get("prefix_tokens"))
    out = pa.pa_decode(pool, to_dev(st.q, w.dtype), tables_dev, lens, scale=float(w.scale),
                       max_context_len=mcl, partition_size=partition_size, keep_cached=keep_cached)
    return slots, out


def oracle_step(w, pool_np: np.ndarray, k: int):
    """The same step on the CPU oracle; returns (slots, pool after the write)."""
    from oracle import paged
    st = w.steps[k]
    if len(st.cow_src):
        pool_np = paged.block_copy_ref(pool_np, st.cow_src, st.cow_dst)
    slots = paged.slot_mapping_ref(w.block_tables, st.write_seq, st.write_pos, w.block_size)
    pool_np = paged.cache_write_ref(pool_np, st.k_new, st.v_new, slots)
    return slots, pool_np
