"""Benchmark of the paged decode hot path on one MI355X.

One step = one pass of the whole path over one batch: slot mapping and cache
write of the step's new tokens (one fused launch, pa_cache_write_at), then
paged decode attention (copy-on-write block copies too when the workload has
them).  Inputs are seeded synthetic
data already resident in HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload 2] [--partition-size 0]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "decode attention KV-read GB/s (and % HBM peak); sequences·layers/sec"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "decode_qwen3_8b_b64_hbm_traffic.md")
PREFILL_TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                    "prefill_4x4100_hbm_traffic.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=str, default="2", choices=["1", "2", "3", "4", "5", "4tp8"],
                    help="1-5 (default: 2, the Qwen3-8B batch-64 layer), or 4tp8: one GPU's share of workload 4 "
                         "at 8-way tensor parallelism (1 KV head, 8 query heads)")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--decode-reps", type=int, default=50, help="timed decode-only launches for the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=12, help="sequences in the oracle's timed sample")
    ap.add_argument("--skip-check", action="store_true",
                    help="time the oracle sample but do not compare it with the GPU's rows")
    ap.add_argument("--prefill", type=int, default=0, metavar="K",
                    help="instead of the decode benchmark: prefill workload K (1: 4 x 4,100-token prompts, "
                         "2: 16 x 100-token chunks over a shared 4,000-token prefix)")
    ap.add_argument("--swap", action="store_true",
                    help="instead of the benchmark: swap copies device <-> pinned host at block sizes 4/16/128")
    ap.add_argument("--block-sweep", action="store_true",
                    help="instead of the benchmark: decode of workloads 2 and 5 at block sizes 4-128")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the summary of workloads 3-5 in the decode line")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill summary in the decode line")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="instead of the benchmark: HBM read rate of a 1 GiB buffer read in order and in "
                         "randomly placed 4/16/64 KiB pieces (the decode kernel's practical ceiling)")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the read-ceiling summary in the decode line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="PAIRS",
                    help="instead of the benchmark: run pa_block_copy over PAIRS distinct block pairs "
                         "(known bytes) 5 times, for scaling hardware byte counters")
    return ap.parse_args()


def kernel_source_digest(name: str = "decode.hip") -> str:
    """Digest of a kernel source's code: comments and blank lines are left out,
    so a comment edit does not invalidate counters taken on the same code."""
    import hashlib
    import re
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_121_amd", "csrc", name)
    with open(src) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def _traffic_json(path: str):
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    start = text.find("```json")
    if start < 0:
        return None
    return json.loads(text[start + 7:text.index("```", start + 7)])


def measured_traffic(workload: str, partition_size: int):
    """HBM bytes per decode launch from the committed counter summary, if it was
    taken on the current decode kernel source at this partition size; else None."""
    t = _traffic_json(TRAFFIC_FILE)
    e = t.get(f"workload{workload}") if t else None
    if not e or e.get("decode_source_sha256_16") != kernel_source_digest() or e.get("partition_size") != partition_size:
        return None
    return e.get("hbm_bytes_per_launch")


def measured_prefill_traffic(k: int):
    """HBM bytes per prefill launch from the committed counter summary, if it was
    taken on the current prefill kernel source; else None."""
    t = _traffic_json(PREFILL_TRAFFIC_FILE)
    e = t.get(f"prefill{k}") if t else None
    if not e or e.get("prefill_source_sha256_16") != kernel_source_digest("prefill.hip"):
        return None
    return e.get("hbm_bytes_per_launch")


def prefill_algorithmic_bytes(w) -> int:
    """Bytes one prefill launch must move at least: each sequence's visible K/V
    rows once (a block shared by several sequences counts once per sequence),
    the queries once, the fp32 output once."""
    elt = 2
    kv = int(np.sum(w.context_lens)) * 2 * w.num_kv_heads * w.head_dim * elt
    q = w.total_tokens * w.num_q_heads * w.head_dim * elt
    out = w.total_tokens * w.num_q_heads * w.head_dim * 4
    return kv + q + out


def settle(fn, ms: float = 100.0, cap: int = 3000):
    """Run ``fn`` untimed for about ``ms`` milliseconds: the GPU's clocks ramp up over the
    first tens of milliseconds of load (a 33-launch batch of 0.2 ms decodes measures 20 %
    slower at first than at steady state), so every timed region starts after this."""
    import torch
    fn()  # the first call may also load code objects
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    once = max(time.perf_counter() - t0, 1e-5)
    for _ in range(min(cap, max(10, int(ms * 1e-3 / once)))):
        fn()
    torch.cuda.synchronize()


def block_manager_timing(w, steps: int = 32):
    """Host bookkeeping of one decode step with the native block manager (include/pa_blocks.h):
    every sequence of the workload appends one token (growth, copy-on-write check, slot), then
    the batch's block tables are exported.  The manager gets the workload's pool size or, where
    that pool is full already (the 70B-shaped batch fills every block), the blocks its
    sequences reach after the appended tokens plus the null block."""
    import paged_kv_cache_121_amd as pa
    lens = w.steps[0].context_lens
    S, B = len(lens), w.block_size
    need = int(sum(-(-(int(L) + steps) // B) for L in lens)) + 1
    bm = pa.pa_bm_create(max(w.num_blocks, need), B, reserve_null_block=True)
    seqs = np.array([pa.pa_bm_add_sequence(bm) for _ in range(S)], dtype=np.int64)
    for i, L in enumerate(lens):
        pa.pa_bm_allocate_prompt(bm, int(seqs[i]), int(L) - 1)
    width = -(-(int(lens.max()) + steps) // B)
    t0 = time.perf_counter()
    for _ in range(steps):
        pa.pa_bm_append_tokens(bm, seqs)
    t_append = (time.perf_counter() - t0) / steps
    t0 = time.perf_counter()
    for _ in range(steps):
        pa.pa_bm_block_tables(bm, seqs, width)
    t_tables = (time.perf_counter() - t0) / steps
    pa.pa_bm_destroy(bm)
    return {"sequences": S, "append_step_us": round(t_append * 1e6, 1),
            "append_ns_per_sequence": round(t_append * 1e9 / S, 1),
            "tables_export_us": round(t_tables * 1e6, 1)}


def prefix_cache_timing(seed: int = 0):
    """The prefix-repetition run of the serving-stack page through the native manager: 64 prompts
    of a 4,000-token prefix plus 100 private tokens, 16 in flight, 64 answer tokens each, in a
    38,348-block pool of 16-token blocks.  Reports the host cost of prefix-cached admission
    (chained SHA-256 over the prompt's blocks, lookup, touch, allocation), the peak blocks in use
    and the tokens that had to be computed."""
    import paged_kv_cache_121_amd as pa
    rng = np.random.default_rng(seed)
    nblocks, B, conc, prompts, out_len = 38348, 16, 16, 64, 64
    shared = rng.integers(0, 1 << 17, 4000).astype(np.int32)
    bm = pa.pa_bm_create(nblocks, B, reserve_null_block=True)
    peak = missed = total = 0
    t_admit = []
    t_step = []
    for wave in range(prompts // conc):
        running = []
        for _ in range(conc):
            toks = np.concatenate([shared, rng.integers(0, 1 << 17, 100).astype(np.int32)])
            sid = pa.pa_bm_add_sequence(bm)
            t0 = time.perf_counter()
            hit = pa.pa_bm_allocate_prompt_cached(bm, sid, toks)
            t_admit.append(time.perf_counter() - t0)
            missed += len(toks) - hit
            total += len(toks)
            running.append(sid)
        seqs = np.array(running, dtype=np.int64)
        for _ in range(out_len):
            new = rng.integers(0, 1 << 17, conc).astype(np.int32)
            t0 = time.perf_counter()
            pa.pa_bm_append_tokens(bm, seqs)
            for i, sid in enumerate(running):
                pa.pa_bm_commit_tokens(bm, sid, new[i:i + 1])
            t_step.append(time.perf_counter() - t0)
            peak = max(peak, nblocks - 1 - pa.pa_bm_num_free(bm))
        for sid in running:
            pa.pa_bm_free_sequence(bm, sid)
    toks = np.concatenate([shared, shared[:100]])
    t0 = time.perf_counter()
    reps = 20
    for _ in range(reps):
        pa.pa_bm_hash_blocks(toks, B)
    t_hash = (time.perf_counter() - t0) / reps
    pa.pa_bm_destroy(bm)
    t_admit = np.array(t_admit)
    return {"prompts": prompts, "in_flight": conc, "prompt_tokens": total, "computed_tokens": missed,
            "peak_blocks": peak, "peak_pct_of_pool": round(100 * peak / nblocks, 2),
            "admit_us_first_prompt": round(t_admit[0] * 1e6, 1),
            "admit_us_median": round(float(np.median(t_admit)) * 1e6, 1),
            "hash_4100_tokens_us": round(t_hash * 1e6, 1),
            "decode_step_bookkeeping_us": round(float(np.median(t_step)) * 1e6, 1)}


def _oracle_step_tasks(w, seqs):
    """The oracle's inputs for the step of workload ``w`` on sequences ``seqs``: each
    sequence's blocks as generated (the step's copy-on-write sources in place of their copies)
    with its new token's write to replay (``oracle.parallel.sequence_task``)."""
    from oracle.parallel import sequence_task
    st = w.steps[0]
    cow = dict(zip(st.cow_dst.tolist(), st.cow_src.tolist()))
    tasks = []
    for s in seqs:
        L = int(st.context_lens[s])
        row = np.array([cow.get(int(b), int(b)) for b in w.block_tables[s, :-(-L // w.block_size)]], dtype=np.int64)
        mine = np.nonzero(st.write_seq == s)[0]
        tasks.append(sequence_task(w.pool, row, L, st.q[s], float(w.scale),
                                   (st.write_pos[mine], st.k_new[mine], st.v_new[mine])))
    return tasks


def cpu_baseline(w, n_seqs: int, got=None):
    """The float64 oracle doing the step (cache write, then decode, every query head) on the
    host's cores: (1) one thread on the first ``n_seqs`` sequences, (2) every sequence of the
    step in a pool of worker processes, one BLAS thread each, on up to 16 of the cores this
    process may use.  Each sequence's blocks are taken out of the generated pool (copy-on-write
    sources included), its new token written, its query heads decoded.  With ``got`` (the GPU's
    output of the same step) every computed row is compared."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.parallel import host_cores, run_task, run_tasks, worker_pool
    st = w.steps[0]
    elt = w.elem_bytes
    kv_of = [int(st.context_lens[s]) * 2 * w.num_kv_heads * w.head_dim * elt for s in range(w.num_seqs)]
    blas = [{"api": d.get("internal_api"), "threads": d.get("num_threads")} for d in threadpool_info()]
    err = 0.0
    # (1) one thread
    sel = list(range(min(n_seqs, w.num_seqs)))
    tasks = _oracle_step_tasks(w, sel)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        res1 = [run_task(t) for t in tasks]
        dt1 = time.perf_counter() - t0
    kv1 = sum(kv_of[s] for s in sel)
    # (2) every sequence, all cores (pool started before the clock: process start-up is not oracle work)
    cores = host_cores()
    workers = min(cores, 16)
    tasks = _oracle_step_tasks(w, range(w.num_seqs))
    with worker_pool(workers) as ex:
        run_tasks(tasks[:workers], pool=ex)  # every worker up and its imports done
        t0 = time.perf_counter()
        res = run_tasks(tasks, pool=ex)
        dtn = time.perf_counter() - t0
    kvn = sum(kv_of)
    if got is not None:
        for s, want in enumerate(res):
            err = max(err, float(np.abs(got[s].astype(np.float64) - want).max()))
        for s, want in zip(sel, res1):
            assert np.array_equal(want, res[s])
    return {"value": kvn / dtn / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"float64 oracle step (cache write + decode, all {w.num_q_heads} query heads) of all "
                      f"{w.num_seqs} sequences of the same workload ({kvn / 1e9:.3f} GB of KV) in {dtn:.1f} s on "
                      f"{workers} worker processes, one BLAS thread each",
            "host_cores_available": cores, "blas_threads_main_process": blas,
            "seq_layers_per_s": w.num_seqs / dtn,
            "single_thread": {"value": kv1 / dt1 / 1e9, "unit": "GB/s", "cores": 1,
                              "sample": f"sequences 0-{len(sel) - 1}: {kv1 / 1e9:.3f} GB of KV in {dt1:.1f} s",
                              "seq_layers_per_s": len(sel) / dt1},
            "rows_compared": w.num_seqs * w.num_q_heads if got is not None else 0,
            "max_abs_err_vs_gpu": err if got is not None else None}


def read_ceiling(dev, total_bytes: int = 1 << 30, reps: int = 20, seed: int = 0):
    """HBM read rate of a ``total_bytes`` buffer read once, in order and in randomly placed
    pieces of 4, 16 and 64 KiB (read_probe.hip: the decode kernel's 16-byte non-temporal loads,
    1 KiB per wavefront load), best over a sweep of grid sizes and loads in flight.  The decode
    of a paged cache reads 4 KiB (block, head) tiles of randomly placed blocks, so the random
    4 KiB rate is its practical ceiling; HIP events over ``reps`` launches after a settle.
    ``in_order_lds_dma``: the in-order read through direct-to-LDS loads (global_load_lds,
    the prefill's load path), 2-8 chunks in flight per wave."""
    import ctypes

    import torch
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m paged_kv_cache_121_amd.build)")
    lib = ctypes.CDLL(path)
    lib.pa_probe_read.restype = ctypes.c_int
    lib.pa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.empty(total_bytes, dtype=torch.uint8, device=dev)
    grids, unrolls = (512, 1024, 2048, 4096), (1, 2, 4, 8)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator().manual_seed(seed)
    out = {}
    for label, piece, shuffled in (("in_order", 65536, False), ("random_4KiB", 4096, True),
                                   ("random_16KiB", 16384, True), ("random_64KiB", 65536, True)):
        n = total_bytes // piece
        order = (torch.randperm(n, generator=g) if shuffled else torch.arange(n)).to(torch.int32).to(dev)
        rates = {}
        for grid in grids:
            for u in unrolls:
                def run():
                    rc = lib.pa_probe_read(ctypes.c_void_p(buf.data_ptr()), piece, ctypes.c_void_p(order.data_ptr()),
                                           n, grid, u, ctypes.c_void_p(sink.data_ptr()),
                                           ctypes.c_void_p(stream.cuda_stream))
                    assert rc == 0, rc
                settle(run, ms=20.0)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    run()
                e1.record(stream)
                torch.cuda.synchronize()
                rates[f"grid{grid}_x{u}"] = total_bytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
        best = max(rates, key=rates.get)
        out[label] = {"piece_bytes": piece, "best_gbs": round(rates[best], 1),
                      "pct_hbm_peak": round(100 * rates[best] / HBM_PEAK_GBS, 2), "best_launch": best,
                      "all_gbs": {k: round(v, 1) for k, v in rates.items()}}
    # the same in-order read through direct-to-LDS loads (the prefill's path)
    lib.pa_probe_read_lds.restype = ctypes.c_int
    lib.pa_probe_read_lds.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    rates = {}
    for grid in (256, 512, 1024, 2048):
        for u in (2, 4, 8):
            def run_lds():
                rc = lib.pa_probe_read_lds(ctypes.c_void_p(buf.data_ptr()), total_bytes, grid, u,
                                           ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
                assert rc == 0, rc
            settle(run_lds, ms=20.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                run_lds()
            e1.record(stream)
            torch.cuda.synchronize()
            rates[f"grid{grid}_x{u}"] = total_bytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    best = max(rates, key=rates.get)
    out["in_order_lds_dma"] = {"piece_bytes": total_bytes, "best_gbs": round(rates[best], 1),
                               "pct_hbm_peak": round(100 * rates[best] / HBM_PEAK_GBS, 2), "best_launch": best,
                               "all_gbs": {k: round(v, 1) for k, v in rates.items()}}
    del buf, sink
    torch.cuda.empty_cache()
    return {"bytes": total_bytes, "reps": reps, **out}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_cpu_baseline(w, got, rows: int = 12):
    """The float64 oracle on a bounded sample of the prefill: ``rows`` query rows of the
    first sequence, evenly spread, all heads, one thread; compared with the GPU's rows."""
    from threadpoolctl import threadpool_limits

    from oracle import paged
    n = int(w.query_start_loc[1])
    ctx = int(w.context_lens[0])
    nb = -(-ctx // w.block_size)
    pick = sorted(set(np.linspace(0, n - 1, num=min(rows, n)).astype(int).tolist()))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        small = w.pool[w.block_tables[0, :nb]].copy()
        tbl = np.arange(nb, dtype=np.int32)[None, :]
        sl = paged.slot_mapping_ref(tbl, np.zeros(n, dtype=np.int32), w.write_pos[:n], w.block_size)
        small = paged.cache_write_ref(small, w.k_new[:n], w.v_new[:n], sl)
        err = 0.0
        keys = 0
        for i in pick:
            want = paged.prefill_ref(small, w.q[i:i + 1], [0, 1], [ctx - n + i + 1], tbl, float(w.scale))
            err = max(err, float(np.abs(got[i].astype(np.float64) - want[0]).max()))
            keys += ctx - n + i + 1
        dt = time.perf_counter() - t0
    flops = 4 * w.head_dim * w.num_q_heads * keys
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 oracle prefill of {len(pick)} rows of sequence 0 (all {w.num_q_heads} heads, "
                      f"{keys} visible keys in all), one thread, {dt:.1f} s",
            "max_abs_err_vs_gpu": err}


def prefill_measurement(k: int, dev, reps: int = 20, warmup: int = 3, cpu: bool = True):
    """Time pa_prefill on prefill workload k (chunk K/V written first by pa_cache_write).

    Algorithmic work = the causal attention's multiply-adds: 4 * D * Hq flops
    per (query row, visible key); the row sums the kernel forms on the matrix
    cores and the masked halves of diagonal tiles are overhead, not work."""
    import torch

    import paged_kv_cache_121_amd as pa
    from workloads import PREFILL_NAMES, make_prefill
    w = make_prefill(k)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    pool = pa.PagedKVPool(bf(w.pool))
    tables = i32(w.block_tables)
    slots = pa.pa_slot_mapping(pool, tables, i32(w.write_seq), i32(w.write_pos))
    kn, vn = bf(w.k_new), bf(w.v_new)
    pa.pa_cache_write(pool, kn, vn, slots)
    q, qsl, lens = bf(w.q), i32(w.query_start_loc), i32(w.context_lens)
    mq = int(np.diff(w.query_start_loc).max())
    out = torch.empty((w.total_tokens, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)

    def run():
        pa.pa_prefill(pool, q, qsl, lens, tables, scale=float(w.scale), max_query_len=mq, out=out)

    settle(run)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = w.attention_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    base = prefill_cpu_baseline(w, out.cpu().numpy()) if cpu else None
    return {"workload": f"prefill workload {k}: {PREFILL_NAMES[k]}", "tokens": w.total_tokens,
            "flops": flops, "us": round(ms * 1e3, 1), "tflops": round(tflops, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_prefill_traffic(k), "kernel": "prefill_kernel",
                         "algorithmic_flops_per_launch": flops,
                         "algorithmic_bytes_per_launch": prefill_algorithmic_bytes(w)},
            "cpu_baseline": base,
            "sampled_max_abs_err": base["max_abs_err_vs_gpu"] if base else None}


def block_size_sweep(dev, workloads=(2, 5), sizes=(4, 8, 16, 32, 64, 128), reps: int = 30, warmup: int = 3):
    """Decode time and memory waste against the block size (the pages' block-size trade-off).

    Each workload keeps its context lengths and its cache memory (613,568 token slots) and is
    stored at every block size; one cache write + decode step is warmed up, then decode alone
    is timed with events around each launch.  Waste = slots reserved in last blocks minus
    tokens; lookups = block-table entries the step reads."""
    import torch

    import paged_kv_cache_121_amd as pa
    from workloads import make_block_size_sweep
    rows = []
    for k in workloads:
        t0 = time.perf_counter()
        ref = None
        for w in make_block_size_sweep(k, sizes):
            B = w.block_size
            st = w.steps[0]

            def bf(a):
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

            def i32(a):
                return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

            pool = pa.PagedKVPool(bf(w.pool))
            del w.pool
            tables, lens, q = i32(w.block_tables), i32(st.context_lens), bf(st.q)
            slots = pa.pa_slot_mapping(pool, tables, i32(st.write_seq), i32(st.write_pos))
            pa.pa_cache_write(pool, bf(st.k_new), bf(st.v_new), slots)
            max_len = int(st.context_lens.max())
            part = pa.pa_decode_partition_size(pool, w.num_seqs, w.num_q_heads, max_len)
            out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
            nbytes = pa.pa_decode_workspace_size(pool, w.num_seqs, w.num_q_heads, max_len, part)
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

            def decode():
                pa.pa_decode(pool, q, tables, lens, scale=float(w.scale), max_context_len=max_len,
                             partition_size=part, out=out, workspace=ws)

            settle(decode)
            for _ in range(warmup):
                decode()
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream(dev)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in ev:
                a.record(stream)
                decode()
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
            got = out.cpu().numpy()
            if not np.isfinite(got).all():
                print(f"[bench] NON-FINITE OUTPUT at B={B}", file=sys.stderr)
                sys.exit(1)
            # every block size holds the same tokens: outputs agree up to summation order
            ref = got if ref is None else ref
            diff = float(np.abs(got - ref).max())
            if not diff <= 1e-4:
                print(f"[bench] BLOCK SIZE {B} DISAGREES with B={sizes[0]}: {diff}", file=sys.stderr)
                sys.exit(1)
            L = st.context_lens.astype(np.int64)
            blocks = -(-L // B)
            kv = w.kv_bytes(0)
            gbs = kv / (ms * 1e-3) / 1e9
            rows.append({"workload": k, "block_size": B, "num_seqs": w.num_seqs, "context_tokens": int(L.sum()),
                         "partition_size": part, "decode_us": round(ms * 1e3, 2), "decode_gbs": round(gbs, 1),
                         "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                         "table_lookups": int(blocks.sum()), "reserved_slots": int((blocks * B).sum()),
                         "wasted_slots": int((blocks * B - L).sum()),
                         "waste_pct": round(100 * float((blocks * B - L).sum()) / float((blocks * B).sum()), 3),
                         f"max_abs_diff_vs_B{sizes[0]}": diff})
            print(f"[bench] block-size sweep: workload {k} B={B}: {rows[-1]['decode_us']} us "
                  f"({rows[-1]['pct_hbm_peak']} % of peak), built in {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
            del pool, tables, lens, q, out, ws, slots, w
            torch.cuda.empty_cache()
            t0 = time.perf_counter()
    return rows


def d2d_copy_gbs(dev, nbytes: int = 2 << 30, reps: int = 10):
    """A plain device-to-device copy of ``nbytes`` (torch's copy kernel): bytes read / time,
    the practical streaming rate beside the 8 TB/s peak (each byte is also written)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    del a, b
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "read_gbs": round(nbytes / t / 1e9, 1), "read_plus_write_gbs": round(2 * nbytes / t / 1e9, 1)}


def unique_kv_bytes(w, k: int) -> int:
    """K/V bytes of the distinct physical slots step k's decode reads: a block shared by
    several sequences (a common prefix) counts once, with the most tokens any of its readers
    uses (a sequence uses a block's slots from offset 0).  Equal to the logical bytes when no
    block is shared."""
    st = w.steps[k]
    B = w.block_size
    used = {}
    for s in range(w.num_seqs):
        L = int(st.context_lens[s])
        nb = -(-L // B)
        for j, b in enumerate(w.block_tables[s, :nb].tolist()):
            n = B if j < nb - 1 else L - (nb - 1) * B
            used[b] = max(used.get(b, 0), n)
    return sum(used.values()) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes


def other_workloads(dev, ks=(3, 4, 5, "4tp8"), reps: int = 20, check: bool = True):
    """Every step of workloads 3-5 in turn (copy-on-write copies, slot mapping and cache write
    in one launch, decode) and decode alone on step 0: HIP-event times, KV GB/s and % of peak.
    With ``check``, step 0's output (every row) is compared with the float64 oracle run on
    up to 16 worker processes, whose time is reported beside it.
    Output and workspace are allocated once, and the decode-only launches run back to back
    between one pair of events (a call of 30 us is otherwise timed with the binding's per-call
    host work in it).  "4tp8" is one GPU's share of workload 4 under 8-way tensor parallelism
    over heads (1 KV head, 8 query heads, the same sequences): the shape one GPU of a sharded
    70B layer runs."""
    import torch

    import paged_kv_cache_121_amd as pa
    from workloads import CONFIG_NAMES, make_config, make_tp_share
    out = {}
    for k in ks:
        t0 = time.perf_counter()
        w = make_tp_share(8) if k == "4tp8" else make_config(k)
        bf = w.dtype == "bf16"

        def d(a):
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf else np.ascontiguousarray(a))
            return (t.view(torch.bfloat16) if bf else t).to(dev)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

        pool = pa.PagedKVPool(d(w.pool))
        unique_kv = unique_kv_bytes(w, 0)
        tables = i32(w.block_tables)
        keep = bool(w.meta.get("prefix_tokens"))
        steps = []
        for st in w.steps:
            steps.append((i32(st.cow_src), i32(st.cow_dst), i32(st.write_seq), i32(st.write_pos), d(st.k_new),
                          d(st.v_new), d(st.q), i32(st.context_lens), int(st.context_lens.max()), len(st.cow_src)))
        stream = torch.cuda.current_stream(dev)
        out_buf = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
        need = max(pa.pa_decode_workspace_size(pool, w.num_seqs, w.num_q_heads, int(st.context_lens.max()))
                   for st in w.steps)
        work = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

        def run(i, decode_only=False):
            cs, cd, ws, wp, kn, vn, q, lens, mx, ncow = steps[i]
            if not decode_only:
                if ncow:
                    pa.pa_block_copy(pool, cs, cd)
                pa.pa_cache_write_at(pool, kn, vn, tables, ws, wp)
            return pa.pa_decode(pool, q, tables, lens, scale=float(w.scale), max_context_len=mx, keep_cached=keep,
                                out=out_buf, workspace=work)

        # warm-up: every kernel loaded and the clocks up (a step repeated writes the same values)
        settle(lambda: run(0))
        # the workload's steps in order; a one-step workload repeats its step (same writes)
        order = list(range(len(steps))) if len(steps) > 1 else [0] * reps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in order:
            o = run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / len(order)
        if not torch.isfinite(o).all():
            print(f"[bench] NON-FINITE OUTPUT in workload {k}", file=sys.stderr)
            sys.exit(1)
        settle(lambda: run(0, True), ms=30.0)
        e0.record(stream)
        for _ in range(reps):
            run(0, True)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        kv = w.kv_bytes(0)
        # step 0's output again (later steps write only positions step 0 does not read), against
        # the oracle on every sequence
        oracle = None
        if check:
            from oracle.parallel import host_cores, run_tasks, worker_pool
            got0 = run(0, True).cpu().numpy()
            workers = min(host_cores(), 16)
            tasks = _oracle_step_tasks(w, range(w.num_seqs))
            with worker_pool(workers) as ex:
                t1 = time.perf_counter()
                want = run_tasks(tasks, pool=ex)
                t_or = time.perf_counter() - t1
            err = max(float(np.abs(got0[s].astype(np.float64) - wv).max()) for s, wv in enumerate(want))
            if not err <= 2e-3:
                print(f"[bench] PARITY FAILURE in workload {k}: max abs err {err}", file=sys.stderr)
                sys.exit(1)
            oracle = {"rows": w.num_seqs * w.num_q_heads, "max_abs_err": err, "oracle_s": round(t_or, 2),
                      "cores": workers, "kind": "float64 oracle, step 0, every sequence (worker start-up excluded)"}
            del tasks, want
        del w.pool
        name = (CONFIG_NAMES[4] + "; one GPU's share at 8-way tensor parallelism: 1 KV head, 8 query heads"
                if k == "4tp8" else CONFIG_NAMES[k])
        out[f"workload{k}"] = {"workload": name, "steps": len(steps), "timed_steps": len(order),
                               "step_us": round(ms_step * 1e3, 2),
                               "decode_us": round(ms * 1e3, 2), "kv_bytes": kv,
                               "decode_gbs": round(kv / ms / 1e6, 1),
                               "pct_hbm_peak": round(100 * kv / ms / 1e6 / HBM_PEAK_GBS, 2),
                               "kv_cache_policy": "keep cached" if keep else "stream",
                               "unique_kv_bytes": unique_kv,
                               "decode_gbs_unique": round(unique_kv / ms / 1e6, 1),
                               "pct_hbm_peak_unique": round(100 * unique_kv / ms / 1e6 / HBM_PEAK_GBS, 2),
                               "partition_size": pa.pa_decode_partition_size(pool, w.num_seqs, w.num_q_heads,
                                                                             steps[0][8]),
                               "oracle_check": oracle}
        print(f"[bench] workload {k}: decode {out[f'workload{k}']['decode_us']} us "
              f"({out[f'workload{k}']['pct_hbm_peak']} %), step {out[f'workload{k}']['step_us']} us, "
              f"{time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
        del pool, tables, steps, w
        torch.cuda.empty_cache()
    return out


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def swap_measurement(dev, total_mib: int = 512, sizes=(4, 16, 128), reps: int = 5, dma_blocks: int = 1024):
    """Swap-out (device -> pinned host) and swap-in of ``total_mib`` MiB of blocks of a
    Qwen3-8B layer (8 KV heads, D128, bf16) at several block sizes.

    kernel: one pa_swap_blocks launch over every (scattered) pair.  per-block DMA: one
    copy per block (a transfer per block, as a copy engine would be driven), timed on
    ``dma_blocks`` blocks and scaled.  contiguous DMA: one copy of the same bytes in one
    piece, the host link's practical ceiling."""
    import torch

    import paged_kv_cache_121_amd as pa
    rows = []
    stream = torch.cuda.current_stream(dev)
    for B in sizes:
        block_bytes = 2 * 8 * B * 128 * 2
        n = total_mib * 2**20 // block_bytes
        devpool = pa.PagedKVPool(torch.randn((2 * n, 2, 8, B, 128), device=dev).to(torch.bfloat16))
        host = pa.HostKVPool.empty(n, 8, B, 128, torch.bfloat16)
        g = torch.randperm(2 * n, device=dev)[:n].to(torch.int32)   # scattered device blocks
        h = torch.randperm(n, device=dev).to(torch.int32)

        def timed(fn, k=reps):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(k):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / k * 1e-3

        t_out = timed(lambda: pa.pa_swap_blocks(devpool, host, g, h))
        t_in = timed(lambda: pa.pa_swap_blocks(host, devpool, h, g))
        ok = torch.equal(devpool.data[g.long()].view(torch.int16).cpu(), host.data[h.long().cpu()].view(torch.int16))
        m = min(dma_blocks, n)
        gl, hl = g[:m].tolist(), h[:m].tolist()

        def per_block():
            for i in range(m):
                host.data[hl[i]].copy_(devpool.data[gl[i]], non_blocking=True)

        t_pb = timed(per_block, 1) * n / m
        t_contig = timed(lambda: host.data.copy_(devpool.data[:n], non_blocking=True))
        nbytes = n * block_bytes
        rows.append({"block_size": B, "block_bytes": block_bytes, "blocks": n, "bytes": nbytes,
                     "kernel_out_gbs": round(nbytes / t_out / 1e9, 2), "kernel_in_gbs": round(nbytes / t_in / 1e9, 2),
                     "per_block_dma_out_gbs": round(nbytes / t_pb / 1e9, 2),
                     "contiguous_dma_out_gbs": round(nbytes / t_contig / 1e9, 2), "bit_exact": bool(ok)})
        print(f"[bench] swap B={B}: kernel out {rows[-1]['kernel_out_gbs']} GB/s, in {rows[-1]['kernel_in_gbs']} "
              f"GB/s; per-block DMA {rows[-1]['per_block_dma_out_gbs']} GB/s; contiguous "
              f"{rows[-1]['contiguous_dma_out_gbs']} GB/s", file=sys.stderr, flush=True)
        if not ok:
            print(f"[bench] SWAP COPY MISMATCH at B={B}", file=sys.stderr)
            sys.exit(1)
        del devpool, host, g, h
        torch.cuda.empty_cache()
    best = max(rows, key=lambda r: r["kernel_out_gbs"])
    return {"sweep": rows,
            "roofline": {"bound": "pcie", "achieved": best["kernel_out_gbs"], "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                         "frac": round(best["kernel_out_gbs"] / PCIE_PEAK_GBS, 4), "traffic": None,
                         "kernel": "block_copy_kernel (device -> pinned host)"}}


def calibrate_copy(pairs: int, dev):
    """pa_block_copy of ``pairs`` distinct 64 KiB blocks (bf16, 8 KV heads, B16, D128):
    reads and writes exactly pairs * 65536 bytes per launch."""
    import torch

    import paged_kv_cache_121_amd as pa
    pool = pa.PagedKVPool(torch.zeros((2 * pairs, 2, 8, 16, 128), dtype=torch.bfloat16, device=dev))
    src = torch.arange(0, pairs, dtype=torch.int32, device=dev)
    dst = torch.arange(pairs, 2 * pairs, dtype=torch.int32, device=dev)
    for _ in range(5):
        pa.pa_block_copy(pool, src, dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_pairs": pairs, "bytes_read_per_launch": pairs * 65536,
                      "bytes_written_per_launch": pairs * 65536}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by sequence or KV head with no exchange step); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_121_amd as pa
    from workloads import CONFIG_NAMES, make_config, make_tp_share

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, dev)
        return
    if args.read_ceiling:
        r = read_ceiling(dev)
        print(json.dumps({"metric": "HBM read GB/s by access pattern (decode roofline reference)", "unit": "GB/s",
                          "n_gpus": 1, "higher_is_better": True, "data": "1 GiB device buffer", **r}), flush=True)
        return
    if args.swap:
        r = swap_measurement(dev)
        print(json.dumps({"metric": "swap copy GB/s (device <-> pinned host)", "unit": "GB/s", "n_gpus": 1,
                          "higher_is_better": True, "dtype": "bf16 blocks", "data": "synthetic", **r}), flush=True)
        return
    if args.block_sweep:
        rows = block_size_sweep(dev, reps=args.decode_reps)
        print(json.dumps({"metric": "decode attention KV-read GB/s against block size", "unit": "GB/s",
                          "n_gpus": 1, "higher_is_better": True, "dtype": "bf16 K/V and Q, fp32 accumulate",
                          "data": "synthetic", "sweep": rows}), flush=True)
        return
    if args.prefill:
        r = prefill_measurement(args.prefill, dev, reps=args.steps, warmup=args.warmup,
                                cpu=not args.no_cpu_baseline)
        if r["sampled_max_abs_err"] is not None and not r["sampled_max_abs_err"] <= 2e-3:
            print(f"[bench] PREFILL PARITY FAILURE: {r['sampled_max_abs_err']}", file=sys.stderr)
            sys.exit(1)
        print(json.dumps({"metric": "prefill attention TFLOP/s", "value": r["tflops"], "unit": "TFLOP/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                          "dtype": "bf16 Q/K/V, fp32 accumulate", "data": "synthetic",
                          "config": {"workload": r["workload"], "tokens": r["tokens"]}, "us": r["us"],
                          "roofline": r["roofline"], "cpu_baseline": r["cpu_baseline"],
                          "sampled_max_abs_err": r["sampled_max_abs_err"]}), flush=True)
        return
    t_gen = time.perf_counter()
    w = make_tp_share(8) if args.workload == "4tp8" else make_config(int(args.workload))
    t_gen = time.perf_counter() - t_gen
    st = w.steps[0]
    print(f"[bench] workload {args.workload}: {w.name} generated in {t_gen:.1f} s", file=sys.stderr, flush=True)

    def dev_data(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def dev_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    pool = pa.PagedKVPool(dev_data(w.pool))
    tables = dev_i32(w.block_tables)
    lens = dev_i32(st.context_lens)
    q = dev_data(st.q)
    k_new, v_new = dev_data(st.k_new), dev_data(st.v_new)
    wseq, wpos = dev_i32(st.write_seq), dev_i32(st.write_pos)
    cow_src, cow_dst = dev_i32(st.cow_src), dev_i32(st.cow_dst)
    max_len = int(st.context_lens.max())
    part = args.partition_size or pa.pa_decode_partition_size(pool, w.num_seqs, w.num_q_heads, max_len)
    nbytes = pa.pa_decode_workspace_size(pool, w.num_seqs, w.num_q_heads, max_len, part)
    workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    slots = torch.empty(len(st.write_seq), dtype=torch.int64, device=dev)
    scale = float(w.scale)
    torch.cuda.synchronize()

    keep_cached = bool(w.meta.get("prefix_tokens"))  # shared prefix blocks: keep K/V in L2

    def decode():
        pa.pa_decode(pool, q, tables, lens, scale=scale, max_context_len=max_len, partition_size=part,
                     out=out, workspace=workspace, keep_cached=keep_cached)

    def step():
        if len(st.cow_src):
            pa.pa_block_copy(pool, cow_src, cow_dst)
        pa.pa_cache_write_at(pool, k_new, v_new, tables, wseq, wpos, slots_out=slots)
        decode()

    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # decode-only launches, each bracketed by events on the stream it runs on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.decode_reps)]
    for a, b in ev:
        a.record(stream)
        decode()
        b.record(stream)
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    dec_avg_ms = float(dec_ms.mean())

    kv_bytes = w.kv_bytes(0)
    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    value = kv_bytes / (ms_step * 1e-3) / 1e9

    got = out.cpu().numpy()
    if not np.isfinite(got).all():
        print("[bench] NON-FINITE DECODE OUTPUT", file=sys.stderr)
        sys.exit(1)

    traffic = measured_traffic(args.workload, part)

    # the oracle runs only here: timed on a bounded sample, its rows checked against the GPU's
    cpu, check = None, None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seqs, None if args.skip_check else got)
        check = cpu["max_abs_err_vs_gpu"]
        if check is not None and not check <= 2e-3:
            print(f"[bench] PARITY FAILURE: max abs err {check}", file=sys.stderr)
            sys.exit(1)
    host_bm = block_manager_timing(w)
    d2d = d2d_copy_gbs(dev)
    ceiling = None if args.no_read_ceiling else read_ceiling(dev)
    others = None if args.no_other_workloads else other_workloads(dev, check=not args.no_cpu_baseline)
    host_prefix = prefix_cache_timing()
    prefill = None
    if not args.no_prefill:
        del pool, workspace, out, q
        torch.cuda.empty_cache()
        prefill = prefill_measurement(1, dev, cpu=not args.no_cpu_baseline)
        chunked = prefill_measurement(2, dev, cpu=False)
        # what the cache saves on the GPU: 16 requests attend 100 uncached rows each over
        # 4,100 keys instead of their whole 4,100-token prompts
        host_prefix["prefill_us_16_cached_chunks"] = chunked["us"]
        host_prefix["prefill_us_4_full_prompts"] = prefill["us"]

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16 K/V and Q, fp32 accumulate", "f32": "f32"}[w.dtype],
        "data": "synthetic (seeded N(0,1) K/V/Q; lengths, placement and sharing per the workload recipe)",
        "config": {
            "workload": f"workload {args.workload}: " + (
                CONFIG_NAMES[4] + "; one GPU's share at 8-way tensor parallelism: 1 KV head, 8 query heads"
                if args.workload == "4tp8" else CONFIG_NAMES[int(args.workload)]),
            "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "pool_blocks": w.num_blocks,
            "context_tokens": int(st.context_lens.sum()), "max_context_len": max_len,
            "partition_size": part, "kv_bytes_per_step": kv_bytes,
            "kv_cache_policy": "keep cached (shared blocks)" if keep_cached else "stream (non-temporal)",
        },
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_gbs": round(achieved, 1),
        "seq_layers_per_s": round(w.num_seqs / (dec_avg_ms * 1e-3), 1),
        "step_seq_layers_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_kernel", "algorithmic_bytes_per_launch": kv_bytes},
        "cpu_baseline": cpu,
        "d2d_copy": d2d,
        "read_ceiling": ceiling,
        "other_workloads": others,
        "block_manager": host_bm,
        "prefix_cache": host_prefix,
        "prefill": prefill,
        "sampled_max_abs_err": check,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
