"""Prefix caching end to end on the GPU: cached blocks stand in for recomputation.

Requests with a common prefix go through the native block manager's
prefix-cached allocation; only their uncached tokens are written
(pa_slot_mapping + pa_cache_write) and attended (pa_prefill), in one batch,
and later decode steps (pa_bm_append_tokens + pa_decode) read the shared
blocks.  K/V/Q depend only on (token id, position), so the oracle checks
every row against attention over the request's whole prompt written into a
private pool, i.e. against computing everything again.  Bar: 2e-3 max-abs.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_121_amd as pa
from oracle import paged
from workloads import make_token_model

from _gpu_util import DEV, i32, say, to_dev

pytestmark = pytest.mark.gpu

ATOL = 2e-3
B = 16
HQ, HKV, D = 32, 8, 128
SCALE = float(np.float32(1.0) / np.sqrt(np.float32(D)))


def private_pool(tm, toks):
    """The oracle's own pool: every token of ``toks`` written into blocks 0.. of a private table."""
    n = len(toks)
    nb = -(-n // B)
    pool = np.full((nb, 2, HKV, B, D), 0x7FC0, dtype=np.uint16)
    _, k, v = tm.qkv(toks, np.arange(n))
    table = np.arange(nb, dtype=np.int32)[None, :]
    slots = paged.slot_mapping_ref(table, np.zeros(n, dtype=np.int32), np.arange(n, dtype=np.int32), B)
    return paged.cache_write_ref(pool, k, v, slots), table


def oracle_rows(tm, toks, first):
    """Attention of positions first..n-1 of ``toks`` over the whole recomputed prompt."""
    pool, table = private_pool(tm, toks)
    n = len(toks)
    q, _, _ = tm.qkv(toks[first:], np.arange(first, n))
    return paged.prefill_ref(pool, q, [0, n - first], [n], table, SCALE)


class Engine:
    """Block manager + device pool: the steps a serving loop would take, in the library's calls."""

    def __init__(self, tm, num_blocks):
        self.tm = tm
        self.bm = pa.pa_bm_create(num_blocks, B, True)
        self.pool = pa.PagedKVPool(torch.full((num_blocks, 2, HKV, B, D), float("nan"), dtype=torch.bfloat16,
                                              device=DEV))
        self.tokens = {}

    def tables(self, sids, width):
        return pa.pa_bm_block_tables(self.bm, sids, width, pad_value=0)

    def prefill(self, prompts):
        """Admit prompts together; write and attend only their uncached tokens."""
        sids, cached = [], []
        for toks in prompts:
            sid = pa.pa_bm_add_sequence(self.bm)
            cached.append(pa.pa_bm_allocate_prompt_cached(self.bm, sid, toks))
            sids.append(sid)
            self.tokens[sid] = list(toks)
        width = max(-(-len(t) // B) for t in prompts) + 8
        tables, lens = self.tables(sids, width)
        seq_idx, pos, ids = [], [], []
        for s, (toks, c) in enumerate(zip(prompts, cached)):
            seq_idx += [s] * (len(toks) - c)
            pos += list(range(c, len(toks)))
            ids += toks[c:]
        q, k, v = self.tm.qkv(ids, pos)
        tdev = i32(tables)
        slots = pa.pa_slot_mapping(self.pool, tdev, i32(seq_idx), i32(pos))
        pa.pa_cache_write(self.pool, to_dev(k, "bf16"), to_dev(v, "bf16"), slots)
        qsl = np.zeros(len(prompts) + 1, dtype=np.int32)
        qsl[1:] = np.cumsum([len(t) - c for t, c in zip(prompts, cached)])
        out = pa.pa_prefill(self.pool, to_dev(q, "bf16"), i32(qsl), i32(lens), tdev, scale=SCALE,
                            max_query_len=int(np.diff(qsl).max()))
        torch.cuda.synchronize()
        return sids, cached, tables, qsl, out.cpu().numpy()

    def decode(self, sids, new_ids):
        """One decode step: append a token per sequence, write its K/V, attend."""
        slots, src, dst = pa.pa_bm_append_tokens(self.bm, sids)
        if len(src):
            pa.pa_block_copy(self.pool, i32(src), i32(dst))
        for sid, t in zip(sids, new_ids):
            pa.pa_bm_commit_tokens(self.bm, sid, [t])
            self.tokens[sid].append(t)
        pos = [len(self.tokens[s]) - 1 for s in sids]
        q, k, v = self.tm.qkv(new_ids, pos)
        pa.pa_cache_write(self.pool, to_dev(k, "bf16"), to_dev(v, "bf16"),
                          torch.from_numpy(slots.astype(np.int64)).to(DEV))
        width = max(-(-len(self.tokens[s]) // B) for s in sids)
        tables, lens = self.tables(sids, width)
        out = pa.pa_decode(self.pool, to_dev(q, "bf16"), i32(tables), i32(lens), scale=SCALE,
                           max_context_len=int(lens.max()), keep_cached=True)
        torch.cuda.synchronize()
        return out.cpu().numpy()


def test_prefix_cached_batch_equals_recomputation():
    rng = np.random.default_rng(77)
    tm = make_token_model(300, vocab=512, max_pos=1024, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)
    eng = Engine(tm, 192)
    shared = [int(t) for t in rng.integers(0, 512, 500)]
    a = shared + [int(t) for t in rng.integers(0, 512, 37)]
    b = shared + [int(t) for t in rng.integers(0, 512, 45)]
    c = list(a)                      # the whole of a again: the hit stops before its last token
    d = shared[:480]                 # block-aligned prompt made of cached blocks: its last block is recomputed
    prompts = [a, b, c, d]
    say("[prefix cached prefill] 4 prompts sharing 500 tokens")
    sids, cached, tables, qsl, got = eng.prefill(prompts)
    assert cached == [0, 496, 528, 464]
    assert (tables[1, :31] == tables[0, :31]).all() and tables[1, 31] != tables[0, 31]
    errs = []
    for s, toks in enumerate(prompts):
        want = oracle_rows(tm, toks, cached[s])
        errs.append(np.abs(got[qsl[s]:qsl[s + 1]] - want).max())
    say(f"    max abs err per request {[f'{e:.2e}' for e in errs]}")
    assert max(errs) <= ATOL

    say("[prefix cached decode] 3 steps over the shared blocks")
    for _ in range(3):
        new = [int(t) for t in rng.integers(0, 512, len(sids))]
        got = eng.decode(sids, new)
        for s, sid in enumerate(sids):
            toks = eng.tokens[sid]
            want = oracle_rows(tm, toks, len(toks) - 1)[0]
            assert np.abs(got[s] - want).max() <= ATOL
    for sid in sids:
        pa.pa_bm_free_sequence(eng.bm, sid)
    pa.pa_bm_destroy(eng.bm)


def test_evicted_blocks_are_recomputed_not_reused():
    rng = np.random.default_rng(78)
    tm = make_token_model(301, vocab=512, max_pos=1024, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D)
    eng = Engine(tm, 48)                      # 47 usable blocks
    p = [int(t) for t in rng.integers(0, 512, 300)]
    say("[prefix eviction] cache, evict, recompute")
    sids, cached, _, _, _ = eng.prefill([p])
    pa.pa_bm_free_sequence(eng.bm, sids[0])
    assert pa.pa_bm_lookup_prefix(eng.bm, p) == 288
    # an unrelated request takes every free block: the cached blocks are overwritten
    other = [int(t) for t in rng.integers(0, 512, 47 * B)]
    osids, ocached, _, _, _ = eng.prefill([other])
    assert ocached == [0] and pa.pa_bm_lookup_prefix(eng.bm, p) == 0
    pa.pa_bm_free_sequence(eng.bm, osids[0])
    sids, cached, _, qsl, got = eng.prefill([p])
    assert cached == [0]
    want = oracle_rows(tm, p, 0)
    assert np.abs(got - want).max() <= ATOL
    # and again: now the prefix is cached and the tail row agrees with recomputation
    sids2, cached2, _, _, got2 = eng.prefill([p])
    assert cached2 == [288]
    assert np.abs(got2 - want[288:]).max() <= ATOL
    pa.pa_bm_destroy(eng.bm)
