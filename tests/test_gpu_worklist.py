"""The work-list decode (batches of 1,024 or more (sequence, KV head) pairs):
a prepass lists the (pair, partition) items that have work, longest first,
and a grid of resident workgroups walks the list.

Which workgroup computes an item does not change its arithmetic, so a batch
decoded through the list gives the same bits as the same sequences decoded
in small batches (one workgroup per (pair, partition), no list) with the same
partition size; and every row matches the float64 oracle.  Empty contexts
give zero rows and invalid ones NaN rows on this path too.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_121_amd as pa
from oracle import paged
from oracle.parallel import run_tasks, sequence_task
from workloads import make_custom

from _gpu_util import device_pool, i32, say, to_dev

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def skewed_lengths(S, seed):
    rng = np.random.default_rng(seed)
    lens = np.clip(np.round(rng.lognormal(np.log(300), 1.0, size=S)), 1, 6000).astype(np.int64)
    lens[::17] = 1
    return lens


@pytest.mark.parametrize("group,part", [(4, 512), (8, 1024), (1, 256)])
def test_work_list_matches_small_batches_and_oracle(group, part):
    S, hkv = 160, 8  # 1,280 pairs: the list path
    lens = skewed_lengths(S, 500 + group)
    w = make_custom(name="worklist", seed=510 + group, dtype="bf16",
                    num_blocks=int(sum(-(-int(L) // 16) for L in lens)) + 16, num_q_heads=hkv * group,
                    num_kv_heads=hkv, head_dim=128, block_size=16, lengths=lens)
    st = w.steps[0]
    pool = device_pool(w)
    slots = pa.pa_slot_mapping(pool, i32(w.block_tables), i32(st.write_seq), i32(st.write_pos))
    pa.pa_cache_write(pool, to_dev(st.k_new, w.dtype), to_dev(st.v_new, w.dtype), slots)
    q, tables, lens_d = to_dev(st.q, w.dtype), i32(w.block_tables), i32(st.context_lens)
    mcl = int(st.context_lens.max())
    need = pa.pa_decode_workspace_size(pool, S, w.num_q_heads, mcl, part)
    say(f"[worklist] G={group} S={S} pairs={S * hkv} partition={part} max len={mcl} workspace={need} B")
    got = pa.pa_decode(pool, q, tables, lens_d, scale=float(w.scale), max_context_len=mcl, partition_size=part)
    # the same sequences 48 at a time (384 pairs: one workgroup per item, no list)
    ref = torch.empty_like(got)
    for a in range(0, S, 48):
        b = min(S, a + 48)
        ref[a:b] = pa.pa_decode(pool, q[a:b].contiguous(), tables[a:b].contiguous(), lens_d[a:b].contiguous(),
                                scale=float(w.scale), max_context_len=mcl, partition_size=part)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "work-list and grid decodes differ"
    out = got.cpu().numpy()
    pool_np = paged.cache_write_ref(w.pool, st.k_new, st.v_new,
                                    paged.slot_mapping_ref(w.block_tables, st.write_seq, st.write_pos, 16))
    want = run_tasks(sequence_task(pool_np, w.block_tables[s], int(st.context_lens[s]), st.q[s], float(w.scale))
                     for s in range(S))
    err = max(float(np.abs(out[s].astype(np.float64) - wv).max()) for s, wv in enumerate(want))
    say(f"    bit-identical to small batches; every row vs oracle: max abs err {err:.3e}")
    assert err <= ATOL


def test_work_list_empty_and_invalid_contexts():
    S, hkv, group = 136, 8, 4  # 1,088 pairs
    lens = skewed_lengths(S, 520)
    w = make_custom(name="worklist-edge", seed=521, dtype="bf16",
                    num_blocks=int(sum(-(-int(L) // 16) for L in lens)) + 16, num_q_heads=hkv * group,
                    num_kv_heads=hkv, head_dim=128, block_size=16, lengths=lens, num_steps=1)
    st = w.steps[0]
    pool = device_pool(w)
    slots = pa.pa_slot_mapping(pool, i32(w.block_tables), i32(st.write_seq), i32(st.write_pos))
    pa.pa_cache_write(pool, to_dev(st.k_new, w.dtype), to_dev(st.v_new, w.dtype), slots)
    L = st.context_lens.copy()
    mcl = int(L.max())
    L[3] = 0            # empty: zero rows
    L[10] = mcl + 5     # beyond max_context_len: NaN rows
    L[20] = -2          # negative: NaN rows
    say(f"[worklist edge] S={S} pairs={S * hkv} lengths 0, >max, <0 among them")
    out = pa.pa_decode(pool, to_dev(st.q, w.dtype), i32(w.block_tables), i32(L), scale=float(w.scale),
                       max_context_len=mcl, partition_size=512).cpu().numpy()
    assert (out[3] == 0).all() and np.isnan(out[10]).all() and np.isnan(out[20]).all()
    pool_np = paged.cache_write_ref(w.pool, st.k_new, st.v_new,
                                    paged.slot_mapping_ref(w.block_tables, st.write_seq, st.write_pos, 16))
    rest = [s for s in range(S) if s not in (3, 10, 20)]
    want = run_tasks([sequence_task(pool_np, w.block_tables[s], int(L[s]), st.q[s], float(w.scale)) for s in rest])
    err = max(float(np.abs(out[s].astype(np.float64) - wv).max()) for s, wv in zip(rest, want))
    say(f"    other rows vs oracle: max abs err {err:.3e}")
    assert err <= ATOL
