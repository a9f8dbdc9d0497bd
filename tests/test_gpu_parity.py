"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: slot mapping, cache writes and block copies bit-exact over the whole
pool; decode outputs within max-abs 2e-3 of the float64 oracle (bf16 or
fp32 K/V, fp32 accumulation).  Reduced workloads keep each workload's
shapes and structure and are checked in full; every seeded case is named
on stderr before its GPU step.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_121_amd as pa
from oracle import paged
from workloads import make_config, make_custom

from _gpu_util import DEV, device_pool, i32, oracle_step, run_step, say, to_dev, to_host

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def decode_oracle(w, pool_np, k):
    st = w.steps[k]
    return paged.decode_ref(pool_np, st.q, w.block_tables, st.context_lens, float(w.scale))


# ------------------------------------------------------------------ slot mapping


def test_slot_mapping_bit_exact_including_out_of_range():
    w = make_config(2, small=True)
    say(f"[slot_mapping] {w.name}")
    pool = device_pool(w)
    tables = i32(w.block_tables)
    S, width = w.block_tables.shape
    rng = np.random.default_rng(21)
    seq = rng.integers(0, S, size=300).astype(np.int32)
    pos = rng.integers(0, width * w.block_size, size=300).astype(np.int32)
    # out-of-range tokens: bad sequence id, negative position, position past the row
    seq[:3] = [-1, S, 0]
    pos[3:6] = [-5, width * w.block_size, 10 ** 6]
    got = to_host(pa.pa_slot_mapping(pool, tables, i32(seq), i32(pos)))
    want = np.full(300, -1, dtype=np.int64)
    for i in range(300):
        if 0 <= seq[i] < S and 0 <= pos[i] < width * w.block_size:
            want[i] = paged.slot_mapping_ref(w.block_tables, [seq[i]], [pos[i]], w.block_size)[0]
    np.testing.assert_array_equal(got, want)


# ------------------------------------------------------------------ cache write and block copy


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_cache_write_bit_exact_whole_pool(k):
    w = make_config(k, small=True)
    say(f"[cache_write] {w.name}")
    pool = device_pool(w)
    tables = i32(w.block_tables)
    st = w.steps[0]
    if len(st.cow_src):
        pa.pa_block_copy(pool, i32(st.cow_src), i32(st.cow_dst))
    slots = pa.pa_slot_mapping(pool, tables, i32(st.write_seq), i32(st.write_pos))
    pa.pa_cache_write(pool, to_dev(st.k_new, w.dtype), to_dev(st.v_new, w.dtype), slots)
    torch.cuda.synchronize()
    want_slots, want_pool = oracle_step(w, w.pool, 0)
    np.testing.assert_array_equal(to_host(slots), want_slots)
    got = to_host(pool.data)
    assert got.tobytes() == want_pool.tobytes()


def test_cache_write_skips_negative_and_out_of_pool_slots():
    w = make_config(2, small=True)
    say("[cache_write skip] cfg2-small")
    pool = device_pool(w)
    rng = np.random.default_rng(22)
    n_slots = w.num_blocks * w.block_size
    slots = np.array([-1, 5, n_slots, n_slots + 77, 3 * 16 + 2, -9], dtype=np.int64)
    k = rng.standard_normal((6, 8, 128)).astype(np.float32)
    v = rng.standard_normal((6, 8, 128)).astype(np.float32)
    from workloads import to_bf16_bits
    k, v = to_bf16_bits(k), to_bf16_bits(v)
    pa.pa_cache_write(pool, to_dev(k, "bf16"), to_dev(v, "bf16"), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    keep = slots.copy()
    keep[(keep < 0) | (keep >= n_slots)] = -1
    want = paged.cache_write_ref(w.pool, k, v, keep)
    assert to_host(pool.data).tobytes() == want.tobytes()


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_cache_write_at_bit_exact_whole_pool(k):
    # slot computation and write in one launch: the same slots and the same pool as the oracle
    w = make_config(k, small=True)
    say(f"[cache_write_at] {w.name}")
    pool = device_pool(w)
    st = w.steps[0]
    if len(st.cow_src):
        pa.pa_block_copy(pool, i32(st.cow_src), i32(st.cow_dst))
    slots = torch.empty(len(st.write_pos), dtype=torch.int64, device=DEV)
    pa.pa_cache_write_at(pool, to_dev(st.k_new, w.dtype), to_dev(st.v_new, w.dtype), i32(w.block_tables),
                         i32(st.write_seq), i32(st.write_pos), slots_out=slots)
    torch.cuda.synchronize()
    want_slots, want_pool = oracle_step(w, w.pool, 0)
    np.testing.assert_array_equal(to_host(slots), want_slots)
    assert to_host(pool.data).tobytes() == want_pool.tobytes()


def test_cache_write_at_skips_tokens_out_of_range():
    # bad sequence ids, negative positions, positions past the table row and table entries
    # outside the pool get slot -1 and write nothing; the others land bit for bit
    w = make_config(2, small=True)
    say("[cache_write_at skip] cfg2-small")
    pool = device_pool(w)
    S, width = w.block_tables.shape
    tables = w.block_tables.copy()
    tables[4, 0] = w.num_blocks + 3
    rng = np.random.default_rng(23)
    seq = rng.integers(0, S, size=40).astype(np.int32)
    pos = rng.integers(0, width * w.block_size, size=40).astype(np.int32)
    seq[:4] = [-1, S, 0, 4]
    pos[:4] = [3, 3, -5, 2]          # token 3 lands in the invalid table entry of sequence 4
    pos[4] = width * w.block_size
    def slot_of(i):
        if 0 <= seq[i] < S and 0 <= pos[i] < width * w.block_size:
            if 0 <= int(tables[seq[i], pos[i] // w.block_size]) < w.num_blocks:
                return int(paged.slot_mapping_ref(tables, [seq[i]], [pos[i]], w.block_size)[0])
        return -1
    # one token per slot (table rows are padded with block 0, so distinct positions can share
    # one): drop later duplicates
    seen, keep = set(), []
    for i in range(40):
        sl = slot_of(i)
        if sl < 0 or sl not in seen:
            seen.add(sl)
            keep.append(i)
    want = np.array([slot_of(i) for i in keep], dtype=np.int64)
    seq, pos = seq[keep], pos[keep]
    n = len(keep)
    from workloads import to_bf16_bits
    kk = to_bf16_bits(rng.standard_normal((n, 8, 128)).astype(np.float32))
    vv = to_bf16_bits(rng.standard_normal((n, 8, 128)).astype(np.float32))
    got_slots = pa.pa_cache_write_at(pool, to_dev(kk, "bf16"), to_dev(vv, "bf16"), i32(tables), i32(seq), i32(pos),
                                     slots_out=torch.empty(n, dtype=torch.int64, device=DEV))
    pa.pa_cache_write_at(pool, to_dev(kk, "bf16"), to_dev(vv, "bf16"), i32(tables), i32(seq), i32(pos))  # no slots out
    torch.cuda.synchronize()
    assert (want[:5] == -1).all() and (want >= 0).sum() > 20
    np.testing.assert_array_equal(to_host(got_slots), want)
    assert to_host(pool.data).tobytes() == paged.cache_write_ref(w.pool, kk, vv, want).tobytes()


def test_block_copy_bit_exact_whole_pool():
    for k in (1, 2, 4):
        w = make_config(k, small=True)
        say(f"[block_copy] {w.name}")
        pool = device_pool(w)
        rng = np.random.default_rng(23 + k)
        ids = rng.permutation(w.num_blocks)
        n = min(12, (w.num_blocks - 1) // 2)
        src, dst = ids[:n].astype(np.int32), ids[n:2 * n].astype(np.int32)
        # one pair with an out-of-range id is skipped
        src_d = np.concatenate([src, [w.num_blocks]]).astype(np.int32)
        dst_d = np.concatenate([dst, [int(ids[2 * n])]]).astype(np.int32)
        pa.pa_block_copy(pool, i32(src_d), i32(dst_d))
        torch.cuda.synchronize()
        want = paged.block_copy_ref(w.pool, src, dst)
        assert to_host(pool.data).tobytes() == want.tobytes()


# ------------------------------------------------------------------ decode parity, reduced workloads


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("partition_size", [0, 64, 512])
def test_decode_step0_matches_oracle(k, partition_size):
    w = make_config(k, small=True)
    if partition_size % w.block_size:
        pytest.skip("partition must be whole blocks")
    say(f"[decode] {w.name} partition_size={partition_size}")
    pool = device_pool(w)
    _, out = run_step(w, pool, i32(w.block_tables), 0, partition_size=partition_size)
    torch.cuda.synchronize()
    _, pool_np = oracle_step(w, w.pool, 0)
    want = decode_oracle(w, pool_np, 0)
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= ATOL
    # the pool after the step also matches bit for bit
    assert to_host(pool.data).tobytes() == pool_np.tobytes()


def test_decode_every_step_of_the_growth_workload():
    w = make_config(5, small=True)
    say(f"[decode steps] {w.name} steps={len(w.steps)}")
    pool = device_pool(w)
    tables = i32(w.block_tables)
    pool_np = w.pool
    for k in range(len(w.steps)):
        _, out = run_step(w, pool, tables, k, partition_size=64)
        _, pool_np = oracle_step(w, pool_np, k)
        want = decode_oracle(w, pool_np, k)
        err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
        say(f"    step {k}: max abs err {err:.3e}")
        assert err <= ATOL
    assert to_host(pool.data).tobytes() == pool_np.tobytes()


# ------------------------------------------------------------------ invariants and closed forms


def _decode_custom(w, pool_np, tables, lens, q, partition_size=0, max_context_len=None, keep_cached=False):
    pool = pa.PagedKVPool(to_dev(pool_np, w.dtype))
    mcl = int(np.max(lens)) if max_context_len is None else max_context_len
    out = pa.pa_decode(pool, to_dev(q, w.dtype), i32(tables), i32(lens), scale=float(w.scale),
                       max_context_len=mcl, partition_size=partition_size, keep_cached=keep_cached)
    return out.cpu().numpy()


@pytest.mark.parametrize("k", [2, 3, 4])
def test_cache_policy_flag_does_not_change_results(k):
    w = make_config(k, small=True)
    say(f"[cache policy] {w.name}")
    _, pool_np = oracle_step(w, w.pool, 0)
    st = w.steps[0]
    a = _decode_custom(w, pool_np, w.block_tables, st.context_lens, st.q, 64, keep_cached=False)
    b = _decode_custom(w, pool_np, w.block_tables, st.context_lens, st.q, 64, keep_cached=True)
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("k,partition_size", [(2, 0), (2, 32), (4, 0), (4, 64)])
def test_bit_identical_under_physical_relabeling(k, partition_size):
    # workload 4 (groups of 8): the matrix-core decode and its combine kernel
    w = make_config(k, small=True)
    say(f"[relabel] {w.name} partition_size={partition_size}")
    st = w.steps[0]
    base = _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q, partition_size)
    perm = np.random.default_rng(31).permutation(w.num_blocks)
    pool2 = np.empty_like(w.pool)
    pool2[perm] = w.pool
    again = _decode_custom(w, pool2, perm[w.block_tables], st.context_lens, st.q, partition_size)
    assert base.tobytes() == again.tobytes()
    # and the result is deterministic run to run
    assert base.tobytes() == _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q,
                                            partition_size).tobytes()


def test_bit_identical_shared_vs_private_prefix():
    w = make_config(3, small=True)
    say(f"[shared vs private] {w.name}")
    st = w.steps[0]
    _, pool_np = oracle_step(w, w.pool, 0)  # the step's copies and writes, done on the CPU
    tables = w.block_tables.copy()
    # give every sequence private copies of the blocks it shares with others
    pool2 = pool_np.copy()
    free = [b for b in range(1, w.num_blocks) if np.isnan(paged.to_f64(pool_np[b, 0, 0, 0, :1])).all()]
    owners = {}
    for s in range(w.num_seqs):
        n = -(-int(st.context_lens[s]) // w.block_size)
        for j in range(n):
            b = int(tables[s, j])
            if b in owners and owners[b] != s:
                nb = free.pop()
                pool2[nb] = pool_np[b]
                tables[s, j] = nb
            else:
                owners.setdefault(b, s)
    shared = _decode_custom(w, pool_np, w.block_tables, st.context_lens, st.q)
    private = _decode_custom(w, pool2, tables, st.context_lens, st.q)
    assert shared.tobytes() == private.tobytes()


def test_padding_poison_and_single_token_closed_form():
    w = make_config(4, small=True)
    say(f"[poison + L=1] {w.name}")
    st = w.steps[0]
    _, pool_np = oracle_step(w, w.pool, 0)
    lens = st.context_lens.copy()
    lens[0] = 1           # one token: output equals that token's value exactly
    lens[1] = 45          # ragged: 13 poisoned slots after it in its second block
    poisoned = pool_np.copy()
    for s in range(w.num_seqs):
        L = int(lens[s])
        for t in range(L, -(-L // w.block_size) * w.block_size):
            b, o = paged.translate(w.block_tables[s], t, w.block_size)
            poisoned[b, :, :, o, :] = 0x7FC0  # bf16 NaN
    got = _decode_custom(w, poisoned, w.block_tables, lens, st.q, partition_size=64)
    assert np.isfinite(got).all()
    want = paged.decode_ref(pool_np, st.q, w.block_tables, lens, float(w.scale))
    assert np.abs(got - want).max() <= ATOL
    b0 = int(w.block_tables[0, 0])
    v0 = paged.to_f64(pool_np[b0, 1, :, 0, :])  # [Hkv][D]
    G = w.num_q_heads // w.num_kv_heads
    for hq in range(w.num_q_heads):
        assert np.array_equal(got[0, hq].astype(np.float64), v0[hq // G])


@pytest.mark.parametrize("case,partition_size", [("cfg2", 0), ("g8", 0), ("g8", 64)])
def test_zero_length_and_invalid_inputs_give_zeros_and_nan_rows(case, partition_size):
    # cfg2: groups of 4 (vector kernel); g8: groups of 8 over bf16 with 32-token blocks
    # (matrix-core kernel), in one partition and split into 64-token partitions
    if case == "cfg2":
        w = make_config(2, small=True)
    else:
        lens = [100, 300, 500, 77, 250, 33]
        w = make_custom(name="edge-rows-g8", seed=97, dtype="bf16", num_blocks=sum(-(-L // 32) for L in lens) + 4,
                        num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=32, lengths=lens)
    say(f"[edge rows] {w.name} partition {partition_size}")
    st = w.steps[0]
    lens = st.context_lens.copy()
    tables = w.block_tables.copy()
    lens[0] = 0                                  # empty context: zeros
    lens[1] = 10 ** 6                            # beyond the table row: NaN
    tables[2, 1] = w.num_blocks + 5              # invalid block id inside the context: NaN
    n3 = -(-int(lens[3]) // w.block_size)
    tables[3, n3:] = -7                          # invalid ids beyond the context: never read
    out = _decode_custom(w, w.pool, tables, lens, st.q, partition_size,
                         max_context_len=int(w.block_tables.shape[1] * w.block_size))
    assert (out[0] == 0).all()
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    good = [s for s in range(w.num_seqs) if s not in (0, 1, 2)]
    want = paged.decode_ref(w.pool, st.q[good], w.block_tables[good], lens[good], float(w.scale))
    assert np.abs(out[good] - want).max() <= ATOL


@pytest.mark.parametrize("block_size", [4, 8, 64, 128])
@pytest.mark.parametrize("group,head_dim,dtype", [(4, 128, "bf16"), (8, 64, "f32"), (1, 128, "bf16"),
                                             (8, 128, "bf16"), (8, 64, "bf16")])
def test_decode_block_size_sweep(block_size, group, head_dim, dtype):
    # small blocks are taken 16 / B to a pipeline stage, large ones in 16-token stages;
    # lengths land inside a stage, on its edge and one past it
    hkv = 2
    lens = [1, 5, 9, 16, 17, 63, 129, 300]
    nb = sum(-(-L // block_size) for L in lens) + 8
    w = make_custom(name="block-size-sweep", seed=43 + block_size, dtype=dtype, num_blocks=nb,
                    num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=head_dim, block_size=block_size,
                    lengths=lens)
    say(f"[block sizes] B={block_size} G={group} D={head_dim} {dtype}")
    for part in (0, 2 * max(block_size, 16)):
        pool = device_pool(w)
        _, out = run_step(w, pool, i32(w.block_tables), 0, partition_size=part)
        _, pool_np = oracle_step(w, w.pool, 0)
        want = decode_oracle(w, pool_np, 0)
        err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
        say(f"    partition {part}: max abs err {err:.3e}")
        assert np.isfinite(out.cpu().numpy()).all() and err <= ATOL


@pytest.mark.parametrize("group,head_dim,block_size,dtype", [
    (1, 128, 16, "bf16"), (2, 128, 32, "bf16"), (8, 64, 16, "bf16"), (4, 64, 32, "f32"), (8, 128, 16, "f32"),
])
def test_decode_other_supported_shapes(group, head_dim, block_size, dtype):
    hkv = 2
    lens = [1, 17, 33, 100, 250]
    w = make_custom(name="shape-sweep", seed=41, dtype=dtype, num_blocks=64, num_q_heads=hkv * group,
                    num_kv_heads=hkv, head_dim=head_dim, block_size=block_size, lengths=lens)
    say(f"[shapes] G={group} D={head_dim} B={block_size} {dtype}")
    for part in (0, 2 * block_size):
        pool = device_pool(w)
        _, out = run_step(w, pool, i32(w.block_tables), 0, partition_size=part)
        _, pool_np = oracle_step(w, w.pool, 0)
        want = decode_oracle(w, pool_np, 0)
        err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
        say(f"    partition {part}: max abs err {err:.3e}")
        assert err <= ATOL


@pytest.mark.parametrize("hkv,group,partition_size", [(3, 2, 64), (3, 2, 128), (1, 4, 256), (8, 1, 512),
                                                      (5, 8, 96)])
def test_decode_mixed_lengths_any_partition_count(hkv, group, partition_size):
    # many sequences of very different lengths, so most (sequence, head) pairs have fewer
    # partitions than the call; pair counts that are not multiples of 8; empty and invalid rows
    rng = np.random.default_rng(hkv * 100 + partition_size)
    lens = np.clip(np.rint(rng.lognormal(np.log(60), 1.2, size=37)), 1, 700).astype(np.int64)
    lens[3], lens[20] = 700, 1
    nb = int(sum(-(-L // 16) for L in lens)) + 4
    w = make_custom(name="mixed-lengths", seed=61 + hkv, dtype="bf16", num_blocks=nb, num_q_heads=hkv * group,
                    num_kv_heads=hkv, head_dim=64, block_size=16, lengths=lens)
    st = w.steps[0]
    say(f"[mixed] Hkv={hkv} G={group} partition {partition_size}: {len(lens)} sequences, max {lens.max()}")
    want = paged.decode_ref(w.pool, st.q, w.block_tables, st.context_lens, float(w.scale))
    got = _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q, partition_size)
    assert np.isfinite(got).all() and np.abs(got - want).max() <= ATOL
    # the same batch with an empty row and a row whose length exceeds the bound
    bad = st.context_lens.copy()
    bad[5], bad[11] = 0, 10 ** 6
    got = _decode_custom(w, w.pool, w.block_tables, bad, st.q, partition_size,
                         max_context_len=int(w.block_tables.shape[1]) * 16)
    assert (got[5] == 0).all() and np.isnan(got[11]).all()
    keep = [s for s in range(len(lens)) if s not in (5, 11)]
    assert np.abs(got[keep] - want[keep]).max() <= ATOL


@pytest.mark.parametrize("group,dtype,block_size,partition_size", [
    (8, "bf16", 32, 0), (8, "bf16", 16, 256), (8, "bf16", 64, 128), (4, "bf16", 16, 0), (8, "f32", 16, 0),
    (1, "bf16", 32, 512)])
def test_decode_running_max_raised_mid_stream(group, dtype, block_size, partition_size):
    # Keys along each KV head's mean query direction with a rising ramp (the running
    # maximum climbs past the lazy-rescale threshold many times inside every stream and
    # partition) and one spike token, so accumulators are rescaled mid-stream; random
    # N(0,1) data never moves the maximum that far after the first stage.
    from workloads import to_bf16_bits
    hkv, D = 2, 128
    lens = np.array([700, 333, 1030, 77, 16, 1], dtype=np.int64)
    nb = int(sum(-(-L // block_size) for L in lens)) + 4
    w = make_custom(name="rising-scores", seed=83 + group, dtype=dtype, num_blocks=nb, num_q_heads=hkv * group,
                    num_kv_heads=hkv, head_dim=D, block_size=block_size, lengths=lens)
    st = w.steps[0]
    say(f"[rescale] G={group} {dtype} B={block_size} partition {partition_size}")
    q = paged.to_f64(st.q)
    pool = w.pool.copy()
    rng = np.random.default_rng(5)
    for s, L in enumerate(lens):
        spike = int(rng.integers(0, L))
        for h in range(hkv):
            u = q[s, h * group:(h + 1) * group].sum(axis=0)
            u /= np.linalg.norm(u)
            # the group's top head ends 100 log2 units above where it starts; the spike adds 60
            top = float((q[s, h * group:(h + 1) * group] @ u).max()) * float(w.scale) * np.log2(np.e)
            for t in range(int(L)):
                c = (100.0 * t / max(int(L) - 1, 1) + (60.0 if t == spike else 0.0)) / top
                kv = (c * u + 0.05 * rng.standard_normal(D)).astype(np.float32)
                b, o = paged.translate(w.block_tables[s], t, block_size)
                pool[b, 0, h, o, :] = to_bf16_bits(kv) if dtype == "bf16" else kv
    want = paged.decode_ref(pool, st.q, w.block_tables, st.context_lens, float(w.scale))
    got = _decode_custom(w, pool, w.block_tables, st.context_lens, st.q, partition_size)
    err = np.abs(got - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL


@pytest.mark.parametrize("group,dtype,partition_size", [(4, "bf16", 1024), (2, "f32", 2048), (4, "f32", 1536),
                                                        (8, "bf16", 2048), (8, "f32", 4096), (1, "bf16", 4096)])
def test_decode_work_shapes_by_partition(group, dtype, partition_size):
    # the launch picks its work shape from the group size and the partition length:
    # 4 waves with 4-token stages, 8 waves with 8-token stages (1,024-2,048-token
    # partitions), or for groups of 8 the 8- or 16-token stages; every shape against the oracle
    hkv = 2
    rng = np.random.default_rng(group * 7 + partition_size)
    lens = np.clip(np.rint(rng.lognormal(np.log(900), 1.0, size=19)), 1, 6000).astype(np.int64)
    lens[0], lens[1] = 6000, 2 * partition_size + 1
    nb = int(sum(-(-L // 16) for L in lens)) + 4
    w = make_custom(name="work-shapes", seed=71 + group, dtype=dtype, num_blocks=nb, num_q_heads=hkv * group,
                    num_kv_heads=hkv, head_dim=128, block_size=16, lengths=lens)
    st = w.steps[0]
    say(f"[work shapes] G={group} {dtype} partition {partition_size}: max {lens.max()}")
    want = paged.decode_ref(w.pool, st.q, w.block_tables, st.context_lens, float(w.scale))
    got = _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q, partition_size)
    assert np.isfinite(got).all() and np.abs(got - want).max() <= ATOL


@pytest.mark.parametrize("group,dtype,block_size,partition_size", [
    (4, "bf16", 4, 8192), (8, "bf16", 4, 4096), (1, "f32", 8, 8192), (2, "bf16", 4, 2048), (4, "f32", 4, 1536)])
def test_decode_long_partitions_of_small_blocks(group, dtype, block_size, partition_size):
    # partitions of up to 2,048 blocks: a workgroup stages two table entries per thread
    # early and the rest (up to six more per thread) in a second pass
    hkv = 2
    lens = np.array([2 * partition_size + 3, 9000, partition_size, partition_size + 1, 1, 700, 4100], dtype=np.int64)
    nb = int(sum(-(-L // block_size) for L in lens)) + 4
    w = make_custom(name="long-partitions", seed=97 + block_size + group, dtype=dtype, num_blocks=nb,
                    num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=128, block_size=block_size, lengths=lens)
    st = w.steps[0]
    say(f"[long partitions] G={group} {dtype} B={block_size} partition {partition_size} "
        f"({partition_size // block_size} blocks)")
    want = paged.decode_ref(w.pool, st.q, w.block_tables, st.context_lens, float(w.scale))
    got = _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q, partition_size)
    err = np.abs(got - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL


def test_decode_many_pairs_with_long_partitions():
    # 1,024 (sequence, KV head) pairs of several partitions would walk a work list, whose
    # workgroups stage at most 512 table entries: 1,024-block partitions take the grid
    # instead, 512-block ones the list; both against the oracle
    rng = np.random.default_rng(2024)
    S, hkv, B = 128, 8, 4
    lens = np.clip(np.rint(rng.lognormal(np.log(40), 0.8, size=S)), 1, 400).astype(np.int64)
    lens[7], lens[90] = 5000, 4097
    nb = int(sum(-(-L // B) for L in lens)) + 4
    w = make_custom(name="many-pairs-long-partitions", seed=131, dtype="bf16", num_blocks=nb,
                    num_q_heads=hkv, num_kv_heads=hkv, head_dim=64, block_size=B, lengths=lens)
    st = w.steps[0]
    say(f"[many pairs] {S} sequences x {hkv} KV heads, B={B}, max {lens.max()}")
    want = paged.decode_ref(w.pool, st.q, w.block_tables, st.context_lens, float(w.scale))
    for part in (4096, 2048):
        got = _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q, part)
        err = np.abs(got - want).max()
        say(f"    partition {part} ({part // B} blocks): max abs err {err:.3e}")
        assert np.isfinite(got).all() and err <= ATOL


# ------------------------------------------------------------------ seeded random shapes


def _random_case(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([4, 8, 16, 32, 64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    hkv = int(rng.integers(1, 4))
    S = int(rng.integers(1, 9))
    lens = np.clip(np.rint(rng.lognormal(np.log(150), 1.0, size=S)), 1, 1200).astype(np.int64)
    unit = max(B, 16)
    part = int(rng.choice([0, unit, 2 * unit, 4 * unit]))
    keep = bool(rng.integers(0, 2))
    return G, D, B, dtype, hkv, lens, part, keep


@pytest.mark.parametrize("group", [4, 8])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 5.0])
def test_decode_any_scale(scale, group):
    # the scale is any float: negative (the softmax favours the smallest q.k), zero (a
    # uniform average over the context) and large (a near-argmax softmax whose running
    # maximum jumps by hundreds of log2 units); vector scores (group 4) and matrix-core
    # scores (group 8), several partitions, against the oracle at the same scale
    lens = np.array([1, 700, 33, 1500, 256], dtype=np.int64)
    hkv = 2
    w = make_custom(name=f"scale-{scale}-g{group}", seed=131 + group, dtype="bf16",
                    num_blocks=int(sum(-(-int(L) // 16) for L in lens)) + 4, num_q_heads=hkv * group,
                    num_kv_heads=hkv, head_dim=128, block_size=16, lengths=lens)
    w.scale = np.float32(scale)
    st = w.steps[0]
    want = paged.decode_ref(w.pool, st.q, w.block_tables, st.context_lens, float(w.scale))
    for part in (0, 256):
        got = _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q, part)
        err = np.abs(got - want).max()
        say(f"[scale {scale}] G={group} partition={part}: max abs err {err:.3e}")
        assert np.isfinite(got).all() and err <= ATOL


@pytest.mark.parametrize("seed", list(range(40)))
def test_decode_seeded_random_shapes(seed):
    # one seeded draw of every supported knob at a time: group, head dim, block size, dtype,
    # KV heads, ragged lengths, partition size and cache policy, against the oracle
    G, D, B, dtype, hkv, lens, part, keep = _random_case(1000 + seed)
    nb = int(sum(-(-L // B) for L in lens)) + 3
    w = make_custom(name=f"random-{seed}", seed=2000 + seed, dtype=dtype, num_blocks=nb, num_q_heads=hkv * G,
                    num_kv_heads=hkv, head_dim=D, block_size=B, lengths=lens)
    st = w.steps[0]
    say(f"[random {seed}] G={G} D={D} B={B} {dtype} Hkv={hkv} S={len(lens)} max={lens.max()} "
        f"partition={part} keep_cached={keep}")
    want = paged.decode_ref(w.pool, st.q, w.block_tables, st.context_lens, float(w.scale))
    got = _decode_custom(w, w.pool, w.block_tables, st.context_lens, st.q, part, keep_cached=keep)
    err = np.abs(got - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL
