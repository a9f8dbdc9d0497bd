"""Pins of the oracle's gather and attention: brute force, a library routine,
closed forms and the invariants the pages state (placement and sharing do not
change the result; padding is never read)."""

import math

import numpy as np
import pytest
import torch

from oracle import alloc
from oracle import paged
from workloads import to_bf16_bits


def brute_force_attention(q, keys, values, scale):
    """Pure-Python attention with the unshifted exponential (a different algorithm)."""
    L, D = len(keys), len(q)
    scores = [scale * sum(float(q[d]) * float(keys[t][d]) for d in range(D)) for t in range(L)]
    w = [math.exp(s) for s in scores]
    z = sum(w)
    return [sum(w[t] * float(values[t][d]) for t in range(L)) / z for d in range(D)]


def build_paged(rng, lengths, num_kv_heads, head_dim, block_size, num_blocks, dtype="f32", free_order=None):
    """Contiguous K/V per sequence first, then scattered token by token into a pool
    through the oracle's allocator and cache write (NaN everywhere else)."""
    shape = (num_blocks, 2, num_kv_heads, block_size, head_dim)
    if dtype == "f32":
        pool = np.full(shape, np.nan, dtype=np.float32)
    else:
        pool = np.full(shape, 0x7FC0, dtype=np.uint16)
    bp = alloc.BlockPool(num_blocks, block_size, free_order=free_order)
    contig, seqs = [], []
    for L in lengths:
        kv = rng.standard_normal((L, 2, num_kv_heads, head_dim)).astype(np.float32)
        if dtype == "bf16":
            kv = to_bf16_bits(kv)
        contig.append(kv)
        s = alloc.Sequence()
        for t in range(L):
            slot, cow = alloc.prepare_write(bp, s, t)
            assert cow is None
            pool = paged.cache_write_ref(pool, kv[t:t + 1, 0], kv[t:t + 1, 1], [slot])
        seqs.append(s)
    width = max(len(s.block_table) for s in seqs)
    tables = np.zeros((len(lengths), width), dtype=np.int32)
    for i, s in enumerate(seqs):
        tables[i, :len(s.block_table)] = s.block_table
    return pool, tables, contig


@pytest.mark.parametrize("block_size,head_dim,lengths,hq,hkv,dtype", [
    (4, 8, [1, 5, 9, 13], 4, 2, "f32"),
    (16, 64, [25, 47, 12], 4, 4, "f32"),
    (32, 8, [70, 33, 1, 32], 8, 2, "f32"),
    (16, 8, [17, 31, 2], 8, 1, "bf16"),
])
def test_decode_matches_brute_force(block_size, head_dim, lengths, hq, hkv, dtype):
    rng = np.random.default_rng(7)
    n_blocks = sum(-(-L // block_size) for L in lengths) + 3
    order = list(rng.permutation(n_blocks))
    pool, tables, contig = build_paged(rng, lengths, hkv, head_dim, block_size, n_blocks, dtype, order)
    q = rng.standard_normal((len(lengths), hq, head_dim)).astype(np.float32)
    if dtype == "bf16":
        q = to_bf16_bits(q)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(head_dim)))
    out = paged.decode_ref(pool, q, tables, lengths, scale)
    g = hq // hkv
    for s, L in enumerate(lengths):
        kv = paged.to_f64(contig[s])
        for h in range(hq):
            bf = brute_force_attention(paged.to_f64(q[s, h]), kv[:, 0, h // g], kv[:, 1, h // g], scale)
            np.testing.assert_allclose(out[s, h], bf, rtol=0, atol=1e-12)
            one = paged.decode_one_ref(pool, q, tables, lengths, scale, s, h)
            np.testing.assert_array_equal(one, out[s, h])


def test_attention_matches_torch_sdpa_float64():
    rng = np.random.default_rng(11)
    L, D = 37, 16
    q = rng.standard_normal(D)
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    scale = 0.3
    ours = paged.attention_ref(q, k, v, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=scale)[0, 0, 0].numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(3)
    D = 8
    v = rng.standard_normal((5, D))
    k = rng.standard_normal((5, D))
    # one token: the output is that token's value exactly
    assert np.array_equal(paged.attention_ref(rng.standard_normal(D), k[:1], v[:1], 0.5), v[0])
    # zero query: uniform weights -> mean of V
    np.testing.assert_allclose(paged.attention_ref(np.zeros(D), k, v, 0.5), v.mean(0), atol=1e-15)
    # identical keys: uniform weights -> mean of V
    np.testing.assert_allclose(paged.attention_ref(rng.standard_normal(D), np.tile(k[:1], (5, 1)), v, 0.5),
                               v.mean(0), atol=1e-14)
    # one dominant logit: that token's value
    kk = np.zeros((5, D))
    kk[3, 0] = 1.0
    q = np.zeros(D)
    q[0] = 2000.0
    np.testing.assert_allclose(paged.attention_ref(q, kk, v, 1.0), v[3], atol=1e-300)
    # the scale enters the exponent: two tokens with scores 0 and scale*1
    k2 = np.array([[0.0], [1.0]])
    v2 = np.array([[0.0], [1.0]])
    for sc in (0.25, 1.0, 3.0):
        w = math.exp(sc) / (1 + math.exp(sc))
        np.testing.assert_allclose(paged.attention_ref(np.array([1.0]), k2, v2, sc), [w], atol=1e-15)


def test_shifted_softmax_handles_large_scores():
    # the max subtraction keeps huge logits finite (an unshifted exp would overflow)
    k = np.array([[1000.0], [999.0]])
    v = np.array([[1.0], [0.0]])
    out = paged.attention_ref(np.array([1.0]), k, v, 1.0)
    np.testing.assert_allclose(out, [1 / (1 + math.exp(-1))], atol=1e-15)


def _random_case(rng, lengths, hkv=2, hq=4, D=8, B=4, extra=5, dtype="f32"):
    n = sum(-(-L // B) for L in lengths) + extra
    pool, tables, _ = build_paged(rng, lengths, hkv, D, B, n, dtype, list(rng.permutation(n)))
    q = rng.standard_normal((len(lengths), hq, D)).astype(np.float32)
    return pool, tables, q


def test_invariant_physical_relabeling():
    rng = np.random.default_rng(5)
    lengths = [9, 14, 3]
    pool, tables, q = _random_case(rng, lengths)
    out = paged.decode_ref(pool, q, tables, lengths, 0.35)
    perm = rng.permutation(pool.shape[0])  # block b moves to perm[b]
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    tables2 = perm[tables].astype(np.int32)
    out2 = paged.decode_ref(pool2, q, tables2, lengths, 0.35)
    assert np.array_equal(out, out2)


def test_invariant_shared_vs_private_prefix():
    rng = np.random.default_rng(6)
    B, D, hkv = 4, 8, 2
    n = 16
    pool = np.full((n, 2, hkv, B, D), np.nan, dtype=np.float32)
    pool[[0, 1, 2, 3]] = rng.standard_normal((4, 2, hkv, B, D))
    # shared: both sequences point at blocks 0,1 then own tails 2 and 3
    shared = np.array([[0, 1, 2], [0, 1, 3]], dtype=np.int32)
    # private: copies of the prefix blocks at 4,5 and 6,7
    pool[[4, 5]] = pool[[0, 1]]
    pool[[6, 7]] = pool[[0, 1]]
    private = np.array([[4, 5, 2], [6, 7, 3]], dtype=np.int32)
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    lens = [11, 10]
    assert np.array_equal(paged.decode_ref(pool, q, shared, lens, 0.4),
                          paged.decode_ref(pool, q, private, lens, 0.4))


def test_invariant_cow_leaves_other_sharers_unchanged():
    rng = np.random.default_rng(8)
    B, D, hkv, n = 4, 8, 1, 12
    bp = alloc.BlockPool(n, B)
    pool = np.full((n, 2, hkv, B, D), np.nan, dtype=np.float32)
    a = alloc.Sequence()
    for t in range(6):  # A's prompt: 6 tokens in blocks 0, 1
        slot, _ = alloc.prepare_write(bp, a, t)
        kv = rng.standard_normal((1, 2, hkv, D)).astype(np.float32)
        pool = paged.cache_write_ref(pool, kv[:, 0], kv[:, 1], [slot])
    b = alloc.fork(bp, a)
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    before = paged.decode_ref(pool, q, [a.block_table], [6], 0.3)
    # B writes its token 6 into the shared block 1: copy first, then write into the copy
    slot, cow = alloc.prepare_write(bp, b, 6)
    assert cow is not None
    pool = paged.block_copy_ref(pool, [cow[0]], [cow[1]])
    kv = rng.standard_normal((1, 2, hkv, D)).astype(np.float32)
    pool = paged.cache_write_ref(pool, kv[:, 0], kv[:, 1], [slot])
    after = paged.decode_ref(pool, q, [a.block_table], [6], 0.3)
    assert np.array_equal(before, after)
    # and B sees A's first six tokens plus its own seventh
    kb, vb = paged.gather_ref(pool, b.block_table, 7, 0)
    ka, va = paged.gather_ref(pool, a.block_table, 6, 0)
    assert np.array_equal(kb[:6], ka) and np.array_equal(vb[:6], va)
    assert np.array_equal(kb[6], kv[0, 0, 0].astype(np.float64))


def test_invariant_padding_and_unused_blocks_never_read():
    rng = np.random.default_rng(9)
    lengths = [5, 11, 2]
    pool, tables, q = _random_case(rng, lengths)  # build_paged leaves every unwritten slot NaN
    out = paged.decode_ref(pool, q, tables, lengths, 0.5)
    assert np.isfinite(out).all()
    # overwrite every finite value outside the live slots with something else: same output
    pool2 = pool.copy()
    pool2[np.isnan(pool2)] = 1e30
    assert np.array_equal(out, paged.decode_ref(pool2, q, tables, lengths, 0.5))


def test_zero_length_gives_zeros():
    rng = np.random.default_rng(10)
    pool, tables, q = _random_case(rng, [4, 1])
    out = paged.decode_ref(pool, q, tables, [0, 1], 0.5)
    assert np.array_equal(out[0], np.zeros_like(out[0]))


def test_bf16_widening_is_exact():
    vals = np.array([1.0, -2.5, 3.140625, 65280.0, 2.0 ** -130, -0.0], dtype=np.float32)
    bits = to_bf16_bits(vals)
    back = paged.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(back, vals.astype(np.float64))
    # rounding to nearest even of the low half
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32)  # exactly between two bf16 values
    np.testing.assert_array_equal(paged.bf16_bits_to_f64(to_bf16_bits(x)), [1.0, 1.0 + 2 ** -6])


def test_cache_write_changes_exactly_the_target_slots():
    rng = np.random.default_rng(12)
    pool = rng.standard_normal((6, 2, 3, 4, 8)).astype(np.float32)
    k = rng.standard_normal((3, 3, 8)).astype(np.float32)
    v = rng.standard_normal((3, 3, 8)).astype(np.float32)
    slots = [5, -1, 22]  # block 1 offset 1; skipped; block 5 offset 2
    out = paged.cache_write_ref(pool, k, v, slots)
    changed = np.argwhere((out != pool).any(axis=-1))
    expect = sorted([(1, kv, h, 1) for kv in (0, 1) for h in range(3)] + [(5, kv, h, 2) for kv in (0, 1) for h in range(3)])
    assert sorted(map(tuple, changed.tolist())) == expect
    assert np.array_equal(out[1, 0, :, 1], k[0]) and np.array_equal(out[1, 1, :, 1], v[0])
    assert np.array_equal(out[5, 0, :, 2], k[2]) and np.array_equal(out[5, 1, :, 2], v[2])


def test_block_copy_copies_whole_blocks_only():
    rng = np.random.default_rng(13)
    pool = rng.standard_normal((8, 2, 2, 4, 4)).astype(np.float32)
    out = paged.block_copy_ref(pool, [1, 6], [3, 0])
    assert np.array_equal(out[3], pool[1]) and np.array_equal(out[0], pool[6])
    for b in (1, 2, 4, 5, 6, 7):
        assert np.array_equal(out[b], pool[b])



# ------------------------------------------------------------------ prefill


def test_prefill_single_query_rows_equal_decode():
    """A chunk of one query per sequence is a decode step (same positions, same keys)."""
    rng = np.random.default_rng(14)
    lengths = [9, 14, 3]
    pool, tables, q = _random_case(rng, lengths)
    dec = paged.decode_ref(pool, q, tables, lengths, 0.4)
    pre = paged.prefill_ref(pool, q, [0, 1, 2, 3], lengths, tables, 0.4)
    assert np.array_equal(dec, pre)


def test_prefill_matches_torch_causal_sdpa_float64():
    """Full prefill (queries = whole context) is textbook causal attention."""
    rng = np.random.default_rng(15)
    lengths = [13, 7]
    hq, hkv, D = 4, 2, 8
    pool, tables, contig = build_paged(rng, lengths, hkv, D, 4, 12, "f32", list(rng.permutation(12)))
    q = rng.standard_normal((sum(lengths), hq, D)).astype(np.float32)
    out = paged.prefill_ref(pool, q, [0, 13, 20], lengths, tables, 0.3)
    start = 0
    for s, L in enumerate(lengths):
        kv = paged.to_f64(contig[s])  # [L][2][Hkv][D]
        for h in range(hq):
            k = torch.from_numpy(kv[:, 0, h // 2])[None, None]
            v = torch.from_numpy(kv[:, 1, h // 2])[None, None]
            qq = torch.from_numpy(q[start:start + L, h].astype(np.float64))[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, is_causal=True, scale=0.3)[0, 0]
            np.testing.assert_allclose(out[start:start + L, h], ref.numpy(), rtol=0, atol=1e-13)
        start += L


def test_chunked_prefill_matches_brute_force():
    """A chunk appended to a cached context: row i sees positions 0 .. ctx - n + i."""
    rng = np.random.default_rng(16)
    lengths = [11, 6]
    chunk = [4, 6]
    hq, hkv, D = 2, 1, 8
    pool, tables, contig = build_paged(rng, lengths, hkv, D, 4, 8, "f32", list(rng.permutation(8)))
    q = rng.standard_normal((sum(chunk), hq, D)).astype(np.float32)
    out = paged.prefill_ref(pool, q, [0, 4, 10], lengths, tables, 0.5)
    row = 0
    for s, L in enumerate(lengths):
        kv = paged.to_f64(contig[s])
        for i in range(chunk[s]):
            pos = L - chunk[s] + i
            for h in range(hq):
                bf = brute_force_attention(q[row, h].astype(np.float64), kv[:pos + 1, 0, 0], kv[:pos + 1, 1, 0], 0.5)
                np.testing.assert_allclose(out[row, h], bf, rtol=0, atol=1e-12)
            row += 1


def test_parallel_runner_equals_the_whole_pool_oracle():
    """oracle.parallel runs decode_ref per sequence on that sequence's blocks (identity table),
    optionally after replaying its writes: the same numbers, bit for bit, as decode_ref and
    cache_write_ref over the whole pool, in this process and in spawned workers."""
    from oracle.parallel import run_tasks, sequence_task
    from workloads import make_custom
    w = make_custom(name="par", seed=11, dtype="bf16", num_blocks=64, num_q_heads=8, num_kv_heads=2,
                    head_dim=64, block_size=16, lengths=[70, 1, 33, 16], num_steps=1)
    st = w.steps[0]
    slots = paged.slot_mapping_ref(w.block_tables, st.write_seq, st.write_pos, w.block_size)
    after = paged.cache_write_ref(w.pool, st.k_new, st.v_new, slots)
    want = paged.decode_ref(after, st.q, w.block_tables, st.context_lens, float(w.scale))
    plain = [sequence_task(after, w.block_tables[s], int(st.context_lens[s]), st.q[s], float(w.scale))
             for s in range(w.num_seqs)]
    replay = [sequence_task(w.pool, w.block_tables[s], int(st.context_lens[s]), st.q[s], float(w.scale),
                            (st.write_pos[s:s + 1], st.k_new[s:s + 1], st.v_new[s:s + 1]))
              for s in range(w.num_seqs)]
    for got in (run_tasks(plain, workers=1), run_tasks(replay, workers=1), run_tasks(replay, workers=2)):
        assert all(np.array_equal(g, want[s]) for s, g in enumerate(got))
