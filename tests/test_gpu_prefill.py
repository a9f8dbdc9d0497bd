"""GPU parity of the MFMA prefill kernel (pa_prefill) against the float64 oracle.

Each case first writes the chunk's K/V through pa_slot_mapping + pa_cache_write
(the prefill write path), then runs pa_prefill; the oracle replays the same
write with its own routines and computes causal attention row by row.
Bar: max-abs error 2e-3.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_121_amd as pa
from oracle import paged
from workloads import make_prefill, make_prefill_custom

from _gpu_util import device_pool, i32, say, to_dev, to_host

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def gpu_prefill(w, pool=None, max_query_len=None):
    pool = pool or device_pool(w)
    tables = i32(w.block_tables)
    slots = pa.pa_slot_mapping(pool, tables, i32(w.write_seq), i32(w.write_pos))
    pa.pa_cache_write(pool, to_dev(w.k_new, w.dtype), to_dev(w.v_new, w.dtype), slots)
    n = np.diff(w.query_start_loc)
    out = pa.pa_prefill(pool, to_dev(w.q, w.dtype), i32(w.query_start_loc), i32(w.context_lens), tables,
                        scale=float(w.scale), max_query_len=int(n.max()) if max_query_len is None else max_query_len)
    torch.cuda.synchronize()
    return pool, out.cpu().numpy()


def oracle_pool(w):
    slots = paged.slot_mapping_ref(w.block_tables, w.write_seq, w.write_pos, w.block_size)
    return paged.cache_write_ref(w.pool, w.k_new, w.v_new, slots)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 5.0])
def test_prefill_any_scale(scale):
    # negative (applied as |scale| on -Q), zero (a uniform average over each row's visible
    # keys) and large (near-argmax, the running maximum raised by hundreds of log2 units)
    w = make_prefill_custom(name=f"prefill-scale-{scale}", seed=141, dtype="bf16", num_blocks=200,
                            num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                            context_lens=[300, 1000, 77], chunk_lens=[300, 130, 77])
    w.scale = np.float32(scale)
    pool, got = gpu_prefill(w)
    pool_np = oracle_pool(w)
    want = paged.prefill_ref(pool_np, w.q, w.query_start_loc, w.context_lens, w.block_tables, float(w.scale))
    err = np.abs(got.astype(np.float64) - want).max()
    say(f"[prefill scale {scale}] max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL


@pytest.mark.parametrize("k", [1, 2])
def test_prefill_small_workloads_match_oracle(k):
    w = make_prefill(k, small=True)
    say(f"[prefill] {w.name}")
    pool, got = gpu_prefill(w)
    pool_np = oracle_pool(w)
    assert to_host(pool.data).tobytes() == pool_np.tobytes()  # the prefill write, bit for bit
    want = paged.prefill_ref(pool_np, w.q, w.query_start_loc, w.context_lens, w.block_tables, float(w.scale))
    err = np.abs(got.astype(np.float64) - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL


@pytest.mark.parametrize("group,head_dim,block_size", [
    (1, 128, 16), (2, 128, 32), (4, 64, 16), (8, 128, 32), (8, 64, 16), (4, 128, 32),
    (4, 128, 4), (2, 64, 8), (2, 64, 4), (4, 128, 64), (8, 128, 128), (1, 64, 128),
])
def test_prefill_shapes_chunks_and_ragged_tails(group, head_dim, block_size):
    hkv = 2
    ctx = [1, 63, 64, 65, 150, 200]
    chunk = [1, 63, 10, 65, 33, 129]   # whole prompts, chunks, a one-row chunk
    nb = sum(-(-L // block_size) for L in ctx) + 8
    w = make_prefill_custom(name="prefill-shapes", seed=7 + group, dtype="bf16", num_blocks=nb,
                            num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=head_dim,
                            block_size=block_size, context_lens=ctx, chunk_lens=chunk)
    say(f"[prefill shapes] G={group} D={head_dim} B={block_size}")
    _, got = gpu_prefill(w)
    want = paged.prefill_ref(oracle_pool(w), w.q, w.query_start_loc, w.context_lens, w.block_tables,
                             float(w.scale))
    err = np.abs(got.astype(np.float64) - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL


def test_prefill_single_row_chunks_agree_with_decode():
    w = make_prefill_custom(name="prefill-vs-decode", seed=31, dtype="bf16", num_blocks=96, num_q_heads=32,
                            num_kv_heads=8, head_dim=128, block_size=16, context_lens=[17, 300, 64, 5],
                            chunk_lens=[1, 1, 1, 1])
    say("[prefill vs decode] one-row chunks")
    pool, got = gpu_prefill(w)
    dec = pa.pa_decode(pool, to_dev(w.q, w.dtype), i32(w.block_tables), i32(w.context_lens), scale=float(w.scale),
                       max_context_len=300).cpu().numpy()
    # prefill carries P as two bf16 parts (within 2^-15 of the fp32 P) where decode keeps
    # fp32 P; both meet the parity bar against the oracle, and they agree far more closely
    want = paged.decode_ref(oracle_pool(w), w.q, w.block_tables, w.context_lens, float(w.scale))
    assert np.abs(dec - want).max() <= ATOL and np.abs(got - want).max() <= ATOL
    diff = np.abs(got - dec).max()
    say(f"    prefill vs decode max abs diff {diff:.3e}")
    assert diff <= 1e-4


@pytest.mark.parametrize("group,block_size", [(4, 16), (8, 32), (1, 64)])
def test_prefill_running_max_raised_mid_row(group, block_size):
    # Queries near one direction per KV head and keys along it with a rising ramp plus a
    # spike: every row's running maximum climbs past the lazy-rescale threshold tile after
    # tile (causal rows see ever larger scores), so O and the row sums are rescaled
    # mid-row; N(0,1) data never moves the maximum that far after the first tile.
    from workloads import to_bf16_bits
    hkv, D = 2, 128
    ctx, chunk = [300, 200, 130], [300, 64, 1]
    nb = sum(-(-L // block_size) for L in ctx) + 8
    w = make_prefill_custom(name="prefill-rising", seed=61 + group, dtype="bf16", num_blocks=nb,
                            num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=D, block_size=block_size,
                            context_lens=ctx, chunk_lens=chunk)
    say(f"[prefill rescale] G={group} B={block_size}")
    rng = np.random.default_rng(9)
    pool_np = oracle_pool(w).copy()
    q = paged.to_f64(w.q).copy()  # [rows][Hq][D]
    log2e = float(np.log2(np.e))
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        r0, r1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
        spike = int(rng.integers(0, L))
        for h in range(hkv):
            u = rng.standard_normal(D)
            u /= np.linalg.norm(u)
            q[r0:r1, h * group:(h + 1) * group] = 3.0 * u + 0.3 * rng.standard_normal((r1 - r0, group, D))
            # scores rise by about 100 log2 units over the context; the spike adds 60
            per_unit = 3.0 * float(w.scale) * log2e
            for t in range(L):
                c = (100.0 * t / max(L - 1, 1) + (60.0 if t == spike else 0.0)) / per_unit
                kv = (c * u + 0.05 * rng.standard_normal(D)).astype(np.float32)
                b, o = paged.translate(w.block_tables[s], t, block_size)
                pool_np[b, 0, h, o, :] = to_bf16_bits(kv)
    qb = to_bf16_bits(q.astype(np.float32))
    pool = pa.PagedKVPool(to_dev(pool_np, "bf16"))
    got = pa.pa_prefill(pool, to_dev(qb, "bf16"), i32(w.query_start_loc), i32(w.context_lens),
                        i32(w.block_tables), scale=float(w.scale), max_query_len=max(chunk)).cpu().numpy()
    want = paged.prefill_ref(pool_np, qb, w.query_start_loc, w.context_lens, w.block_tables, float(w.scale))
    err = np.abs(got.astype(np.float64) - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL


def test_prefill_padding_poison_is_never_read():
    w = make_prefill_custom(name="prefill-poison", seed=41, dtype="bf16", num_blocks=64, num_q_heads=8,
                            num_kv_heads=2, head_dim=128, block_size=16, context_lens=[45, 70],
                            chunk_lens=[45, 20])
    say("[prefill poison]")
    pool_np = oracle_pool(w)
    poisoned = pool_np.copy()
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        for t in range(L, -(-L // 16) * 16):
            b, o = paged.translate(w.block_tables[s], t, 16)
            poisoned[b, :, :, o, :] = 0x7FC0
    pool = pa.PagedKVPool(to_dev(poisoned, "bf16"))
    out = pa.pa_prefill(pool, to_dev(w.q, "bf16"), i32(w.query_start_loc), i32(w.context_lens),
                        i32(w.block_tables), scale=float(w.scale), max_query_len=45).cpu().numpy()
    want = paged.prefill_ref(pool_np, w.q, w.query_start_loc, w.context_lens, w.block_tables, float(w.scale))
    assert np.isfinite(out).all() and np.abs(out - want).max() <= ATOL


def test_prefill_inconsistent_rows_are_nan_and_others_exact():
    w = make_prefill_custom(name="prefill-edge", seed=51, dtype="bf16", num_blocks=64, num_q_heads=8,
                            num_kv_heads=2, head_dim=128, block_size=16, context_lens=[40, 30, 50],
                            chunk_lens=[10, 10, 10])
    say("[prefill edge rows]")
    pool_np = oracle_pool(w)
    pool = pa.PagedKVPool(to_dev(pool_np, "bf16"))
    lens = w.context_lens.copy()
    lens[1] = 5                      # fewer cached tokens than query rows: inconsistent
    tables = w.block_tables.copy()
    out = pa.pa_prefill(pool, to_dev(w.q, "bf16"), i32(w.query_start_loc), i32(lens), i32(tables),
                        scale=float(w.scale), max_query_len=10).cpu().numpy()
    assert np.isnan(out[10:20]).all()
    good = np.r_[0:10, 20:30]
    want = paged.prefill_ref(pool_np, w.q, w.query_start_loc, w.context_lens, w.block_tables, float(w.scale))
    assert np.abs(out[good] - want[good]).max() <= ATOL


@pytest.mark.parametrize("k", [1, 2])
def test_prefill_fullsize_sampled_rows(k):
    w = make_prefill(k)
    say(f"[prefill fullsize] {w.name}: T={w.total_tokens} flops={w.attention_flops() / 1e9:.1f} GFLOP")
    pool, got = gpu_prefill(w)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(60 + k)
    errs = []
    for s in rng.choice(w.num_seqs, size=2, replace=False):
        # the oracle on this sequence alone: its blocks, its written chunk, a few of its rows
        n = int(w.query_start_loc[s + 1] - w.query_start_loc[s])
        ctx = int(w.context_lens[s])
        nb = -(-ctx // w.block_size)
        row = w.block_tables[s, :nb]
        small = w.pool[row].copy()
        tbl = np.arange(nb, dtype=np.int32)[None, :]
        sel = slice(int(w.query_start_loc[s]), int(w.query_start_loc[s + 1]))
        slots = paged.slot_mapping_ref(tbl, np.zeros(n, dtype=np.int32), w.write_pos[sel], w.block_size)
        small = paged.cache_write_ref(small, w.k_new[sel], w.v_new[sel], slots)
        pick = sorted(set([0, n - 1] + list(rng.choice(n, size=3))))
        qs = w.q[sel][pick]
        for j, i in enumerate(pick):
            want = paged.prefill_ref(small, qs[j:j + 1], [0, 1], [ctx - n + i + 1], tbl, float(w.scale))
            errs.append(np.abs(got[int(w.query_start_loc[s]) + i].astype(np.float64) - want[0]).max())
    say(f"    {len(errs)} sampled rows, max abs err {max(errs):.3e}")
    assert max(errs) <= ATOL


@pytest.mark.parametrize("seed", list(range(24)))
def test_prefill_seeded_random_shapes(seed):
    # one seeded draw of group, head dim, block size, KV heads, contexts and chunk lengths
    # (whole prompts, chunks, single rows) at a time, against the oracle; contexts of up to
    # 1,500 tokens take the tile loop through both buffer parities many times over
    rng = np.random.default_rng(3000 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([4, 8, 16, 32, 64, 128]))
    hkv = int(rng.integers(1, 3))
    S = int(rng.integers(1, 5))
    ctx = [int(x) for x in rng.integers(1, 400 if seed < 8 else 1500, size=S)]
    chunk = [int(rng.choice([c, max(1, c // 3), 1])) for c in ctx]
    nb = sum(-(-L // B) for L in ctx) + 4
    w = make_prefill_custom(name=f"prefill-random-{seed}", seed=4000 + seed, dtype="bf16", num_blocks=nb,
                            num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D, block_size=B, context_lens=ctx,
                            chunk_lens=chunk)
    say(f"[prefill random {seed}] G={G} D={D} B={B} Hkv={hkv} contexts {ctx} chunks {chunk}")
    _, got = gpu_prefill(w)
    want = paged.prefill_ref(oracle_pool(w), w.q, w.query_start_loc, w.context_lens, w.block_tables,
                             float(w.scale))
    err = np.abs(got.astype(np.float64) - want).max()
    say(f"    max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL


@pytest.mark.parametrize("mode", ["1e5", "1e20", "spikes"])
def test_prefill_values_beyond_fp16_range(mode):
    # Paging leaves the attention result unchanged ([HRL] section 8) over the whole bf16
    # range of V, not only where a narrower type could hold it: V scaled by 1e5 (beyond
    # fp16's 65,504), by 1e20, or N(0,1) with 1 % of the entries scaled by 1e20.  The bar is
    # the 2e-3 parity bound scaled by max|V| (the output is a convex combination of V rows,
    # so every error term of the kernel -- the P parts' 2^-15, fp32 sums -- scales with it).
    from workloads import to_bf16_bits
    hkv, G, D, B = 2, 4, 128, 16
    ctx, chunk = [300, 130, 77], [300, 64, 1]
    nb = sum(-(-L // B) for L in ctx) + 8
    w = make_prefill_custom(name=f"prefill-range-{mode}", seed=71, dtype="bf16", num_blocks=nb,
                            num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D, block_size=B,
                            context_lens=ctx, chunk_lens=chunk)
    rng = np.random.default_rng(72)

    def scaled(bits):
        x = paged.to_f64(bits)
        if mode == "1e5":
            x = x * 1e5
        elif mode == "1e20":
            x = x * 1e20
        else:
            x = np.where(rng.random(x.shape) < 0.01, x * 1e20, x)
        return to_bf16_bits(x.astype(np.float32))

    w.pool[:, 1] = scaled(w.pool[:, 1])
    w.v_new = scaled(w.v_new)
    say(f"[prefill range] V {mode}")
    pool, got = gpu_prefill(w)
    pool_np = oracle_pool(w)
    assert to_host(pool.data).tobytes() == pool_np.tobytes()
    vmax = float(np.nanmax(np.abs(paged.to_f64(pool_np[:, 1]))))
    want = paged.prefill_ref(pool_np, w.q, w.query_start_loc, w.context_lens, w.block_tables, float(w.scale))
    err = float(np.abs(got.astype(np.float64) - want).max())
    say(f"    max|V| {vmax:.3e}, max abs err {err:.3e} = {err / vmax:.2e} of max|V|")
    assert vmax > 65504.0
    assert np.isfinite(got).all() and err <= ATOL * max(1.0, vmax)


def test_prefill_rows_past_max_query_len_are_nan():
    # a sequence with more rows than max_query_len states is inconsistent: all of its rows
    # inside the output are NaN, also those past the row tiles the grid has (max_query_len
    # sizes the grid), and the other sequences are unaffected
    w = make_prefill_custom(name="prefill-long-rows", seed=81, dtype="bf16", num_blocks=64, num_q_heads=8,
                            num_kv_heads=2, head_dim=128, block_size=16, context_lens=[300, 40],
                            chunk_lens=[200, 10])
    say("[prefill rows past max_query_len]")
    pool_np = oracle_pool(w)
    pool = pa.PagedKVPool(to_dev(pool_np, "bf16"))
    out = torch.zeros((w.total_tokens, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda:0")
    pa.pa_prefill(pool, to_dev(w.q, "bf16"), i32(w.query_start_loc), i32(w.context_lens), i32(w.block_tables),
                  scale=float(w.scale), max_query_len=10, out=out)
    got = out.cpu().numpy()
    assert np.isnan(got[0:200]).all()
    want = paged.prefill_ref(pool_np, w.q, w.query_start_loc, w.context_lens, w.block_tables, float(w.scale))
    assert np.abs(got[200:210] - want[200:210]).max() <= ATOL
