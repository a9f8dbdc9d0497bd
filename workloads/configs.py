"""The five decode workloads, seeded, plus reduced variants for fast parity runs.

Every workload is a description of one or more decode steps over a block
pool.  Context lengths count the token written in that step (the new token
goes to position ``length - 1`` and the step's query attends over all
``length`` positions).  Pools are numpy arrays ``[N][2][Hkv][B][D]`` holding
float32 values, or bf16 bit patterns as uint16.  Blocks that hold no token of
any sequence are filled with NaN so that a kernel reading outside a
sequence's blocks cannot go unnoticed.

Seeds (reduced variants use ``100 + k`` in place of ``k``): workloads 2 and
3 draw their lengths from ``numpy.random.default_rng(k)`` and everything
else -- block placement, resident K/V contents, then per step the query and
the new tokens' K and V, in that order -- from ``default_rng(k + 1000)``;
workload 5 draws its lengths from ``default_rng(5)`` (or the next seed that
fits the pool) and the rest from that seed plus 1000; workloads 1 and 4
draw placement, contents and steps from ``default_rng(k)``.  The
tensor-parallel share of workload 4 uses ``default_rng(4 + 1000 * tp)``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CONFIG_NAMES = {
    1: "worked example: lengths 25/47/12, B16, 16-block pool, 4/4 heads, D64, fp32",
    2: "Qwen3-8B layer, batch 64, context 4,100-4,164, B16, bf16, 38,348-block pool",
    3: "Qwen3-8B layer, batch 128, context 12-2,048, 512-token prefix shared by groups of 4, B16, bf16",
    4: "70B-shaped layer, batch 8 x 32,768, 64/8 heads, B32, bf16, 8,192-block pool",
    5: "Qwen3-8B layer, 512 lognormal contexts (median 600), 32 decode steps, B16, bf16, 38,348-block pool",
}

_BF16_NAN = np.uint16(0x7FC0)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs must be finite.  Adding 0x7FFF plus the lowest kept bit and
    truncating the low 16 bits is round-to-nearest-even on the bit pattern.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return to_bf16_bits(x) if dtype == "bf16" else x


def _blocks_for(num_tokens: int, block_size: int) -> int:
    # table rows are sized to hold the tokens (rounded up to whole blocks)
    return (int(num_tokens) + block_size - 1) // block_size


@dataclass
class Step:
    """One decode step: copy-on-write copies, the cache write, then decode."""

    context_lens: np.ndarray  # int32 [S], after this step's write
    q: np.ndarray  # [S][Hq][D] storage dtype
    k_new: np.ndarray  # [T][Hkv][D] storage dtype, T = len(write_seq)
    v_new: np.ndarray
    write_seq: np.ndarray  # int32 [T]: sequence of each written token
    write_pos: np.ndarray  # int32 [T]: its position
    cow_src: np.ndarray  # int32 [P]: shared blocks copied before the write
    cow_dst: np.ndarray  # int32 [P]: the fresh blocks they are copied to
    new_blocks: list = field(default_factory=list)  # (seq, logical index, block) taken this step


@dataclass
class Workload:
    name: str
    dtype: str  # "f32" | "bf16"
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: np.float32
    pool: np.ndarray  # state before the first step
    block_tables: np.ndarray  # int32 [S][max_blocks]; entries past a sequence's blocks are the pad id
    steps: list
    null_block: int | None = None
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def kv_bytes(self, step: int = 0) -> int:
        """K and V bytes of the live context tokens read by one decode of ``step``."""
        lens = self.steps[step].context_lens.astype(np.int64)
        return int(lens.sum()) * 2 * self.num_kv_heads * self.head_dim * self.elem_bytes


def _empty_pool(num_blocks, num_kv_heads, block_size, head_dim, dtype):
    shape = (num_blocks, 2, num_kv_heads, block_size, head_dim)
    if dtype == "bf16":
        return np.full(shape, _BF16_NAN, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


def _fill_blocks(pool, blocks, rng, dtype, chunk=256):
    blocks = np.asarray(sorted(set(int(b) for b in blocks)), dtype=np.int64)
    per_block = pool.shape[1:]
    for i in range(0, len(blocks), chunk):
        sel = blocks[i:i + chunk]
        pool[sel] = _normal(rng, (len(sel),) + per_block, dtype)


def _tables_array(rows, pad):
    width = max(1, max(len(r) for r in rows))
    out = np.full((len(rows), width), pad, dtype=np.int32)
    for s, r in enumerate(rows):
        out[s, :len(r)] = r
    return out


def _decode_step(rng, lens, num_q_heads, num_kv_heads, head_dim, dtype, cow_src=(), cow_dst=(), new_blocks=()):
    S = len(lens)
    q = _normal(rng, (S, num_q_heads, head_dim), dtype)
    k_new = _normal(rng, (S, num_kv_heads, head_dim), dtype)
    v_new = _normal(rng, (S, num_kv_heads, head_dim), dtype)
    return Step(
        context_lens=np.asarray(lens, dtype=np.int32),
        q=q, k_new=k_new, v_new=v_new,
        write_seq=np.arange(S, dtype=np.int32),
        write_pos=(np.asarray(lens, dtype=np.int32) - 1),
        cow_src=np.asarray(cow_src, dtype=np.int32), cow_dst=np.asarray(cow_dst, dtype=np.int32),
        new_blocks=list(new_blocks),
    )


def make_custom(*, name, seed, dtype, num_blocks, num_q_heads, num_kv_heads, head_dim, block_size,
                lengths, placement="free_list", prefix_tokens=0, group=4, num_steps=1):
    """General builder behind every workload.

    ``placement``: ``"free_list"`` keeps block 0 as the null block and pops
    the other blocks from a seeded shuffle of the free list; ``"permutation"``
    uses a seeded permutation of the whole pool.  ``prefix_tokens > 0``
    makes each run of ``group`` consecutive sequences share the blocks of a
    common prefix of that many tokens; a sequence whose write lands in a
    shared block gets a fresh block and a copy first when others still hold
    it, and writes in place when it is the last holder.  ``num_steps > 1``
    grows every sequence by one token per step, taking a fresh block from the
    free list when a write starts a new block.
    """
    rng = np.random.default_rng(seed)
    B = block_size
    lengths = np.asarray(lengths, dtype=np.int64)
    S = len(lengths)
    if placement == "free_list":
        free = list(rng.permutation(np.arange(1, num_blocks)))
        null_block, pad = 0, 0
    elif placement == "permutation":
        free = list(rng.permutation(np.arange(num_blocks)))
        null_block, pad = None, 0
    else:
        raise ValueError(placement)
    free.reverse()  # pop() from the end == take the front of the shuffled queue

    def take():
        if not free:
            raise RuntimeError(f"{name}: pool of {num_blocks} blocks exhausted")
        return int(free.pop())

    rows = [[] for _ in range(S)]
    resident = set()  # blocks whose contents are drawn now
    cow_src, cow_dst = [], []
    if prefix_tokens:
        prefix_blocks = prefix_tokens // B
        assert prefix_blocks * B == prefix_tokens, "the shared prefix must be whole blocks"
        for g0 in range(0, S, group):
            members = list(range(g0, min(S, g0 + group)))
            n_need = [_blocks_for(lengths[s], B) for s in members]
            shared = [take() for _ in range(min(prefix_blocks, max(n_need)))]
            resident.update(shared)
            holders = {b: 0 for b in shared}
            for s, n in zip(members, n_need):
                for j in range(n):
                    if j < prefix_blocks:
                        rows[s].append(shared[j])
                        holders[shared[j]] += 1
                    else:
                        b = take()
                        rows[s].append(b)
                        resident.add(b)
            for s in members:
                j = int(lengths[s] - 1) // B
                if j < prefix_blocks:
                    b = rows[s][j]
                    if holders[b] > 1:
                        fresh = take()
                        holders[b] -= 1
                        rows[s][j] = fresh
                        cow_src.append(b)
                        cow_dst.append(fresh)
    else:
        for s in range(S):
            rows[s] = [take() for _ in range(_blocks_for(lengths[s], B))]
            resident.update(rows[s])

    # blocks the later steps take, in step order then sequence order
    growth = [[] for _ in range(num_steps)]
    for k in range(1, num_steps):
        for s in range(S):
            pos = int(lengths[s]) + k - 1
            if pos % B == 0:
                b = take()
                growth[k].append((s, len(rows[s]), b))
                rows[s].append(b)

    tables = _tables_array(rows, pad)
    pool = _empty_pool(num_blocks, num_kv_heads, B, head_dim, dtype)
    _fill_blocks(pool, resident, rng, dtype)

    steps = []
    for k in range(num_steps):
        steps.append(_decode_step(rng, lengths + k, num_q_heads, num_kv_heads, head_dim, dtype,
                                  cow_src if k == 0 else (), cow_dst if k == 0 else (), growth[k]))
    scale = np.float32(1.0) / np.sqrt(np.float32(head_dim))
    return Workload(name=name, dtype=dtype, num_blocks=num_blocks, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=B, scale=np.float32(scale),
                    pool=pool, block_tables=tables, steps=steps, null_block=null_block,
                    meta={"prefix_tokens": prefix_tokens, "group": group, "placement": placement})


def _lognormal_lengths(rng, n, median, sigma, lo, hi):
    return np.clip(np.rint(rng.lognormal(mean=np.log(median), sigma=sigma, size=n)), lo, hi).astype(np.int64)


def _config5_lengths(small: bool):
    """Workload 5's lognormal lengths and the seed that drew them (redrawn until they fit)."""
    if small:
        S, median, hi, n, steps, seed = 24, 60, 2048, 1024, 4, 105
    else:
        S, median, hi, n, steps, seed = 512, 600, 40960, 38348, 32, 5
    s = seed
    while True:
        rng = np.random.default_rng(s)
        lens = _lognormal_lengths(rng, S, median, 1.0, 1, hi)
        need = sum(_blocks_for(L + steps - 1, 16) for L in lens)
        if need <= n - 1:
            return lens, s
        s += 1


def config_lengths(k: int, small: bool = False) -> np.ndarray:
    """Context lengths of workload 2 or 5 (step 0)."""
    if k == 2:
        rng = np.random.default_rng((100 + k) if small else k)
        return rng.integers(100, 165, size=6) if small else rng.integers(4100, 4165, size=64)
    if k == 5:
        return _config5_lengths(small)[0]
    raise ValueError(f"no length recipe for workload {k}")


def make_block_size_sweep(k: int, sizes):
    """Workload 2 or 5 (one decode step) stored at each block size in ``sizes``, in turn.

    The tokens' K/V, the query and the step's new K/V are drawn once (token
    major), so every block size holds the same contents; each size keeps the
    same cache memory (613,568 token slots re-cut into 613,568 / B blocks) and
    places the sequences' blocks by the seeded free-list recipe.  Slots past a
    sequence's tokens are NaN."""
    lens = config_lengths(k).astype(np.int64)
    S = len(lens)
    Hq, Hkv, D = 32, 8, 128
    rng = np.random.default_rng(3000 + k)
    resident = lens - 1  # the step writes position L - 1
    kv = _normal(rng, (int(resident.sum()), 2, Hkv, D), "bf16")
    step = _decode_step(rng, lens, Hq, Hkv, D, "bf16")
    offs = np.concatenate([[0], np.cumsum(resident)])
    scale = np.float32(1.0) / np.sqrt(np.float32(D))
    for B in sizes:
        n = 613568 // B
        prng = np.random.default_rng(4000 + 1000 * k + B)
        free = list(prng.permutation(np.arange(1, n)))
        free.reverse()
        rows = [[int(free.pop()) for _ in range(_blocks_for(L, B))] for L in lens]
        pool = _empty_pool(n, Hkv, B, D, "bf16")
        for s in range(S):
            nb = len(rows[s])
            buf = np.full((nb * B, 2, Hkv, D), _BF16_NAN, dtype=np.uint16)
            buf[:resident[s]] = kv[offs[s]:offs[s + 1]]
            pool[rows[s]] = buf.reshape(nb, B, 2, Hkv, D).transpose(0, 2, 3, 1, 4)
        yield Workload(name=f"cfg{k}-block-size-{B}", dtype="bf16", num_blocks=n, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, block_size=B, scale=np.float32(scale), pool=pool,
                       block_tables=_tables_array(rows, 0), steps=[step], null_block=0,
                       meta={"prefix_tokens": 0, "placement": "free_list"})


def make_config(k: int, small: bool = False) -> Workload:
    """Workload ``k`` (1-5).  ``small=True`` keeps its shapes and structure at sizes
    the oracle checks in seconds (several tiles, a ragged tail)."""
    seed = (100 + k) if small else k
    if k == 1:
        return make_custom(name="cfg1-worked", seed=seed, dtype="f32", num_blocks=16, num_q_heads=4,
                           num_kv_heads=4, head_dim=64, block_size=16, lengths=[25, 47, 12],
                           placement="permutation")
    if k == 2:
        lens = config_lengths(2, small)
        n = 1024 if small else 38348
        return make_custom(name="cfg2-qwen3-8b-b64" + ("-small" if small else ""), seed=seed + 1000,
                           dtype="bf16", num_blocks=n, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=16, lengths=lens)
    if k == 3:
        rng = np.random.default_rng(seed)
        if small:
            lens = rng.integers(12, 300, size=12)
            n, prefix = 1024, 128
        else:
            lens = rng.integers(12, 2049, size=128)
            n, prefix = 38348, 512
        return make_custom(name="cfg3-mixed-prefix" + ("-small" if small else ""), seed=seed + 1000,
                           dtype="bf16", num_blocks=n, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=16, lengths=lens, prefix_tokens=prefix, group=4)
    if k == 4:
        if small:
            S, L, n = 2, 2048, 128
        else:
            S, L, n = 8, 32768, 8192
        return make_custom(name="cfg4-70b-long" + ("-small" if small else ""), seed=seed, dtype="bf16",
                           num_blocks=n, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=32,
                           lengths=[L] * S, placement="permutation")
    if k == 5:
        n, steps = (1024, 4) if small else (38348, 32)
        lens, s = _config5_lengths(small)
        return make_custom(name="cfg5-high-concurrency" + ("-small" if small else ""), seed=s + 1000,
                           dtype="bf16", num_blocks=n, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=16, lengths=lens, num_steps=steps)
    raise ValueError(f"no workload {k}")


def make_tp_share(tp: int = 8) -> Workload:
    """One GPU's share of the 70B-shaped long-context workload under tensor
    parallelism over heads: the same 8 sequences of 32,768 tokens, 32-token
    blocks and whole-pool permutation placement, with 8 / tp KV heads and
    64 / tp query heads (tp = 8: one KV head serving eight query heads)."""
    assert 8 % tp == 0
    return make_custom(name=f"cfg4-70b-long-tp{tp}-share", seed=4 + 1000 * tp, dtype="bf16", num_blocks=8192,
                       num_q_heads=64 // tp, num_kv_heads=8 // tp, head_dim=128, block_size=32,
                       lengths=[32768] * 8, placement="permutation")


# ---------------------------------------------------------------------------
# prefill workloads
# ---------------------------------------------------------------------------

PREFILL_NAMES = {
    1: "prefill: 4 prompts x 4,100 tokens (whole prompt at once), Qwen3-8B layer, B16, bf16",
    2: "chunked prefill: 16 requests, a 4,000-token prefix shared and cached, 100-token private chunk each, "
       "Qwen3-8B layer, B16, bf16",
}


@dataclass
class PrefillWorkload:
    name: str
    dtype: str
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: np.float32
    pool: np.ndarray            # positions before each chunk are resident
    block_tables: np.ndarray    # int32 [S][max_blocks]
    context_lens: np.ndarray    # int32 [S], chunk included
    query_start_loc: np.ndarray  # int32 [S+1]
    q: np.ndarray               # [T][Hq][D]
    k_new: np.ndarray           # [T][Hkv][D]: the chunk's K, written by the cache write first
    v_new: np.ndarray
    write_seq: np.ndarray       # int32 [T]
    write_pos: np.ndarray       # int32 [T]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    def attention_flops(self) -> int:
        """QK and PV multiply-adds (2 flops each) of the causal rows: 4*D*Hq per (row, key)."""
        keys = 0
        for s in range(self.num_seqs):
            n = int(self.query_start_loc[s + 1] - self.query_start_loc[s])
            ctx = int(self.context_lens[s])
            first = ctx - n + 1  # keys seen by the chunk's first row
            keys += n * first + n * (n - 1) // 2
        return 4 * self.head_dim * self.num_q_heads * keys


def make_prefill_custom(*, name, seed, dtype, num_blocks, num_q_heads, num_kv_heads, head_dim, block_size,
                        context_lens, chunk_lens, shared_prefix_tokens=0):
    """Sequences whose last ``chunk_lens[s]`` positions are this step's queries.

    Positions before the chunk are resident in the pool (drawn here); the
    chunk's K/V are returned for the cache write.  With
    ``shared_prefix_tokens`` (whole blocks), every sequence's table starts with
    the same physical blocks holding one common prefix.
    """
    rng = np.random.default_rng(seed)
    B = block_size
    ctx = np.asarray(context_lens, dtype=np.int64)
    n = np.asarray(chunk_lens, dtype=np.int64)
    assert (n >= 1).all() and (n <= ctx).all()
    S = len(ctx)
    free = list(rng.permutation(np.arange(1, num_blocks)))
    free.reverse()

    def take():
        return int(free.pop())

    shared = []
    if shared_prefix_tokens:
        assert shared_prefix_tokens % B == 0 and (ctx - n >= shared_prefix_tokens).all()
        shared = [take() for _ in range(shared_prefix_tokens // B)]
    rows = []
    for s in range(S):
        row = list(shared)
        while len(row) < _blocks_for(ctx[s], B):
            row.append(take())
        rows.append(row)
    tables = _tables_array(rows, 0)
    pool = _empty_pool(num_blocks, num_kv_heads, B, head_dim, dtype)
    _fill_blocks(pool, set(b for r in rows for b in r), rng, dtype)
    T = int(n.sum())
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(n)
    q = _normal(rng, (T, num_q_heads, head_dim), dtype)
    k_new = _normal(rng, (T, num_kv_heads, head_dim), dtype)
    v_new = _normal(rng, (T, num_kv_heads, head_dim), dtype)
    write_seq = np.repeat(np.arange(S, dtype=np.int32), n)
    write_pos = np.concatenate([np.arange(ctx[s] - n[s], ctx[s]) for s in range(S)]).astype(np.int32)
    scale = np.float32(1.0) / np.sqrt(np.float32(head_dim))
    return PrefillWorkload(name=name, dtype=dtype, num_blocks=num_blocks, num_q_heads=num_q_heads,
                           num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=B, scale=np.float32(scale),
                           pool=pool, block_tables=tables, context_lens=ctx.astype(np.int32), query_start_loc=qsl,
                           q=q, k_new=k_new, v_new=v_new, write_seq=write_seq, write_pos=write_pos,
                           meta={"shared_prefix_tokens": shared_prefix_tokens})


def make_prefill(k: int, small: bool = False) -> PrefillWorkload:
    """Prefill workload ``k`` (1-2); ``small`` keeps the structure at oracle-friendly sizes."""
    seed = 200 + k + (100 if small else 0)
    if k == 1:
        if small:
            lens, n_blocks = [130, 77, 64, 1], 64
        else:
            lens, n_blocks = [4100] * 4, 38348
        return make_prefill_custom(name="prefill-4x4100" + ("-small" if small else ""), seed=seed, dtype="bf16",
                                   num_blocks=n_blocks, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                   block_size=16, context_lens=lens, chunk_lens=lens)
    if k == 2:
        if small:
            S, prefix, chunk, n_blocks = 3, 96, 37, 64
        else:
            S, prefix, chunk, n_blocks = 16, 4000, 100, 38348
        return make_prefill_custom(name="chunked-prefill-shared-prefix" + ("-small" if small else ""), seed=seed,
                                   dtype="bf16", num_blocks=n_blocks, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                   block_size=16, context_lens=[prefix + chunk] * S, chunk_lens=[chunk] * S,
                                   shared_prefix_tokens=prefix)
    raise ValueError(f"no prefill workload {k}")


# ---------------------------------------------------------------- token-determined K/V for prefix caching


@dataclass
class TokenModel:
    """Stand-in for a model layer whose K, V and Q depend only on (token id, position).

    Two prompts with the same leading tokens then hold bit-identical K/V over
    that prefix, which is what lets a cached block stand in for recomputing
    it.  Values are embedding-plus-position sums rounded to bf16; nothing of
    the attention method is computed here.
    """

    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    embed: np.ndarray  # float32 [vocab][Hq + 2 Hkv][D]
    pos: np.ndarray    # float32 [max_pos][Hq + 2 Hkv][D]

    def _rows(self, ids, positions):
        ids = np.asarray(ids, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        return self.embed[ids] + self.pos[positions]

    def qkv(self, ids, positions):
        """(q [T][Hq][D], k [T][Hkv][D], v [T][Hkv][D]) as bf16 bit patterns."""
        x = to_bf16_bits(self._rows(ids, positions))
        hq, hkv = self.num_q_heads, self.num_kv_heads
        return (np.ascontiguousarray(x[:, :hq]), np.ascontiguousarray(x[:, hq:hq + hkv]),
                np.ascontiguousarray(x[:, hq + hkv:]))


def make_token_model(seed: int, vocab: int, max_pos: int, num_q_heads: int, num_kv_heads: int,
                     head_dim: int) -> TokenModel:
    rng = np.random.default_rng(seed)
    rows = num_q_heads + 2 * num_kv_heads
    embed = rng.standard_normal((vocab, rows, head_dim), dtype=np.float32)
    pos = 0.5 * rng.standard_normal((max_pos, rows, head_dim), dtype=np.float32)
    return TokenModel(num_q_heads, num_kv_heads, head_dim, embed, pos)
