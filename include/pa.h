/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV-cache decode path.
 *
 * The operations follow the pages this library was built from:
 *   [AINEW] "PagedAttention: KV-cache virtual memory technique improves
 *           inference efficiency" (news.ainew.jp; the title is Japanese on
 *           the page)
 *   [SALIV] "How PagedAttention Eliminates KV-Cache Fragmentation"
 *   [VIBE]  "PagedAttention, explained." (vibeengines.com)
 *   [HRL]   "What Does PagedAttention Actually Optimize?" (hrletsgo.me)
 *   [TSS]   "Paged Attention: Virtual Memory for the KV Cache"
 *           (theservingstack.com)
 *
 * General contract (every entry point):
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise;
 *     the pa_pool descriptor itself is a host struct read during the call.
 *   - A call validates its scalar arguments on the host, enqueues its
 *     kernels on `stream` and returns; it never synchronises the stream.
 *   - The caller owns all memory.  The library allocates nothing and keeps
 *     no pointer after the call returns.
 *   - Scalar errors return a negative pa_status and enqueue nothing.  A
 *     failed launch returns PA_ERR_HIP.  A call with zero work returns PA_OK
 *     and enqueues nothing.
 *   - Device contents are the caller's contract.  Kernels never access
 *     memory outside the buffers described here, whatever those contents
 *     are: an out-of-range id or slot is skipped (writes, copies, slot
 *     mapping) or turns the affected outputs into NaN (decode), as each
 *     entry point states.
 *   - Calls that overlap on one stream run in order; calls on different
 *     streams that touch the same pool region race.
 *
 * Checked mode (environment variable PA_CHECK=1, read at every call):
 *   before launching, an entry point copies the index arrays it was given
 *   (slots, seq ids, positions, tables, lengths, copy pairs, query starts)
 *   to the host, waits for them, and returns PA_ERR_INVALID_ARG without
 *   launching anything when it finds
 *     - a written slot outside the pool, or two tokens of one write with the
 *       same slot ([TSS] "Finding a token": one slot per token);
 *     - a token whose sequence id lies outside [0, num_seqs) or whose
 *       position lies beyond its table row (a negative position is padding
 *       and passes);
 *     - a copy pair with an id outside its pool, two pairs with the same
 *       destination, or (inside one pool) a destination that is also a
 *       source ([AINEW] copy-on-write passage: the shared block is never
 *       written in place);
 *     - a context length that is negative, exceeds max_context_len or the
 *       table row, or a table id outside [0, num_blocks) among the first
 *       ceil(len / block_size) entries of a row that attention reads;
 *     - prefill bounds that are inconsistent (see pa_prefill).
 *   Checked mode synchronises the stream and allocates host memory, so it is
 *   a debugging aid: under graph capture it returns PA_ERR_UNSUPPORTED.
 *   Without it (the default) the kernels skip such entries or return NaN
 *   rows, as each entry point states, and never touch memory outside the
 *   described buffers.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes */
  PA_ERR_UNSUPPORTED = -2, /* a shape or dtype this build has no kernel for   */
  PA_ERR_WORKSPACE = -3,   /* decode workspace missing or too small           */
  PA_ERR_HIP = -4          /* the HIP runtime rejected a launch               */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/*
 * pa_decode flags.
 *   PA_DECODE_STREAM (0): K/V loads carry the non-temporal hint.  Each byte
 *     of K/V is read once per step, so nothing worth keeping is evicted from
 *     L2 (the faster choice when sequences do not share blocks).
 *   PA_DECODE_KEEP_CACHED: K/V loads use the normal cache policy.  Pass it
 *     when sequences of the batch share physical blocks (a common prefix,
 *     [AINEW] copy-on-write passage; [TSS] "Sharing a prefix"): the later
 *     readers of a shared block then hit in L2.
 */
typedef enum { PA_DECODE_STREAM = 0, PA_DECODE_KEEP_CACHED = 1 } pa_decode_flags;

/*
 * The physical block pool ([AINEW] "PagedAttention in one picture";
 * [TSS] "Paging": fixed-size blocks carved out of the cache memory).
 * `base` points at num_blocks * 2 * num_kv_heads * block_size * head_dim
 * elements laid out as [num_blocks][2][num_kv_heads][block_size][head_dim]:
 * index 0 of the second axis holds K and index 1 holds V, so one physical
 * block is one contiguous chunk and each (block, head) K or V tile is
 * contiguous.  Supported: block_size a power of two up to 256 (slot
 * mapping, cache write, block copy, swap), of which pa_decode and
 * pa_prefill take 4, 8, 16, 32, 64 and 128 ([AINEW] block-size figure, 4 /
 * 16 / 64; [VIBE] evaluation, 16 to 128); head_dim 64 or 128; dtype PA_F32
 * or PA_BF16 (bf16 = upper half of an IEEE binary32).
 */
typedef struct {
  void *base;
  int64_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t dtype; /* pa_dtype */
} pa_pool;

/*
 * Slot of each token written this step ([TSS] "Finding a token: position,
 * block, slot": the slot is the physical block times the block size plus the
 * offset inside the block; [HRL] section 5 for the table lookup).
 *   block_tables : int32 [num_seqs][max_blocks_per_seq], physical block ids.
 *   seq_ids      : int32 [num_tokens], the sequence of each token.
 *   positions    : int32 [num_tokens], its position inside that sequence.
 *   slot_mapping : int64 [num_tokens], output.
 * slot = block_tables[seq][pos / block_size] * block_size + pos % block_size.
 * A token whose seq id lies outside [0, num_seqs), whose position is
 * negative or beyond the table row, or whose table entry lies outside
 * [0, num_blocks) gets slot -1 (which pa_cache_write skips).
 */
int pa_slot_mapping(const pa_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                    int32_t num_seqs, const int32_t *seq_ids, const int32_t *positions,
                    int64_t *slot_mapping, int32_t num_tokens, hipStream_t stream);

/*
 * Scatter each new token's K and V into its slot ([VIBE] vLLM procedure
 * step 4; [HRL] section 17 `write_kv`; the fused write kernel named in
 * [VIBE] "Across GPUs").
 *   k_new, v_new : [num_tokens][num_kv_heads][head_dim], pool dtype.
 *   slot_mapping : int64 [num_tokens].
 * pool[slot / B][0][h][slot % B][:] = k_new[i][h][:] and likewise V at index
 * 1, for every head, copied bit for bit.  Negative slots and slots at or
 * beyond num_blocks * block_size are skipped.  Two tokens with the same slot
 * in one call is a caller error (which one lands is unspecified; checked
 * mode refuses it).
 */
int pa_cache_write(const pa_pool *pool, const void *k_new, const void *v_new,
                   const int64_t *slot_mapping, int32_t num_tokens, hipStream_t stream);

/*
 * pa_slot_mapping and pa_cache_write in one launch: token i's slot is
 * computed from (seq_ids[i], positions[i]) through block_tables exactly as
 * pa_slot_mapping computes it, and its K and V rows are written there as
 * pa_cache_write writes them (a token whose slot is -1 is skipped).  The
 * pages' step writes the new token's K/V at its (block, offset) slot right
 * after finding it ([TSS] "Finding a token"; [VIBE] vLLM procedure step 4);
 * doing both in one kernel saves a launch per decode step.
 *   k_new, v_new : [num_tokens][num_kv_heads][head_dim], pool dtype.
 *   block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions : as for
 *                  pa_slot_mapping.
 *   slot_mapping : int64 [num_tokens] receiving the slots, or NULL.
 * Same argument checks and errors as the two calls; two tokens with the
 * same slot in one call is a caller error (refused in checked mode).
 */
int pa_cache_write_at(const pa_pool *pool, const void *k_new, const void *v_new, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, int32_t num_seqs, const int32_t *seq_ids,
                      const int32_t *positions, int64_t *slot_mapping, int32_t num_tokens, hipStream_t stream);

/*
 * Whole-block copies for copy-on-write ([AINEW] copy-on-write passage;
 * [SALIV] "Advanced Memory Sharing and Copy-on-Write"; [VIBE] step 6 and
 * the block-copy kernel named in "Across GPUs").
 *   src_blocks, dst_blocks : int32 [num_pairs].
 * pool[dst[j]] = pool[src[j]] for every pair: K and V, every head, every
 * slot.  A pair with an id outside [0, num_blocks) is skipped.  Destinations
 * must be distinct and must not appear among the sources (else the result
 * is unspecified; checked mode refuses such pairs).
 */
int pa_block_copy(const pa_pool *pool, const int32_t *src_blocks, const int32_t *dst_blocks,
                  int32_t num_pairs, hipStream_t stream);

/*
 * Swap copies: whole blocks from one pool to another of the same geometry,
 * either of which may live in pinned host memory (allocated with
 * hipHostMalloc) -- the swap-out and swap-in of [VIBE] "The vLLM procedure"
 * step 8 and [HRL] section 12.  dst->base block dst_blocks[j] receives
 * src->base block src_blocks[j] (K and V, every head, every slot).  One
 * kernel moves every pair, the host side over the host link, instead of one
 * transfer per block.
 *   src_blocks, dst_blocks : int32 [num_pairs], device memory.
 * A pair with an id outside its pool is skipped; destinations must be
 * distinct.  Errors (nothing is launched): pools that differ in
 * num_kv_heads, block_size, head_dim or dtype, or a base that is neither
 * device memory nor pinned host memory the device addresses at the same
 * address (PA_ERR_INVALID_ARG).  The host side must stay allocated and
 * untouched by the host until the stream reaches the copy.
 */
int pa_swap_blocks(const pa_pool *src, const pa_pool *dst, const int32_t *src_blocks, const int32_t *dst_blocks,
                   int32_t num_pairs, hipStream_t stream);

/*
 * Partition size (tokens) pa_decode uses when passed partition_size == 0.
 * Returns a positive multiple of the block size, or a negative pa_status.
 * The automatic choice splits the sequences into equal partitions so a call
 * has at least 512 workgroups (256, one per compute unit, where groups of 8
 * over bf16 pools with blocks of 16 tokens or more take their scores from
 * the matrix cores), caps partitions at 2,048 tokens in batches of 1,024 or
 * more (sequence, KV head) pairs, and stays between 256 tokens and 512
 * blocks.  It depends only on these arguments.
 */
int32_t pa_decode_partition_size(const pa_pool *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len);

/*
 * Device workspace bytes pa_decode needs for these arguments (the
 * split-context partials and, for skewed batches of many pairs, the work
 * list): 0 when every sequence fits one partition (no workspace needed), or
 * a negative
 * pa_status for arguments pa_decode would refuse (a bad pool, negative
 * sizes, num_q_heads not a multiple of num_kv_heads, a partition_size that
 * is not a multiple of max(block_size, 16) or exceeds 2,048 blocks).  The pool
 * descriptor stands for the separate KV-head count and head size of a plain
 * shape signature (it also fixes the block size, which the automatic
 * partition depends on), and partition_size is the one pa_decode will get,
 * since the partial results grow with the number of partitions.
 */
int64_t pa_decode_workspace_size(const pa_pool *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * One decode step of paged attention ([VIBE] step 5: the kernel fetches key
 * and value blocks through the table, block by block; [HRL] section 8: the
 * result is ordinary softmax(q K^T * scale) V; [HRL] section 14: per token,
 * logical block, physical block, offset, read).
 *   q            : [num_seqs][num_q_heads][head_dim], pool dtype.
 *   out          : float32 [num_seqs][num_q_heads][head_dim], output.
 *   block_tables : int32 [num_seqs][max_blocks_per_seq].
 *   context_lens : int32 [num_seqs], tokens each query attends over (the
 *                  token written this step included).
 *   scale        : multiplier of q.k (usually 1/sqrt(head_dim)).
 *   max_context_len : host-known upper bound of context_lens.
 *   partition_size  : tokens per split-context partition; 0 = automatic;
 *                  else a positive multiple of max(block_size, 16), at
 *                  most 2,048 blocks.
 *   flags        : PA_DECODE_STREAM or PA_DECODE_KEEP_CACHED (see above).
 *   workspace    : scratch for split-context partial results, at least
 *                  pa_decode_workspace_size() bytes, 256-byte aligned (may
 *                  be NULL when that size is 0).  Contents need no
 *                  initialisation.
 * Calls sharing a workspace must not overlap in time (calls on one stream
 * never do).  A call launches one kernel, plus a small combine kernel when
 * some sequence spans more than one partition.  Batches of 1,024 or more
 * (sequence, KV head) pairs whose sequences may span several partitions
 * (skewed lengths) first launch a one-workgroup prepass that lists the
 * (pair, partition) items with work, longest first, in the workspace; the
 * decode's resident workgroups then take items from that list (results are
 * the same bits as without it).  Query head hq reads KV head
 * hq / (num_q_heads / num_kv_heads); the group size must be 1, 2, 4 or 8.
 * At most 65,535 sequences, and (num_seqs * num_kv_heads + 8) * partitions
 * below 2^31 (PA_ERR_UNSUPPORTED otherwise).
 * Output rows of a sequence with a context length of 0 are zero; rows of a
 * sequence whose context length is negative, exceeds max_context_len or its
 * table row, or whose table holds an id outside [0, num_blocks) among its
 * first ceil(len / block_size) entries, are NaN.
 */
int pa_decode(const pa_pool *pool, const void *q, float *out, const int32_t *block_tables,
              int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
              int32_t num_q_heads, float scale, int32_t max_context_len, int32_t partition_size,
              int32_t flags, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode without allocation, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments, kernels and results as pa_decode
 * with no workspace arguments.  The split-context partials go to a static
 * device array of the library, 32 MiB on each device it runs on, held until
 * the process ends; a call whose partials need more (see
 * pa_decode_workspace_size) returns PA_ERR_WORKSPACE and launches nothing.
 * Every call on one device shares that array and leaves its contents behind
 * (nothing in it needs clearing: each call writes every partial it reads), so
 * calls that overlap in time on one device race -- calls on one stream never
 * do.  `stream` must belong to the current device (PA_ERR_INVALID_ARG
 * otherwise).  The first call on a device looks the array's address up
 * (hipGetSymbolAddress); no call allocates, frees or synchronises.  Checked
 * mode does not apply here (it allocates host memory).
 */
int pa_decode_noalloc(const pa_pool *pool, const void *q, float *out, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                      int32_t num_q_heads, float scale, int32_t max_context_len, int32_t partition_size,
                      int32_t flags, hipStream_t stream);

/*
 * Prefill or chunked prefill: many query rows per sequence, causal
 * ([HRL] section 9, prefill computes a prompt's tokens together; [TSS]
 * "Next", chunked prefill takes a prompt a chunk at a time; [HRL] section 8
 * for the formula).  The K/V of every position must already be in the pool
 * (pa_cache_write).
 *   q               : [total_tokens][num_q_heads][head_dim], bf16.
 *   out             : float32 [total_tokens][num_q_heads][head_dim].
 *   query_start_loc : int32 [num_seqs + 1]; sequence s owns rows
 *                     query_start_loc[s] .. query_start_loc[s+1]-1, which are
 *                     its last n_s positions: row i is at position
 *                     context_lens[s] - n_s + i and attends over cached
 *                     positions 0 .. that position.
 *   context_lens    : int32 [num_seqs], cached tokens (this chunk included).
 *   block_tables    : int32 [num_seqs][max_blocks_per_seq].
 *   max_query_len   : host-known upper bound of n_s.
 * bf16 pools only: both contractions run on the bf16 matrix cores, V as
 * stored over bf16's whole range and the probabilities as two bf16 parts
 * (within 2^-15 of their fp32 values); head_dim 64 or 128; block size 4, 8,
 * 16, 32, 64 or 128; group size 1, 2, 4 or 8.  Finite results need finite K
 * and V in the context and |v| * context * 256 below the fp32 maximum (the
 * unnormalised sums are fp32).  Every row of a sequence whose bounds are
 * inconsistent (n_s < 0, n_s > context length, n_s > max_query_len, rows
 * outside [0, total_tokens), context beyond the table row) is NaN where it
 * lies inside the output, and so is every row of a row tile (256 / group
 * tokens of one KV head's query heads) whose keys take a table id outside
 * [0, num_blocks).
 */
int pa_prefill(const pa_pool *pool, const void *q, float *out, const int32_t *query_start_loc,
               const int32_t *context_lens, const int32_t *block_tables, int32_t max_blocks_per_seq,
               int32_t num_seqs, int32_t num_q_heads, int32_t total_tokens, int32_t max_query_len, float scale,
               hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *pa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
