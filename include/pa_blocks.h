/*
 * pa_blocks.h -- host-side block manager of the paged KV cache (C ABI).
 *
 * The bookkeeping around the kernels of pa.h, as the pages describe it:
 *   [TSS]   "Paging: blocks handed out as tokens arrive" and "Inside vLLM:
 *           the block pool": a pool of fixed-size blocks, a free queue
 *           taken from the front, a reference count per allocated block, a
 *           never-allocated null block 0, and ordered freeing (a block whose
 *           count reaches zero goes to the back of the queue when its
 *           contents may be reused, else to the front);
 *   [HRL]   "What Does PagedAttention Actually Optimize?" section 17
 *           (ensure_capacity: a sequence grows by one block when a write
 *           reaches past its table) and section 18 (blocks return on finish);
 *   [AINEW] copy-on-write passage, [SALIV] "Advanced Memory Sharing and
 *           Copy-on-Write", [VIBE] vLLM procedure step 6: a write into a
 *           block with more than one reference first clones it to a fresh
 *           block, drops one reference of the original and repoints only
 *           the writer's table;
 *   [TSS]   "Finding a token": slot = block * block_size + offset;
 *   [TSS]   "Sharing a prefix: one copy for many requests": prefix caching
 *           (see the prefix caching section below).
 *
 * Everything here runs on the host and touches no device memory: it emits
 * the slots, copy-on-write pairs and block tables that pa.h's kernels take.
 * A manager is not thread-safe; use one per scheduling thread.  All
 * pointers are host pointers.  Errors return a negative status (pa.h's
 * pa_status values plus PA_ERR_OUT_OF_BLOCKS) and leave the manager exactly
 * as it was before the call.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* No free block is left for the request ([VIBE] step 7: where vLLM preempts). */
#define PA_ERR_OUT_OF_BLOCKS (-5)
/* An unknown sequence id. */
#define PA_ERR_NO_SEQUENCE (-6)
/* The sequence is swapped out: only pa_bm_swap_in, pa_bm_free_sequence and
 * the queries take it. */
#define PA_ERR_SWAPPED (-7)

typedef struct pa_block_manager pa_block_manager;

/*
 * Create a manager of num_blocks blocks of block_size tokens.  With
 * reserve_null_block != 0, block 0 is never handed out.  free_order (may be
 * NULL: ascending ids) lists the initial free queue front to back; it must
 * hold distinct ids in [0, num_blocks); ids it omits start out unavailable
 * (held by something outside this manager).  The null block is dropped from
 * it.  *out receives the manager; release it with pa_bm_destroy.
 */
int pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t reserve_null_block,
                 const int32_t *free_order, int64_t free_order_len, pa_block_manager **out);
void pa_bm_destroy(pa_block_manager *bm);

/* A new, empty sequence; *seq_out receives its id (ids are never reused). */
int pa_bm_add_sequence(pa_block_manager *bm, int64_t *seq_out);

/*
 * A new sequence whose table points at the first num_shared_blocks blocks of
 * `parent` (all of them when negative), each gaining one reference; its
 * token count is min(parent's, num_shared_blocks * block_size).
 */
int pa_bm_fork(pa_block_manager *bm, int64_t parent, int32_t num_shared_blocks, int64_t *child_out);

/*
 * Prefill allocation: grow `seq` to ceil(num_tokens / block_size) blocks
 * ([VIBE] step 3) and set its token count to max(count, num_tokens).
 */
int pa_bm_allocate_prompt(pa_block_manager *bm, int64_t seq, int32_t num_tokens);

/*
 * Make position `position` of `seq` writable: grow the table to cover it,
 * then copy-on-write if the block holding it has more than one reference.
 * *slot receives the token's slot; *cow_src / *cow_dst receive the block
 * pair to copy before the write, or -1 when none is needed.  The sequence's
 * token count becomes max(count, position + 1).  The block written leaves
 * the prefix cache if it was in it (its contents change); a position whose
 * token id was committed (pa_bm_commit_tokens) is PA_ERR_INVALID_ARG.
 */
int pa_bm_prepare_write(pa_block_manager *bm, int64_t seq, int32_t position, int64_t *slot, int32_t *cow_src,
                        int32_t *cow_dst);

/*
 * One decode step for n sequences: each appends one token at its current
 * token count (growth, copy-on-write, slot), in array order.  slots_out
 * [n]; the copy-on-write pairs go to cow_src_out / cow_dst_out (room for n
 * pairs each) and their count to *num_cow_out.  All or nothing: when the
 * free queue cannot cover every new and copied block, nothing changes and
 * PA_ERR_OUT_OF_BLOCKS is returned.  A sequence listed twice is invalid.
 */
int pa_bm_append_tokens(pa_block_manager *bm, const int64_t *seqs, int32_t n, int64_t *slots_out,
                        int32_t *cow_src_out, int32_t *cow_dst_out, int32_t *num_cow_out);

/*
 * Release every block of `seq`, last block first, and forget it ([HRL]
 * section 18 step 8).  Blocks reaching zero references go to the back of the
 * free queue when reusable != 0 or when they are in the prefix cache (they
 * keep their digest until an allocation takes them), else to the front.
 */
int pa_bm_free_sequence(pa_block_manager *bm, int64_t seq, int32_t reusable);

/*
 * Block tables of n sequences as int32 [n][max_blocks_per_seq] (entries past
 * a sequence's blocks are pad_value) plus their token counts lens_out[n].
 * A sequence with more than max_blocks_per_seq blocks is an error.
 */
int pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seqs, int32_t n, int32_t max_blocks_per_seq,
                       int32_t pad_value, int32_t *tables_out, int32_t *lens_out);

/*
 * ---- Prefix caching ([TSS] "Sharing a prefix: one copy for many requests").
 *
 * Each full block of a sequence whose token ids are known has a 32-byte
 * digest chained over everything before it: d_j = SHA-256(d_{j-1} || ids of
 * block j as little-endian int32), d_{-1} = 32 zero bytes (the page fixes
 * the inputs of the hash, not the function; SHA-256 is FIPS 180-4).  The
 * manager keeps a table digest -> block.  A block enters the table when its
 * last id is known (pa_bm_allocate_prompt_cached, pa_bm_commit_tokens)
 * unless the block already has a digest or the digest already has a block;
 * it leaves when an allocation takes it from the free queue (eviction) or a
 * write changes it.  Partial blocks are never in the table.
 */

/*
 * Chained digests of the full blocks of tokens[num_tokens] (ids as given),
 * starting from `parent` (32 bytes; NULL: zeros), into digests_out
 * [num_tokens / block_size][32].  Returns the number of full blocks.
 * Stateless; needs no manager.
 */
int pa_bm_hash_blocks(const int32_t *tokens, int64_t num_tokens, int32_t block_size, const uint8_t *parent,
                      uint8_t *digests_out);

/*
 * How many tokens of a prompt tokens[num_tokens] are found in the cache: the
 * longest run of leading blocks whose digests are in the table, at most
 * floor((num_tokens - 1) / block_size) blocks (a prompt always computes at
 * least its last token), times block_size.  Changes nothing.
 */
int pa_bm_lookup_prefix(pa_block_manager *bm, const int32_t *tokens, int32_t num_tokens,
                        int32_t *num_cached_tokens);

/*
 * Prefill allocation with prefix caching for an empty sequence: the cached
 * leading blocks (as pa_bm_lookup_prefix finds them) are touched -- one more
 * reference, off the free queue if idle -- and head the table; the rest of
 * ceil(num_tokens / block_size) blocks come from the free queue.  The ids
 * are committed and every full block of the prompt enters the table.
 * *num_cached_tokens receives the tokens whose K/V need not be computed.
 * All or nothing (PA_ERR_OUT_OF_BLOCKS); a sequence with blocks or tokens
 * already is PA_ERR_INVALID_ARG.
 */
int pa_bm_allocate_prompt_cached(pa_block_manager *bm, int64_t seq, const int32_t *tokens, int32_t num_tokens,
                                 int32_t *num_cached_tokens);

/*
 * Commit the ids of the next n tokens of `seq` (after those already
 * committed; they must lie within its token count, i.e. their slots were
 * prepared) and enter every block they complete.  A forked sequence starts
 * with its parent's ids over the shared span.
 */
int pa_bm_commit_tokens(pa_block_manager *bm, int64_t seq, const int32_t *ids, int32_t n);

/* Blocks in the prefix cache table. */
int64_t pa_bm_num_cached(const pa_block_manager *bm);

/* 1 and the block's digest into digest_out[32] if it is in the table, else 0. */
int pa_bm_block_digest(const pa_block_manager *bm, int32_t block, uint8_t *digest_out);

/*
 * ---- Swapping ([VIBE] "The vLLM procedure" steps 7-8: when blocks run out,
 * all of a sequence's blocks are evicted at once, sequences sharing blocks
 * together, and evicted blocks are copied to CPU memory and back later;
 * [HRL] section 12 "Understanding Swap and Eviction").
 *
 * The manager keeps a host pool of its own (block ids 0..num_host_blocks-1,
 * a free queue taken from the front, freed blocks to the front, a count per
 * block).  The copies themselves are pa_swap_blocks (pa.h) over the pairs
 * these calls return.
 */

/* Size the host pool (ids 0..n-1, all free).  Refused while any sequence is swapped out. */
int pa_bm_set_host_pool(pa_block_manager *bm, int64_t num_host_blocks);

/*
 * Swap out the group seqs[n] (distinct sequences on the GPU).  Their tables
 * are walked in order; the first time a GPU block is met it gets a fresh
 * host block and one (GPU block, host block) pair is emitted, later holders
 * in the group share that host block; then each sequence drops its GPU
 * references, last block first (a block still held outside the group stays;
 * a block reaching zero goes to the free queue as pa_bm_free_sequence puts
 * it).  gpu_blocks_out / host_blocks_out need room for as many pairs as the
 * group has distinct blocks (at most the sum of their block counts);
 * *num_pairs_out receives the count.  All or nothing: PA_ERR_OUT_OF_BLOCKS
 * when the host pool has fewer free blocks than the group's distinct
 * blocks; PA_ERR_SWAPPED when a listed sequence is already out.
 */
int pa_bm_swap_out(pa_block_manager *bm, const int64_t *seqs, int32_t n, int32_t *gpu_blocks_out,
                   int32_t *host_blocks_out, int32_t *num_pairs_out);

/*
 * The reverse for a group of swapped-out sequences: (host block, GPU block)
 * pairs, GPU blocks from the free queue (all or nothing), host references
 * dropped last block first.  Listing a sequence on the GPU is
 * PA_ERR_INVALID_ARG.
 */
int pa_bm_swap_in(pa_block_manager *bm, const int64_t *seqs, int32_t n, int32_t *host_blocks_out,
                  int32_t *gpu_blocks_out, int32_t *num_pairs_out);

/* Host pool queries: free blocks, one block's count, the free queue front to back. */
int64_t pa_bm_num_free_host(const pa_block_manager *bm);
int32_t pa_bm_host_refcount(const pa_block_manager *bm, int32_t block);
int64_t pa_bm_host_free_queue(const pa_block_manager *bm, int32_t *out, int64_t cap);
/* 1 if the sequence is swapped out, 0 if on the GPU. */
int pa_bm_sequence_on_host(const pa_block_manager *bm, int64_t seq);

/* Queries: counts, one block's references, one sequence's shape, the queue. */
int64_t pa_bm_num_free(const pa_block_manager *bm);
int64_t pa_bm_num_sequences(const pa_block_manager *bm);
int32_t pa_bm_refcount(const pa_block_manager *bm, int32_t block);
int pa_bm_sequence_info(const pa_block_manager *bm, int64_t seq, int32_t *num_tokens, int32_t *num_blocks);
/* Free queue front to back into out[cap]; returns the queue length (may exceed cap). */
int64_t pa_bm_free_queue(const pa_block_manager *bm, int32_t *out, int64_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
