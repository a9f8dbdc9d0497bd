// Internal declarations shared by the C ABI (pa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

// Largest partition, in blocks, whose table entries one workgroup stages in
// LDS: 2,048 for a grid launch, 512 for a work-list launch (whose persistent
// workgroups pay for every extra register and LDS byte in residency; calls
// with longer partitions take the grid).
constexpr int kMaxPartitionBlocks = 2048;
constexpr int kMaxListPartitionBlocks = 512;
// Query rows (GQA head x token) one prefill workgroup takes: 16 per row group,
// two groups per wave, 8 waves.
constexpr int kPrefillRowGroups = 2;
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRows = 16 * kPrefillRowGroups * kPrefillWaves;

struct PoolDesc {
  char *base;
  int64_t num_blocks;
  int num_kv_heads;
  int block_size;
  int head_dim;
  int dtype;
  int elem_bytes;
  int64_t row_bytes;    // head_dim * elem_bytes: one token of one head, K or V
  int64_t tile_bytes;   // block_size * row_bytes: one (block, head) K or V tile
  int64_t block_bytes;  // 2 * num_kv_heads * tile_bytes: one physical block
};

struct DecodeArgs {
  PoolDesc pool;
  const void *q;
  float *out;
  const int32_t *block_tables;
  int max_blocks_per_seq;
  const int32_t *context_lens;
  int num_seqs;
  int num_q_heads;
  float scale;
  int max_context_len;
  int partition_blocks;  // blocks per split-context partition
  int num_partitions;    // ceil(max_context_len / (partition_blocks * block_size))
  bool stream_loads;     // non-temporal K/V loads (PA_DECODE_STREAM)
  float *ws_o;           // [S][Hq][P][D] unnormalised partial outputs
  float *ws_ml;          // [S][Hq][P][2] running max (log2 units) and sum
  int32_t *items;        // work list (null: one workgroup per (pair, partition))
  int32_t *n_items;      // its length, written by the list's prepass
  int32_t *next_item;    // items taken so far past the first per workgroup (reset by the prepass)
};

struct PrefillArgs {
  PoolDesc pool;
  const void *q;
  float *out;
  const int32_t *query_start_loc;
  const int32_t *context_lens;
  const int32_t *block_tables;
  int max_blocks_per_seq;
  int num_seqs;
  int num_q_heads;
  int total_tokens;
  int max_query_len;
  float scale;
};

// Workspace layout of one decode call; every region 256-byte aligned.
// Partials only when some sequence may span several partitions; the work
// list (int32 per (pair, partition) plus its length) only for list launches.
struct WorkspaceLayout {
  size_t o_off, ml_off, items_off, n_items_off, total;  // n_items_off: item count, then the take counter
};
WorkspaceLayout decode_workspace_layout(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                        int num_partitions, bool work_list);
// Whether a decode call walks a work list: batches of many (sequence, KV
// head) pairs, whose lengths are likely skewed, with sequences that may
// span several partitions (measured: 5-6 % faster on 512 lognormal contexts;
// a batch of 1,024 pairs of at most one partition each is 10 % slower with
// the list's prepass than with the grid).
bool decode_uses_work_list(int num_seqs, int num_kv_heads, int num_partitions, int partition_blocks);

hipError_t launch_slot_mapping(const PoolDesc &pool, const int32_t *tables, int max_blocks_per_seq,
                               int num_seqs, const int32_t *seq_ids, const int32_t *positions,
                               int64_t *slots, int num_tokens, hipStream_t stream);
hipError_t launch_cache_write(const PoolDesc &pool, const void *k_new, const void *v_new,
                              const int64_t *slots, int num_tokens, hipStream_t stream);
hipError_t launch_cache_write_at(const PoolDesc &pool, const void *k_new, const void *v_new,
                                 const int32_t *tables, int max_blocks_per_seq, int num_seqs, const int32_t *seq_ids,
                                 const int32_t *positions, int64_t *slots, int num_tokens, hipStream_t stream);
hipError_t launch_block_copy(const PoolDesc &pool, const int32_t *src, const int32_t *dst, int num_pairs,
                             hipStream_t stream);
// Whole-block copies from one pool to another of the same geometry (bases as
// the device sees them; either may be pinned host memory).
hipError_t launch_swap(const char *src_base, int64_t src_num_blocks, char *dst_base, int64_t dst_num_blocks,
                       int64_t block_bytes, const int32_t *src, const int32_t *dst, int num_pairs,
                       hipStream_t stream);
// Returns hipErrorInvalidValue when no kernel is built for the shape.
hipError_t launch_decode(const DecodeArgs &args, hipStream_t stream);
bool decode_supported(int dtype, int head_dim, int block_size, int group);
// True where decode takes its scores from the matrix cores (bf16, groups of 8,
// blocks of 16 tokens or more); the launch shape and partitioning follow it.
bool decode_matrix_core_scores(int dtype, int group, int block_size);
hipError_t launch_prefill(const PrefillArgs &args, hipStream_t stream);
bool prefill_supported(int dtype, int head_dim, int block_size, int group);

}  // namespace pa
