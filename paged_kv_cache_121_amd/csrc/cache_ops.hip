// Slot mapping, cache write and block copy kernels for gfx950.
// Citation keys ([HRL], [VIBE], [TSS], ...) name the source pages listed with
// their titles at the top of include/pa.h.
//
// All three are pure data movement.  The cache write and the block copy move
// 16-byte words per lane so that a wavefront touches whole, contiguous
// 1 KiB spans; every index is checked against the pool before it is used.

#include "pa_internal.h"

namespace pa {
namespace {

// slot = table[seq][pos / B] * B + pos % B  ([TSS] "Finding a token"); any
// id or position outside its buffer yields -1.
__device__ __forceinline__ int64_t token_slot(const int32_t *__restrict__ tables, int max_blocks_per_seq,
                                              int num_seqs, int seq, int pos, int block_size, int64_t num_blocks) {
  if (seq < 0 || seq >= num_seqs || pos < 0) return -1;
  const int logical = pos / block_size;
  if (logical >= max_blocks_per_seq) return -1;
  const int64_t block = tables[(int64_t)seq * max_blocks_per_seq + logical];
  if (block < 0 || block >= num_blocks) return -1;
  return block * block_size + (pos - logical * block_size);
}

// One lane per token.
__global__ void __launch_bounds__(256)
slot_mapping_kernel(const int32_t *__restrict__ tables, int max_blocks_per_seq, int num_seqs,
                    const int32_t *__restrict__ seq_ids, const int32_t *__restrict__ positions,
                    int64_t *__restrict__ slots, int num_tokens, int block_size, int64_t num_blocks) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_tokens) return;
  slots[i] = token_slot(tables, max_blocks_per_seq, num_seqs, seq_ids[i], positions[i], block_size, num_blocks);
}

// The workgroup's token's 2 * Hkv rows (K then V, one per KV head) are split
// into 16-byte words; word w of row r goes to
// pool[slot / B][r / Hkv][r % Hkv][slot % B][w * 16 bytes ...].
__device__ __forceinline__ void write_token_rows(char *__restrict__ pool, int num_kv_heads, int block_size,
                                                 int64_t row_bytes, int64_t tile_bytes, int64_t block_bytes,
                                                 const char *__restrict__ k_new, const char *__restrict__ v_new,
                                                 int token, int64_t slot) {
  const int64_t block = slot / block_size;
  const int64_t offset = slot - block * block_size;
  const int words_per_row = (int)(row_bytes / 16);
  const int total_words = 2 * num_kv_heads * words_per_row;
  for (int w = threadIdx.x; w < total_words; w += blockDim.x) {
    const int row = w / words_per_row;  // 0..2*Hkv-1: K rows first, then V rows
    const int word = w - row * words_per_row;
    const int kv = row / num_kv_heads;
    const int head = row - kv * num_kv_heads;
    const char *src = (kv ? v_new : k_new) + ((int64_t)token * num_kv_heads + head) * row_bytes + word * 16;
    char *dst = pool + block * block_bytes + (int64_t)(kv * num_kv_heads + head) * tile_bytes +
                offset * row_bytes + word * 16;
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
  }
}

// One workgroup per written token, slot given.
__global__ void __launch_bounds__(256)
cache_write_kernel(char *__restrict__ pool, int64_t num_slots, int num_kv_heads, int block_size,
                   int64_t row_bytes, int64_t tile_bytes, int64_t block_bytes,
                   const char *__restrict__ k_new, const char *__restrict__ v_new,
                   const int64_t *__restrict__ slots) {
  const int token = blockIdx.x;
  const int64_t slot = slots[token];
  if (slot < 0 || slot >= num_slots) return;
  write_token_rows(pool, num_kv_heads, block_size, row_bytes, tile_bytes, block_bytes, k_new, v_new, token, slot);
}

// One workgroup per written token, slot computed from (sequence, position)
// through the table (the slot mapping and the write in one launch); the slot
// is also stored when `slots` is not null.
__global__ void __launch_bounds__(256)
cache_write_at_kernel(char *__restrict__ pool, int num_kv_heads, int block_size, int64_t row_bytes,
                      int64_t tile_bytes, int64_t block_bytes, const char *__restrict__ k_new,
                      const char *__restrict__ v_new, const int32_t *__restrict__ tables, int max_blocks_per_seq,
                      int num_seqs, const int32_t *__restrict__ seq_ids, const int32_t *__restrict__ positions,
                      int64_t *__restrict__ slots, int64_t num_blocks) {
  const int token = blockIdx.x;
  const int64_t slot =
      token_slot(tables, max_blocks_per_seq, num_seqs, seq_ids[token], positions[token], block_size, num_blocks);
  if (slots != nullptr && threadIdx.x == 0) slots[token] = slot;
  if (slot < 0) return;  // a valid slot lies below num_blocks * block_size
  write_token_rows(pool, num_kv_heads, block_size, row_bytes, tile_bytes, block_bytes, k_new, v_new, token, slot);
}

// Grid (pairs, slices): each workgroup copies one 16 KiB slice of one block,
// four 16-byte words per lane with all loads issued before the stores.  The
// source and destination pools may differ (a swap between device memory and
// pinned host memory reads or writes the host side over the host link; one
// launch keeps every pair's transfer in flight together).
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopySlice = (int64_t)kCopyThreads * kCopyUnroll * 16;

__global__ void __launch_bounds__(kCopyThreads)
block_copy_kernel(const char *__restrict__ src_pool, int64_t src_num_blocks, char *__restrict__ dst_pool,
                  int64_t dst_num_blocks, int64_t block_bytes, const int32_t *__restrict__ src_blocks,
                  const int32_t *__restrict__ dst_blocks) {
  const int pair = blockIdx.x;
  const int64_t src = src_blocks[pair];
  const int64_t dst = dst_blocks[pair];
  if (src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks) return;
  const int64_t base = (int64_t)blockIdx.y * kCopySlice;
  const uint4 *s = reinterpret_cast<const uint4 *>(src_pool + src * block_bytes + base);
  uint4 *d = reinterpret_cast<uint4 *>(dst_pool + dst * block_bytes + base);
  const int64_t words = (block_bytes - base) / 16 < kCopySlice / 16 ? (block_bytes - base) / 16 : kCopySlice / 16;
  uint4 buf[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t w = threadIdx.x + (int64_t)u * kCopyThreads;
    if (w < words) buf[u] = s[w];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t w = threadIdx.x + (int64_t)u * kCopyThreads;
    if (w < words) d[w] = buf[u];
  }
}

}  // namespace

hipError_t launch_slot_mapping(const PoolDesc &pool, const int32_t *tables, int max_blocks_per_seq,
                               int num_seqs, const int32_t *seq_ids, const int32_t *positions,
                               int64_t *slots, int num_tokens, hipStream_t stream) {
  const int threads = 256;
  const int grid = (num_tokens + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(threads), 0, stream, tables, max_blocks_per_seq,
                     num_seqs, seq_ids, positions, slots, num_tokens, pool.block_size, pool.num_blocks);
  return hipGetLastError();
}

hipError_t launch_cache_write(const PoolDesc &pool, const void *k_new, const void *v_new,
                              const int64_t *slots, int num_tokens, hipStream_t stream) {
  const int words = (int)(2 * pool.num_kv_heads * pool.row_bytes / 16);
  const int threads = words >= 256 ? 256 : ((words + 63) / 64) * 64;
  hipLaunchKernelGGL(cache_write_kernel, dim3(num_tokens), dim3(threads), 0, stream, pool.base,
                     pool.num_blocks * pool.block_size, pool.num_kv_heads, pool.block_size, pool.row_bytes,
                     pool.tile_bytes, pool.block_bytes, static_cast<const char *>(k_new),
                     static_cast<const char *>(v_new), slots);
  return hipGetLastError();
}

hipError_t launch_cache_write_at(const PoolDesc &pool, const void *k_new, const void *v_new,
                                 const int32_t *tables, int max_blocks_per_seq, int num_seqs, const int32_t *seq_ids,
                                 const int32_t *positions, int64_t *slots, int num_tokens, hipStream_t stream) {
  const int words = (int)(2 * pool.num_kv_heads * pool.row_bytes / 16);
  const int threads = words >= 256 ? 256 : ((words + 63) / 64) * 64;
  hipLaunchKernelGGL(cache_write_at_kernel, dim3(num_tokens), dim3(threads), 0, stream, pool.base,
                     pool.num_kv_heads, pool.block_size, pool.row_bytes, pool.tile_bytes, pool.block_bytes,
                     static_cast<const char *>(k_new), static_cast<const char *>(v_new), tables,
                     max_blocks_per_seq, num_seqs, seq_ids, positions, slots, pool.num_blocks);
  return hipGetLastError();
}

hipError_t launch_block_copy(const PoolDesc &pool, const int32_t *src, const int32_t *dst, int num_pairs,
                             hipStream_t stream) {
  return launch_swap(pool.base, pool.num_blocks, pool.base, pool.num_blocks, pool.block_bytes, src, dst, num_pairs,
                     stream);
}

hipError_t launch_swap(const char *src_base, int64_t src_num_blocks, char *dst_base, int64_t dst_num_blocks,
                       int64_t block_bytes, const int32_t *src, const int32_t *dst, int num_pairs,
                       hipStream_t stream) {
  const int slices = (int)((block_bytes + kCopySlice - 1) / kCopySlice);
  hipLaunchKernelGGL(block_copy_kernel, dim3(num_pairs, slices), dim3(kCopyThreads), 0, stream, src_base,
                     src_num_blocks, dst_base, dst_num_blocks, block_bytes, src, dst);
  return hipGetLastError();
}

}  // namespace pa
