// C ABI of the paged KV-cache decode path: argument checks, workspace sizing,
// partition choice and kernel launches.  No allocation, no synchronisation.

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_set>
#include <vector>

#include "pa_blocks.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr size_t kAlign = 256;
// Automatic partitioning.  A call wants at least kMinWorkgroups workgroups
// (two per compute unit) so every CU streams; few (sequence, KV head) pairs
// are therefore split into equal partitions.  The matrix-core decode kernel
// (groups of 8) wants one workgroup per CU instead: measured on 8 x 32,768
// tokens of a 64-head / 8-KV-head layer, 8,192-token partitions (256
// workgroups) took 161 us against 171 us at 4,096 and 177 us at 2,048.  Batches with many pairs are
// likely to mix short and long contexts, so their partitions are capped at
// kSkewedPartitionTokens to keep one long sequence from becoming the tail.
constexpr int64_t kMinWorkgroups = 512;
constexpr int64_t kMinWorkgroupsMatrixCore = 256;
constexpr int64_t kManyPairs = 1024;
constexpr int kSkewedPartitionTokens = 2048;
constexpr int kMinAutoPartitionTokens = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_pool(const pa_pool *p, PoolDesc *d) {
  if (p == nullptr || p->base == nullptr) return PA_ERR_INVALID_ARG;
  if (p->num_blocks <= 0 || p->num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  // any power of two up to 256 for the data-movement kernels; attention
  // kernels check their own block sizes
  if (p->block_size <= 0 || p->block_size > 256 || (p->block_size & (p->block_size - 1)) != 0)
    return PA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (p->dtype != PA_F32 && p->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (p->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  d->base = static_cast<char *>(p->base);
  d->num_blocks = p->num_blocks;
  d->num_kv_heads = p->num_kv_heads;
  d->block_size = p->block_size;
  d->head_dim = p->head_dim;
  d->dtype = p->dtype;
  d->elem_bytes = p->dtype == PA_BF16 ? 2 : 4;
  d->row_bytes = (int64_t)p->head_dim * d->elem_bytes;
  d->tile_bytes = d->row_bytes * p->block_size;
  d->block_bytes = 2 * d->tile_bytes * p->num_kv_heads;
  // slot ids are int64 and block ids int32 in the tables
  if (p->num_blocks > INT32_MAX) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// The address a kernel uses for a pool base: device memory as is, pinned host
// memory (hipHostMalloc) only where the device address equals the host one.
// Anything else -- pageable host memory, an unknown pointer -- is refused, so
// no kernel is launched on memory the device cannot reach.
int device_view(char *p, char **out) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_INVALID_ARG;
  }
  if (a.type == hipMemoryTypeDevice) {
    *out = p;
    return PA_OK;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer == p) {
    *out = p;
    return PA_OK;
  }
  return PA_ERR_INVALID_ARG;
}

int partition_unit(int block_size) { return block_size < 16 ? 16 : block_size; }

int auto_partition_tokens(int block_size, int num_seqs, int num_kv_heads, int max_context_len, int64_t min_wg) {
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  const int64_t want_parts = pairs >= min_wg ? 1 : (min_wg + pairs - 1) / pairs;
  int64_t part = (max_context_len + want_parts - 1) / want_parts;
  if (pairs >= kManyPairs && part > kSkewedPartitionTokens) part = kSkewedPartitionTokens;
  if (part < kMinAutoPartitionTokens) part = kMinAutoPartitionTokens;
  // partitions hold whole decode units (one block, or 16 tokens of small blocks)
  const int unit = partition_unit(block_size);
  part = (part + unit - 1) / unit * unit;
  const int64_t cap = (int64_t)kMaxPartitionBlocks * block_size / unit * unit;
  if (part > cap) {
    // as few partitions as the cap allows, of equal length (no near-empty last one)
    const int64_t nparts = (max_context_len + cap - 1) / cap;
    part = ((max_context_len + nparts - 1) / nparts + unit - 1) / unit * unit;
  }
  return (int)part;
}

// Resolves the partition size in tokens, or returns a negative status.
int resolve_partition(const PoolDesc &pool, int num_seqs, int num_q_heads, int max_context_len,
                      int partition_size) {
  if (partition_size == 0) {
    const int group = num_q_heads / pool.num_kv_heads;
    const int64_t min_wg = decode_matrix_core_scores(pool.dtype, group, pool.block_size) ? kMinWorkgroupsMatrixCore
                                                                                         : kMinWorkgroups;
    return auto_partition_tokens(pool.block_size, num_seqs, pool.num_kv_heads, max_context_len, min_wg);
  }
  if (partition_size < 0 || partition_size % partition_unit(pool.block_size) != 0) return PA_ERR_INVALID_ARG;
  if (partition_size / pool.block_size > kMaxPartitionBlocks) return PA_ERR_UNSUPPORTED;
  return partition_size;
}

// ---- checked mode.  With PA_CHECK=1 in the environment (read at every
// call), each entry point copies the index arrays it is given to the host,
// waits for them, and refuses (PA_ERR_INVALID_ARG, nothing launched) the
// device contents the kernels would otherwise only skip or turn into NaN.  It
// synchronises the stream and allocates host memory, so it cannot run under
// graph capture (PA_ERR_UNSUPPORTED there).
bool checked_mode() {
  const char *e = std::getenv("PA_CHECK");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

// Copies n elements of a device array to `dst` on `stream` and waits.
template <typename T>
int fetch_host(std::vector<T> &dst, const T *src, size_t n, hipStream_t stream) {
  dst.resize(n);
  if (n == 0) return PA_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (cs != hipStreamCaptureStatusNone) return PA_ERR_UNSUPPORTED;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  return PA_OK;
}

// Slots of one write ([TSS] "Finding a token": one slot per written token):
// non-negative slots must lie inside the pool and be pairwise distinct;
// negative ones are skipped by the write and pass.
int check_slots(const PoolDesc &d, const std::vector<int64_t> &slots) {
  const int64_t num_slots = d.num_blocks * d.block_size;
  std::unordered_set<int64_t> seen;
  seen.reserve(slots.size() * 2);
  for (const int64_t s : slots) {
    if (s < 0) continue;
    if (s >= num_slots || !seen.insert(s).second) return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

// Slots of (sequence, position) tokens through the tables, as the slot
// mapping computes them; a token that would get -1 other than by a negative
// position (padding) is refused.
int checked_token_slots(const PoolDesc &d, const int32_t *tables, int max_blocks_per_seq, int num_seqs,
                        const int32_t *seq_ids, const int32_t *positions, int num_tokens, hipStream_t stream,
                        std::vector<int64_t> &slots) {
  std::vector<int32_t> tb, sq, ps;
  int st = fetch_host(tb, tables, (size_t)num_seqs * max_blocks_per_seq, stream);
  if (st == PA_OK) st = fetch_host(sq, seq_ids, (size_t)num_tokens, stream);
  if (st == PA_OK) st = fetch_host(ps, positions, (size_t)num_tokens, stream);
  if (st != PA_OK) return st;
  slots.assign(num_tokens, -1);
  for (int i = 0; i < num_tokens; ++i) {
    const int seq = sq[i], pos = ps[i];
    if (pos < 0) continue;
    if (seq < 0 || seq >= num_seqs || pos / d.block_size >= max_blocks_per_seq) return PA_ERR_INVALID_ARG;
    const int64_t b = tb[(size_t)seq * max_blocks_per_seq + pos / d.block_size];
    if (b < 0 || b >= d.num_blocks) return PA_ERR_INVALID_ARG;
    slots[i] = b * d.block_size + pos % d.block_size;
  }
  return PA_OK;
}

// Copy pairs ([AINEW] copy-on-write passage: the shared source is never
// written): ids inside their pools, destinations distinct and, inside one
// pool, disjoint from the sources.
int check_pairs(int64_t src_blocks, int64_t dst_blocks, bool same_pool, const int32_t *src, const int32_t *dst,
                int num_pairs, hipStream_t stream) {
  std::vector<int32_t> s, t;
  int st = fetch_host(s, src, (size_t)num_pairs, stream);
  if (st == PA_OK) st = fetch_host(t, dst, (size_t)num_pairs, stream);
  if (st != PA_OK) return st;
  std::unordered_set<int32_t> dsts;
  dsts.reserve((size_t)num_pairs * 2);
  for (int j = 0; j < num_pairs; ++j) {
    if (s[j] < 0 || s[j] >= src_blocks || t[j] < 0 || t[j] >= dst_blocks) return PA_ERR_INVALID_ARG;
    if (!dsts.insert(t[j]).second) return PA_ERR_INVALID_ARG;
  }
  if (same_pool)
    for (int j = 0; j < num_pairs; ++j)
      if (dsts.count(s[j])) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// The table entries attention reads: the first ceil(len / B) of each row,
// every one inside the pool.
int check_table_prefixes(const PoolDesc &d, const std::vector<int32_t> &tb, int max_blocks_per_seq,
                         const std::vector<int32_t> &lens) {
  for (size_t s = 0; s < lens.size(); ++s) {
    const int64_t nb = ((int64_t)lens[s] + d.block_size - 1) / d.block_size;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = tb[s * max_blocks_per_seq + j];
      if (b < 0 || b >= d.num_blocks) return PA_ERR_INVALID_ARG;
    }
  }
  return PA_OK;
}

int check_decode_inputs(const PoolDesc &d, const int32_t *tables, int max_blocks_per_seq, const int32_t *lens_dev,
                        int num_seqs, int max_context_len, hipStream_t stream) {
  std::vector<int32_t> tb, lens;
  int st = fetch_host(lens, lens_dev, (size_t)num_seqs, stream);
  if (st == PA_OK) st = fetch_host(tb, tables, (size_t)num_seqs * max_blocks_per_seq, stream);
  if (st != PA_OK) return st;
  for (const int32_t L : lens)
    if (L < 0 || L > max_context_len || (int64_t)L > (int64_t)max_blocks_per_seq * d.block_size)
      return PA_ERR_INVALID_ARG;
  return check_table_prefixes(d, tb, max_blocks_per_seq, lens);
}

int check_prefill_inputs(const PoolDesc &d, const int32_t *qsl_dev, const int32_t *lens_dev, const int32_t *tables,
                         int max_blocks_per_seq, int num_seqs, int total_tokens, int max_query_len,
                         hipStream_t stream) {
  std::vector<int32_t> qsl, lens, tb;
  int st = fetch_host(qsl, qsl_dev, (size_t)num_seqs + 1, stream);
  if (st == PA_OK) st = fetch_host(lens, lens_dev, (size_t)num_seqs, stream);
  if (st == PA_OK) st = fetch_host(tb, tables, (size_t)num_seqs * max_blocks_per_seq, stream);
  if (st != PA_OK) return st;
  if (qsl[0] < 0 || qsl[num_seqs] > total_tokens) return PA_ERR_INVALID_ARG;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t n = (int64_t)qsl[s + 1] - qsl[s];
    if (n < 0 || n > lens[s] || n > max_query_len) return PA_ERR_INVALID_ARG;
    if (lens[s] < 0 || (int64_t)lens[s] > (int64_t)max_blocks_per_seq * d.block_size) return PA_ERR_INVALID_ARG;
  }
  return check_table_prefixes(d, tb, max_blocks_per_seq, lens);
}

// Validates pa_decode's scalar arguments and fills `a` (workspace left
// unbound); *ws_need receives the workspace bytes the call needs (0 when
// every sequence fits one partition).  Returns PA_OK with nothing to do when
// num_seqs is 0.
int prepare_decode(const pa_pool *pool, const void *q, float *out, const int32_t *block_tables,
                   int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                   float scale, int32_t max_context_len, int32_t partition_size, int32_t flags, DecodeArgs *a,
                   size_t *ws_need) {
  PoolDesc d;
  *ws_need = 0;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % d.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (flags & ~PA_DECODE_KEEP_CACHED) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * d.block_size > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (!decode_supported(d.dtype, d.head_dim, d.block_size, num_q_heads / d.num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (q == nullptr || out == nullptr || block_tables == nullptr || context_lens == nullptr)
    return PA_ERR_INVALID_ARG;
  const int part = resolve_partition(d, num_seqs, num_q_heads, max_context_len, partition_size);
  if (part < 0) return part;
  const int parts = max_context_len == 0 ? 1 : (max_context_len + part - 1) / part;
  // one workgroup per (pair, partition), pairs rounded up to a multiple of 8
  if (((int64_t)num_seqs * d.num_kv_heads + 8) * parts > INT32_MAX) return PA_ERR_UNSUPPORTED;
  a->pool = d;
  a->q = q;
  a->out = out;
  a->block_tables = block_tables;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->context_lens = context_lens;
  a->num_seqs = num_seqs;
  a->num_q_heads = num_q_heads;
  a->scale = scale;
  a->max_context_len = max_context_len;
  a->partition_blocks = part / d.block_size;
  a->num_partitions = parts;
  a->stream_loads = (flags & PA_DECODE_KEEP_CACHED) == 0;
  *ws_need = decode_workspace_layout(num_seqs, num_q_heads, d.num_kv_heads, d.head_dim, parts,
                                     decode_uses_work_list(num_seqs, d.num_kv_heads, parts, a->partition_blocks))
                  .total;
  return PA_OK;
}

// Points the split-context partials and the work list of `a` into a
// workspace of the size prepare_decode asked for (256-byte aligned).
void bind_workspace(DecodeArgs *a, char *base) {
  const bool list =
      decode_uses_work_list(a->num_seqs, a->pool.num_kv_heads, a->num_partitions, a->partition_blocks);
  const WorkspaceLayout w = decode_workspace_layout(a->num_seqs, a->num_q_heads, a->pool.num_kv_heads,
                                                    a->pool.head_dim, a->num_partitions, list);
  if (a->num_partitions > 1) {
    a->ws_o = reinterpret_cast<float *>(base + w.o_off);
    a->ws_ml = reinterpret_cast<float *>(base + w.ml_off);
  }
  if (list) {
    a->items = reinterpret_cast<int32_t *>(base + w.items_off);
    a->n_items = reinterpret_cast<int32_t *>(base + w.n_items_off);
    a->next_item = a->n_items + 1;
  }
}

// ---- decode without allocation (pa_decode_noalloc): the split-context
// partials go to this file-scope device array instead of a caller's
// workspace.  Every device the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address is taken once
// per device with hipGetSymbolAddress and only that address is used.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
char *g_scratch_address[kMaxScratchDevices];  // per device; null until first taken

// Device address of `scratch` on the current device, which must be the
// stream's device.
int scratch_address(hipStream_t stream, char **out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (stream != nullptr) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) {
      (void)hipGetLastError();
      return PA_ERR_INVALID_ARG;
    }
    if (sd != cur) return PA_ERR_INVALID_ARG;
  }
  if (cur < 0 || cur >= kMaxScratchDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_address[cur] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch_address[cur] = static_cast<char *>(p);
  }
  *out = g_scratch_address[cur];
  return PA_OK;
}

}  // namespace

WorkspaceLayout decode_workspace_layout(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                        int num_partitions, bool work_list) {
  WorkspaceLayout w{};
  size_t off = 0;
  if (num_partitions > 1) {
    const size_t rows = (size_t)num_seqs * num_q_heads * num_partitions;
    w.o_off = off;
    off += align_up(rows * head_dim * sizeof(float));
    w.ml_off = off;
    off += align_up(rows * 2 * sizeof(float));
  }
  if (work_list) {
    w.items_off = off;
    off += align_up((size_t)num_seqs * num_kv_heads * num_partitions * sizeof(int32_t));
    w.n_items_off = off;
    off += align_up(2 * sizeof(int32_t));
  }
  w.total = off;
  return w;
}

bool decode_uses_work_list(int num_seqs, int num_kv_heads, int num_partitions, int partition_blocks) {
  return num_partitions > 1 && (int64_t)num_seqs * num_kv_heads >= kManyPairs &&
         partition_blocks <= kMaxListPartitionBlocks;
}

}  // namespace pa

using namespace pa;

extern "C" {

const char *pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failure";
    case PA_ERR_OUT_OF_BLOCKS: return "out of free blocks";
    case PA_ERR_NO_SEQUENCE: return "unknown sequence id";
    case PA_ERR_SWAPPED: return "sequence is swapped out";
    default: return "unknown status";
  }
}

int pa_slot_mapping(const pa_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                    int32_t num_seqs, const int32_t *seq_ids, const int32_t *positions,
                    int64_t *slot_mapping, int32_t num_tokens, hipStream_t stream) {
  PoolDesc d;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (seq_ids == nullptr || positions == nullptr || slot_mapping == nullptr) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && max_blocks_per_seq > 0 && block_tables == nullptr) return PA_ERR_INVALID_ARG;
  if (checked_mode()) {
    std::vector<int64_t> slots;
    const int c = checked_token_slots(d, block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions, num_tokens,
                                      stream, slots);
    if (c != PA_OK) return c;
  }
  return status_of(launch_slot_mapping(d, block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions,
                                       slot_mapping, num_tokens, stream));
}

int pa_cache_write(const pa_pool *pool, const void *k_new, const void *v_new, const int64_t *slot_mapping,
                   int32_t num_tokens, hipStream_t stream) {
  PoolDesc d;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr) return PA_ERR_INVALID_ARG;
  if (checked_mode()) {
    std::vector<int64_t> slots;
    int c = fetch_host(slots, slot_mapping, (size_t)num_tokens, stream);
    if (c == PA_OK) c = check_slots(d, slots);
    if (c != PA_OK) return c;
  }
  return status_of(launch_cache_write(d, k_new, v_new, slot_mapping, num_tokens, stream));
}

int pa_cache_write_at(const pa_pool *pool, const void *k_new, const void *v_new, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, int32_t num_seqs, const int32_t *seq_ids, const int32_t *positions,
                      int64_t *slot_mapping, int32_t num_tokens, hipStream_t stream) {
  PoolDesc d;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr || seq_ids == nullptr || positions == nullptr) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && max_blocks_per_seq > 0 && block_tables == nullptr) return PA_ERR_INVALID_ARG;
  if (checked_mode()) {
    std::vector<int64_t> slots;
    int c = checked_token_slots(d, block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions, num_tokens, stream,
                                slots);
    if (c == PA_OK) c = check_slots(d, slots);
    if (c != PA_OK) return c;
  }
  return status_of(launch_cache_write_at(d, k_new, v_new, block_tables, max_blocks_per_seq, num_seqs, seq_ids,
                                         positions, slot_mapping, num_tokens, stream));
}

int pa_block_copy(const pa_pool *pool, const int32_t *src_blocks, const int32_t *dst_blocks, int32_t num_pairs,
                  hipStream_t stream) {
  PoolDesc d;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (src_blocks == nullptr || dst_blocks == nullptr) return PA_ERR_INVALID_ARG;
  if (checked_mode()) {
    const int c = check_pairs(d.num_blocks, d.num_blocks, true, src_blocks, dst_blocks, num_pairs, stream);
    if (c != PA_OK) return c;
  }
  return status_of(launch_block_copy(d, src_blocks, dst_blocks, num_pairs, stream));
}

int pa_swap_blocks(const pa_pool *src, const pa_pool *dst, const int32_t *src_blocks, const int32_t *dst_blocks,
                   int32_t num_pairs, hipStream_t stream) {
  PoolDesc s, d;
  int st = check_pool(src, &s);
  if (st != PA_OK) return st;
  st = check_pool(dst, &d);
  if (st != PA_OK) return st;
  if (s.num_kv_heads != d.num_kv_heads || s.block_size != d.block_size || s.head_dim != d.head_dim ||
      s.dtype != d.dtype)
    return PA_ERR_INVALID_ARG;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (src_blocks == nullptr || dst_blocks == nullptr) return PA_ERR_INVALID_ARG;
  char *sv = nullptr, *dv = nullptr;
  if (device_view(s.base, &sv) != PA_OK || device_view(d.base, &dv) != PA_OK) return PA_ERR_INVALID_ARG;
  if (checked_mode()) {
    const int c = check_pairs(s.num_blocks, d.num_blocks, sv == dv, src_blocks, dst_blocks, num_pairs, stream);
    if (c != PA_OK) return c;
  }
  return status_of(launch_swap(sv, s.num_blocks, dv, d.num_blocks, s.block_bytes, src_blocks, dst_blocks, num_pairs,
                               stream));
}

int32_t pa_decode_partition_size(const pa_pool *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len) {
  PoolDesc d;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  return resolve_partition(d, num_seqs, num_q_heads, max_context_len, 0);
}

int64_t pa_decode_workspace_size(const pa_pool *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t partition_size) {
  PoolDesc d;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if (num_q_heads % d.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  const int part = resolve_partition(d, num_seqs, num_q_heads, max_context_len, partition_size);
  if (part < 0) return part;
  if (num_seqs == 0) return 0;
  const int parts = max_context_len == 0 ? 1 : (max_context_len + part - 1) / part;  // as pa_decode
  return (int64_t)decode_workspace_layout(num_seqs, num_q_heads, d.num_kv_heads, d.head_dim, parts,
                                          decode_uses_work_list(num_seqs, d.num_kv_heads, parts, part / d.block_size))
      .total;
}

int pa_decode(const pa_pool *pool, const void *q, float *out, const int32_t *block_tables,
              int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
              float scale, int32_t max_context_len, int32_t partition_size, int32_t flags, void *workspace,
              size_t workspace_bytes, hipStream_t stream) {
  DecodeArgs a{};
  size_t need = 0;
  const int st = prepare_decode(pool, q, out, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                scale, max_context_len, partition_size, flags, &a, &need);
  if (st != PA_OK || num_seqs == 0) return st;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return PA_ERR_WORKSPACE;
    bind_workspace(&a, static_cast<char *>(workspace));
  }
  if (checked_mode()) {
    const int c = check_decode_inputs(a.pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                      max_context_len, stream);
    if (c != PA_OK) return c;
  }
  return status_of(launch_decode(a, stream));
}

int pa_decode_noalloc(const pa_pool *pool, const void *q, float *out, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                      int32_t num_q_heads, float scale, int32_t max_context_len, int32_t partition_size,
                      int32_t flags, hipStream_t stream) {
  DecodeArgs a{};
  size_t need = 0;
  const int st = prepare_decode(pool, q, out, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                scale, max_context_len, partition_size, flags, &a, &need);
  if (st != PA_OK || num_seqs == 0) return st;
  if (need > kScratchBytes) return PA_ERR_WORKSPACE;
  if (need > 0) {
    char *ws = nullptr;
    const int s2 = scratch_address(stream, &ws);
    if (s2 != PA_OK) return s2;
    bind_workspace(&a, ws);
  }
  return status_of(launch_decode(a, stream));
}

int pa_prefill(const pa_pool *pool, const void *q, float *out, const int32_t *query_start_loc,
               const int32_t *context_lens, const int32_t *block_tables, int32_t max_blocks_per_seq,
               int32_t num_seqs, int32_t num_q_heads, int32_t total_tokens, int32_t max_query_len, float scale,
               hipStream_t stream) {
  PoolDesc d;
  const int st = check_pool(pool, &d);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || total_tokens < 0 || max_query_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % d.num_kv_heads != 0 || !std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * d.block_size > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (!prefill_supported(d.dtype, d.head_dim, d.block_size, num_q_heads / d.num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_query_len == 0 || total_tokens == 0) return PA_OK;
  {  // one workgroup per (row tile, KV head, sequence), in a one-dimensional grid
    const int64_t tokens_per_tile = kPrefillRows / (num_q_heads / d.num_kv_heads);
    const int64_t tiles = ((int64_t)max_query_len + tokens_per_tile - 1) / tokens_per_tile;
    if (tiles * d.num_kv_heads * num_seqs > INT32_MAX - 64) return PA_ERR_UNSUPPORTED;
  }
  if (q == nullptr || out == nullptr || query_start_loc == nullptr || context_lens == nullptr ||
      block_tables == nullptr)
    return PA_ERR_INVALID_ARG;
  if (checked_mode()) {
    const int c = check_prefill_inputs(d, query_start_loc, context_lens, block_tables, max_blocks_per_seq, num_seqs,
                                       total_tokens, max_query_len, stream);
    if (c != PA_OK) return c;
  }
  PrefillArgs a{};
  a.pool = d;
  a.q = q;
  a.out = out;
  a.query_start_loc = query_start_loc;
  a.context_lens = context_lens;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.total_tokens = total_tokens;
  a.max_query_len = max_query_len;
  a.scale = scale;
  return status_of(launch_prefill(a, stream));
}

}  // extern "C"
