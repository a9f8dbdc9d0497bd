// Host-side block manager of the paged KV cache (see include/pa_blocks.h).
//
// The free queue is a doubly linked list threaded through per-block arrays,
// so taking the front, returning a block to either end and unlinking a
// block from the middle are all O(1).  Every mutating call first checks
// that it can complete (enough free blocks, valid ids) and only then
// changes state, so a failed call leaves the manager untouched.

#include "pa_blocks.h"

#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"

namespace {

struct Sequence {
  int32_t num_tokens = 0;
  std::vector<int32_t> table;  // logical block -> physical block
};

}  // namespace

struct pa_block_manager {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> refcount;
  // free queue: links by block id; kNone ends the list
  static constexpr int32_t kNone = -1;
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> queued;
  int32_t head = kNone, tail = kNone;
  int64_t queue_len = 0;
  std::unordered_map<int64_t, Sequence> seqs;
  int64_t next_seq = 0;

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = kNone;
    if (tail != kNone) next[tail] = b; else head = b;
    tail = b;
    queued[b] = 1;
    ++queue_len;
  }
  void push_front(int32_t b) {
    next[b] = head;
    prev[b] = kNone;
    if (head != kNone) prev[head] = b; else tail = b;
    head = b;
    queued[b] = 1;
    ++queue_len;
  }
  void unlink(int32_t b) {
    if (prev[b] != kNone) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] != kNone) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = kNone;
    queued[b] = 0;
    --queue_len;
  }
  // Callers check queue_len first.
  int32_t allocate() {
    const int32_t b = head;
    unlink(b);
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b, bool reusable) {
    if (--refcount[b] == 0) {
      if (reusable) push_back(b); else push_front(b);
    }
  }
  Sequence *find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Sequence *find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  // Blocks a write at `position` needs: growth blocks, plus one copy when
  // the (existing) target block is shared.
  int64_t blocks_for_write(const Sequence &s, int32_t position) const {
    const int64_t logical = position / block_size;
    if (logical >= (int64_t)s.table.size()) return logical + 1 - (int64_t)s.table.size();
    return refcount[s.table[logical]] > 1 ? 1 : 0;
  }
  // Grow + copy-on-write + slot; the caller has checked the free blocks.
  void do_write(Sequence &s, int32_t position, int64_t *slot, int32_t *cow_src, int32_t *cow_dst) {
    const int32_t logical = position / block_size;
    while ((int32_t)s.table.size() <= logical) s.table.push_back(allocate());
    int32_t b = s.table[logical];
    *cow_src = *cow_dst = -1;
    if (refcount[b] > 1) {
      const int32_t fresh = allocate();
      release(b, false);  // still referenced by the other holders
      s.table[logical] = fresh;
      *cow_src = b;
      *cow_dst = fresh;
      b = fresh;
    }
    s.num_tokens = std::max(s.num_tokens, position + 1);
    *slot = (int64_t)b * block_size + (position - logical * block_size);
  }
};

extern "C" {

int pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t reserve_null_block, const int32_t *free_order,
                 int64_t free_order_len, pa_block_manager **out) {
  if (out == nullptr || num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) return PA_ERR_INVALID_ARG;
  if (free_order == nullptr && free_order_len != 0) return PA_ERR_INVALID_ARG;
  std::vector<uint8_t> seen(num_blocks, 0);
  for (int64_t i = 0; i < free_order_len; ++i) {
    const int32_t b = free_order[i];
    if (b < 0 || b >= num_blocks || seen[b]) return PA_ERR_INVALID_ARG;
    seen[b] = 1;
  }
  pa_block_manager *bm = new (std::nothrow) pa_block_manager();
  if (bm == nullptr) return PA_ERR_INVALID_ARG;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  bm->prev.assign(num_blocks, pa_block_manager::kNone);
  bm->next.assign(num_blocks, pa_block_manager::kNone);
  bm->queued.assign(num_blocks, 0);
  const bool null0 = reserve_null_block != 0;
  if (free_order == nullptr) {
    for (int64_t b = null0 ? 1 : 0; b < num_blocks; ++b) bm->push_back((int32_t)b);
  } else {
    for (int64_t i = 0; i < free_order_len; ++i)
      if (!(null0 && free_order[i] == 0)) bm->push_back(free_order[i]);
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

int pa_bm_add_sequence(pa_block_manager *bm, int64_t *seq_out) {
  if (bm == nullptr || seq_out == nullptr) return PA_ERR_INVALID_ARG;
  const int64_t id = bm->next_seq++;
  bm->seqs.emplace(id, Sequence{});
  *seq_out = id;
  return PA_OK;
}

int pa_bm_fork(pa_block_manager *bm, int64_t parent, int32_t num_shared_blocks, int64_t *child_out) {
  if (bm == nullptr || child_out == nullptr) return PA_ERR_INVALID_ARG;
  const Sequence *p = bm->find(parent);
  if (p == nullptr) return PA_ERR_NO_SEQUENCE;
  const int32_t have = (int32_t)p->table.size();
  const int32_t n = num_shared_blocks < 0 ? have : std::min(num_shared_blocks, have);
  Sequence child;
  child.table.assign(p->table.begin(), p->table.begin() + n);
  child.num_tokens = (int32_t)std::min<int64_t>(p->num_tokens, (int64_t)n * bm->block_size);
  for (int32_t b : child.table) ++bm->refcount[b];
  const int64_t id = bm->next_seq++;
  bm->seqs.emplace(id, std::move(child));
  *child_out = id;
  return PA_OK;
}

int pa_bm_allocate_prompt(pa_block_manager *bm, int64_t seq, int32_t num_tokens) {
  if (bm == nullptr || num_tokens < 0) return PA_ERR_INVALID_ARG;
  Sequence *s = bm->find(seq);
  if (s == nullptr) return PA_ERR_NO_SEQUENCE;
  const int64_t want = ((int64_t)num_tokens + bm->block_size - 1) / bm->block_size;
  const int64_t need = std::max<int64_t>(0, want - (int64_t)s->table.size());
  if (need > bm->queue_len) return PA_ERR_OUT_OF_BLOCKS;
  for (int64_t i = 0; i < need; ++i) s->table.push_back(bm->allocate());
  s->num_tokens = std::max(s->num_tokens, num_tokens);
  return PA_OK;
}

int pa_bm_prepare_write(pa_block_manager *bm, int64_t seq, int32_t position, int64_t *slot, int32_t *cow_src,
                        int32_t *cow_dst) {
  if (bm == nullptr || slot == nullptr || cow_src == nullptr || cow_dst == nullptr || position < 0)
    return PA_ERR_INVALID_ARG;
  Sequence *s = bm->find(seq);
  if (s == nullptr) return PA_ERR_NO_SEQUENCE;
  if (bm->blocks_for_write(*s, position) > bm->queue_len) return PA_ERR_OUT_OF_BLOCKS;
  bm->do_write(*s, position, slot, cow_src, cow_dst);
  return PA_OK;
}

int pa_bm_append_tokens(pa_block_manager *bm, const int64_t *seqs, int32_t n, int64_t *slots_out,
                        int32_t *cow_src_out, int32_t *cow_dst_out, int32_t *num_cow_out) {
  if (bm == nullptr || n < 0 || num_cow_out == nullptr) return PA_ERR_INVALID_ARG;
  if (n > 0 && (seqs == nullptr || slots_out == nullptr || cow_src_out == nullptr || cow_dst_out == nullptr))
    return PA_ERR_INVALID_ARG;
  // validate and count what the whole step needs before changing anything
  std::vector<Sequence *> ss(n);
  std::unordered_set<int64_t> distinct;
  std::unordered_map<int32_t, int64_t> writers;  // shared target block -> writers in this step
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    ss[i] = bm->find(seqs[i]);
    if (ss[i] == nullptr) return PA_ERR_NO_SEQUENCE;
    if (!distinct.insert(seqs[i]).second) return PA_ERR_INVALID_ARG;
    const Sequence &s = *ss[i];
    const int64_t logical = s.num_tokens / bm->block_size;
    if (logical >= (int64_t)s.table.size()) {
      need += logical + 1 - (int64_t)s.table.size();
    } else if (bm->refcount[s.table[logical]] > 1) {
      ++writers[s.table[logical]];
    }
  }
  // a shared block with r references written by k holders is copied min(k, r-1) times
  for (const auto &kv : writers) need += std::min<int64_t>(kv.second, bm->refcount[kv.first] - 1);
  if (need > bm->queue_len) return PA_ERR_OUT_OF_BLOCKS;
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    bm->do_write(*ss[i], ss[i]->num_tokens, &slots_out[i], &src, &dst);
    if (src >= 0) {
      cow_src_out[ncow] = src;
      cow_dst_out[ncow] = dst;
      ++ncow;
    }
  }
  *num_cow_out = ncow;
  return PA_OK;
}

int pa_bm_free_sequence(pa_block_manager *bm, int64_t seq, int32_t reusable) {
  if (bm == nullptr) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
  for (int32_t b : it->second.table) bm->release(b, reusable != 0);
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seqs, int32_t n, int32_t max_blocks_per_seq,
                       int32_t pad_value, int32_t *tables_out, int32_t *lens_out) {
  if (bm == nullptr || n < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if (n > 0 && (seqs == nullptr || tables_out == nullptr || lens_out == nullptr)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const Sequence *s = bm->find(seqs[i]);
    if (s == nullptr) return PA_ERR_NO_SEQUENCE;
    if ((int64_t)s->table.size() > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence *s = bm->find(seqs[i]);
    int32_t *row = tables_out + (int64_t)i * max_blocks_per_seq;
    const int32_t nb = (int32_t)s->table.size();
    std::copy(s->table.begin(), s->table.end(), row);
    std::fill(row + nb, row + max_blocks_per_seq, pad_value);
    lens_out[i] = s->num_tokens;
  }
  return PA_OK;
}

int64_t pa_bm_num_free(const pa_block_manager *bm) { return bm ? bm->queue_len : PA_ERR_INVALID_ARG; }

int64_t pa_bm_num_sequences(const pa_block_manager *bm) {
  return bm ? (int64_t)bm->seqs.size() : PA_ERR_INVALID_ARG;
}

int32_t pa_bm_refcount(const pa_block_manager *bm, int32_t block) {
  if (bm == nullptr || block < 0 || block >= bm->num_blocks) return PA_ERR_INVALID_ARG;
  return bm->refcount[block];
}

int pa_bm_sequence_info(const pa_block_manager *bm, int64_t seq, int32_t *num_tokens, int32_t *num_blocks) {
  if (bm == nullptr || num_tokens == nullptr || num_blocks == nullptr) return PA_ERR_INVALID_ARG;
  const Sequence *s = bm->find(seq);
  if (s == nullptr) return PA_ERR_NO_SEQUENCE;
  *num_tokens = s->num_tokens;
  *num_blocks = (int32_t)s->table.size();
  return PA_OK;
}

int64_t pa_bm_free_queue(const pa_block_manager *bm, int32_t *out, int64_t cap) {
  if (bm == nullptr || (out == nullptr && cap > 0)) return PA_ERR_INVALID_ARG;
  int64_t i = 0;
  for (int32_t b = bm->head; b != pa_block_manager::kNone; b = bm->next[b], ++i)
    if (i < cap) out[i] = b;
  return i;
}

}  // extern "C"
