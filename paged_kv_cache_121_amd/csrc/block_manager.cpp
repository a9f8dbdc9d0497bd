// Host-side block manager of the paged KV cache (see include/pa_blocks.h).
//
// The free queue is a doubly linked list threaded through per-block arrays,
// so taking the front, returning a block to either end and unlinking a
// block from the middle are all O(1).  Every mutating call first checks
// that it can complete (enough free blocks, valid ids) and only then
// changes state, so a failed call leaves the manager untouched.
//
// Prefix caching keeps a hash table from a full block's chained digest to
// the block holding it, and the reverse per block.  The digest is SHA-256
// (FIPS 180-4), written out below from the standard's definition.

#include "pa_blocks.h"

#include <algorithm>
#include <array>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"

#if defined(__x86_64__)
#include <cpuid.h>
#include <immintrin.h>
#endif

namespace {

// ---------------------------------------------------------------- SHA-256 (FIPS 180-4)

using Digest = std::array<uint8_t, 32>;

// First 32 bits of the fractional parts of the cube roots of the first 64 primes.
constexpr uint32_t kRound[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4, 0xab1c5ed5,
    0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe, 0x9bdc06a7, 0xc19bf174,
    0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f, 0x4a7484aa, 0x5cb0a9dc, 0x76f988da,
    0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7, 0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967,
    0x27b70a85, 0x2e1b2138, 0x4d2c6dfc, 0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85,
    0xa2bfe8a1, 0xa81a664b, 0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070,
    0x19a4c116, 0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7, 0xc67178f2};
// First 32 bits of the fractional parts of the square roots of the first 8 primes.
constexpr uint32_t kInit[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                               0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

// The compression function over n consecutive 64-byte chunks, portable.
void compress_portable(uint32_t h[8], const uint8_t *data, size_t n) {
  for (; n > 0; --n, data += 64) {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t)data[4 * t] << 24 | (uint32_t)data[4 * t + 1] << 16 | (uint32_t)data[4 * t + 2] << 8 |
             (uint32_t)data[4 * t + 3];
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], k = h[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t t1 = k + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) + kRound[t] + w[t];
      const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
      k = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d;
    h[4] += e; h[5] += f; h[6] += g; h[7] += k;
  }
}

#if defined(__x86_64__)
// The same function on the x86 SHA extensions (Intel's SHA-NI: SHA256RNDS2 does two
// rounds on a state split as ABEF / CDGH, SHA256MSG1 / SHA256MSG2 extend the message
// schedule four words at a time).  Lane 0 of a register holds the earliest word.
__attribute__((target("sha,sse4.1,ssse3"))) void compress_shani(uint32_t h[8], const uint8_t *data, size_t n) {
  const __m128i bswap = _mm_set_epi8(12, 13, 14, 15, 8, 9, 10, 11, 4, 5, 6, 7, 0, 1, 2, 3);
  const __m128i abcd = _mm_loadu_si128((const __m128i *)&h[0]);
  const __m128i efgh = _mm_loadu_si128((const __m128i *)&h[4]);
  const __m128i badc = _mm_shuffle_epi32(abcd, 0xB1);  // lanes b a d c
  const __m128i hgfe = _mm_shuffle_epi32(efgh, 0x1B);  // lanes h g f e
  __m128i abef = _mm_alignr_epi8(badc, hgfe, 8);       // lanes f e b a
  __m128i cdgh = _mm_blend_epi16(hgfe, badc, 0xF0);    // lanes h g d c
  for (; n > 0; --n, data += 64) {
    const __m128i abef0 = abef, cdgh0 = cdgh;
    __m128i w[4];
    for (int j = 0; j < 16; ++j) {
      if (j < 4) {
        w[j] = _mm_shuffle_epi8(_mm_loadu_si128((const __m128i *)(data + 16 * j)), bswap);
      } else {
        // words 4j..4j+3 from words 4j-16.. (w[j%4]), 4j-12.., 4j-8.., 4j-4..
        const __m128i &m16 = w[j & 3], &m12 = w[(j + 1) & 3], &m8 = w[(j + 2) & 3], &m4 = w[(j + 3) & 3];
        __m128i t = _mm_sha256msg1_epu32(m16, m12);  // + sigma0 of words 4j-15..4j-12
        t = _mm_add_epi32(t, _mm_alignr_epi8(m4, m8, 4));  // + words 4j-7..4j-4
        w[j & 3] = _mm_sha256msg2_epu32(t, m4);      // + sigma1 of words 4j-2..4j+1
      }
      __m128i wk = _mm_add_epi32(w[j & 3], _mm_loadu_si128((const __m128i *)&kRound[4 * j]));
      cdgh = _mm_sha256rnds2_epu32(cdgh, abef, wk);  // rounds 4j, 4j+1: new ABEF in cdgh
      wk = _mm_shuffle_epi32(wk, 0x0E);
      abef = _mm_sha256rnds2_epu32(abef, cdgh, wk);  // rounds 4j+2, 4j+3
    }
    abef = _mm_add_epi32(abef, abef0);
    cdgh = _mm_add_epi32(cdgh, cdgh0);
  }
  const __m128i x = _mm_shuffle_epi32(abef, 0x1B);  // lanes a b e f
  const __m128i y = _mm_shuffle_epi32(cdgh, 0x1B);  // lanes c d g h
  _mm_storeu_si128((__m128i *)&h[0], _mm_unpacklo_epi64(x, y));
  _mm_storeu_si128((__m128i *)&h[4], _mm_unpackhi_epi64(x, y));
}

bool cpu_has_sha() {
  unsigned a, b, c, d;
  if (!__get_cpuid(1, &a, &b, &c, &d) || !(c & bit_SSE4_1) || !(c & bit_SSSE3)) return false;
  if (!__get_cpuid_count(7, 0, &a, &b, &c, &d)) return false;
  return (b & (1u << 29)) != 0;  // CPUID.(EAX=7,ECX=0):EBX.SHA
}
#endif

using CompressFn = void (*)(uint32_t *, const uint8_t *, size_t);

// The SHA extensions when the CPU has them, unless PA_SHA256_PORTABLE is set.
CompressFn pick_compress() {
#if defined(__x86_64__)
  const char *env = std::getenv("PA_SHA256_PORTABLE");
  if ((env == nullptr || env[0] == '\0' || env[0] == '0') && cpu_has_sha()) return compress_shani;
#endif
  return compress_portable;
}

const CompressFn compress = pick_compress();

Digest sha256(const uint8_t *msg, size_t len) {
  uint32_t h[8];
  std::memcpy(h, kInit, sizeof h);
  const size_t whole = len / 64;
  if (whole) compress(h, msg, whole);
  // padding: 0x80, zeros, then the message length in bits, big-endian
  uint8_t tail[128] = {};
  const size_t rest = len - 64 * whole;
  std::memcpy(tail, msg + 64 * whole, rest);
  tail[rest] = 0x80;
  const size_t tail_len = rest + 9 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)len * 8;
  for (int i = 0; i < 8; ++i) tail[tail_len - 1 - i] = (uint8_t)(bits >> (8 * i));
  compress(h, tail, tail_len / 64);
  Digest out;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
  return out;
}

// Digest of one full block: SHA-256 over the parent's digest, then the
// block's token ids as little-endian int32.
Digest hash_block(const Digest &parent, const int32_t *ids, int32_t block_size, std::vector<uint8_t> &buf) {
  buf.resize(32 + 4 * (size_t)block_size);
  std::memcpy(buf.data(), parent.data(), 32);
#if __BYTE_ORDER__ == __ORDER_LITTLE_ENDIAN__
  std::memcpy(buf.data() + 32, ids, 4 * (size_t)block_size);
#else
  for (int32_t i = 0; i < block_size; ++i) {
    const uint32_t v = (uint32_t)ids[i];
    for (int j = 0; j < 4; ++j) buf[32 + 4 * (size_t)i + j] = (uint8_t)(v >> (8 * j));
  }
#endif
  return sha256(buf.data(), buf.size());
}

struct DigestHash {
  size_t operator()(const Digest &d) const {
    uint64_t v;
    std::memcpy(&v, d.data(), 8);
    return (size_t)v;
  }
};

struct Sequence {
  int32_t num_tokens = 0;
  std::vector<int32_t> table;   // logical block -> physical block
  std::vector<int32_t> tokens;  // committed token ids (a prefix of the positions)
  std::vector<Digest> chain;    // digest of each full block of `tokens`
  bool on_host = false;         // swapped out: `table` holds host pool blocks
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
  // prefix cache: digest -> block, and each block's digest while it has one
  std::unordered_map<Digest, int32_t, DigestHash> cached;
  std::vector<Digest> digest_of;
  std::vector<uint8_t> has_digest;
  std::vector<uint8_t> scratch;  // hashing buffer
  // host pool for swapped-out sequences: its own block ids, counts and free queue
  std::vector<int32_t> host_ref;
  std::deque<int32_t> host_free;

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
  void forget(int32_t b) {
    if (has_digest[b]) {
      cached.erase(digest_of[b]);
      has_digest[b] = 0;
    }
  }
  // Enter b under d unless b already has a digest or d already has a block.
  void enter(int32_t b, const Digest &d) {
    if (has_digest[b] || cached.count(d)) return;
    cached.emplace(d, b);
    digest_of[b] = d;
    has_digest[b] = 1;
  }
  // Callers check queue_len first.  A cached block taken here is evicted.
  int32_t allocate() {
    const int32_t b = head;
    unlink(b);
    refcount[b] = 1;
    forget(b);
    return b;
  }
  // One more reference to a cached block, off the free queue if it was idle.
  void touch(int32_t b) {
    if (refcount[b] == 0 && queued[b]) unlink(b);
    ++refcount[b];
  }
  // At zero references: back of the queue if reusable or cached, else front.
  void release(int32_t b, bool reusable) {
    if (--refcount[b] == 0) {
      if (reusable || has_digest[b]) push_back(b); else push_front(b);
    }
  }
  // Host pool: take the front, return to the front.
  int32_t host_allocate() {
    const int32_t h = host_free.front();
    host_free.pop_front();
    host_ref[h] = 1;
    return h;
  }
  void host_release(int32_t h) {
    if (--host_ref[h] == 0) host_free.push_front(h);
  }
  // Record ids past the committed ones (the caller checked they fit in
  // num_tokens) and enter every block they complete.
  void commit(Sequence &s, const int32_t *ids, int32_t n) {
    s.tokens.insert(s.tokens.end(), ids, ids + n);
    const size_t full = s.tokens.size() / block_size;
    while (s.chain.size() < full) {
      const size_t j = s.chain.size();
      static const Digest kRoot{};
      const Digest &parent = j == 0 ? kRoot : s.chain[j - 1];
      s.chain.push_back(hash_block(parent, s.tokens.data() + j * block_size, block_size, scratch));
      enter(s.table[j], s.chain[j]);
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
  // Grow + copy-on-write + slot; the caller has checked the free blocks and
  // that the position is not committed.  The written block loses its digest.
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
    forget(b);
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
  bm->digest_of.assign(num_blocks, Digest{});
  bm->has_digest.assign(num_blocks, 0);
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
  if (p->on_host) return PA_ERR_SWAPPED;
  const int32_t have = (int32_t)p->table.size();
  const int32_t n = num_shared_blocks < 0 ? have : std::min(num_shared_blocks, have);
  Sequence child;
  child.table.assign(p->table.begin(), p->table.begin() + n);
  child.num_tokens = (int32_t)std::min<int64_t>(p->num_tokens, (int64_t)n * bm->block_size);
  const size_t ntok = std::min<size_t>(p->tokens.size(), (size_t)child.num_tokens);
  child.tokens.assign(p->tokens.begin(), p->tokens.begin() + ntok);
  child.chain.assign(p->chain.begin(), p->chain.begin() + ntok / bm->block_size);
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
  if (s->on_host) return PA_ERR_SWAPPED;
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
  if (s->on_host) return PA_ERR_SWAPPED;
  if ((size_t)position < s->tokens.size()) return PA_ERR_INVALID_ARG;  // committed
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
    if (ss[i]->on_host) return PA_ERR_SWAPPED;
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
  const std::vector<int32_t> &t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) {  // last block first
    if (it->second.on_host) bm->host_release(*b); else bm->release(*b, reusable != 0);
  }
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
    if (s->on_host) return PA_ERR_SWAPPED;
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

int pa_bm_hash_blocks(const int32_t *tokens, int64_t num_tokens, int32_t block_size, const uint8_t *parent,
                      uint8_t *digests_out) {
  if (num_tokens < 0 || block_size <= 0 || (num_tokens > 0 && tokens == nullptr)) return PA_ERR_INVALID_ARG;
  const int64_t full = num_tokens / block_size;
  if (full > INT32_MAX || (full > 0 && digests_out == nullptr)) return PA_ERR_INVALID_ARG;
  Digest h{};
  if (parent != nullptr) std::memcpy(h.data(), parent, 32);
  std::vector<uint8_t> buf;
  for (int64_t j = 0; j < full; ++j) {
    h = hash_block(h, tokens + j * block_size, block_size, buf);
    std::memcpy(digests_out + 32 * j, h.data(), 32);
  }
  return (int)full;
}

namespace {
// Digests of the full blocks of a prompt, and how many leading ones are
// cached, at most floor((n - 1) / B).
int32_t prompt_hits(pa_block_manager *bm, const int32_t *tokens, int32_t n, std::vector<Digest> &digests,
                    std::vector<int32_t> &hit_blocks) {
  const int32_t B = bm->block_size;
  const int32_t full = n / B;
  const int32_t limit = n > 0 ? (n - 1) / B : 0;
  digests.resize(full);
  hit_blocks.clear();
  Digest h{};
  bool run = true;
  for (int32_t j = 0; j < full; ++j) {
    h = hash_block(h, tokens + (int64_t)j * B, B, bm->scratch);
    digests[j] = h;
    if (run && j < limit) {
      auto it = bm->cached.find(h);
      if (it == bm->cached.end()) run = false; else hit_blocks.push_back(it->second);
    }
  }
  return (int32_t)hit_blocks.size();
}
}  // namespace

int pa_bm_lookup_prefix(pa_block_manager *bm, const int32_t *tokens, int32_t num_tokens,
                        int32_t *num_cached_tokens) {
  if (bm == nullptr || num_cached_tokens == nullptr || num_tokens < 0 || (num_tokens > 0 && tokens == nullptr))
    return PA_ERR_INVALID_ARG;
  std::vector<Digest> digests;
  std::vector<int32_t> hits;
  *num_cached_tokens = prompt_hits(bm, tokens, num_tokens, digests, hits) * bm->block_size;
  return PA_OK;
}

int pa_bm_allocate_prompt_cached(pa_block_manager *bm, int64_t seq, const int32_t *tokens, int32_t num_tokens,
                                 int32_t *num_cached_tokens) {
  if (bm == nullptr || num_cached_tokens == nullptr || num_tokens < 0 || (num_tokens > 0 && tokens == nullptr))
    return PA_ERR_INVALID_ARG;
  Sequence *s = bm->find(seq);
  if (s == nullptr) return PA_ERR_NO_SEQUENCE;
  if (s->on_host) return PA_ERR_SWAPPED;
  if (!s->table.empty() || s->num_tokens != 0) return PA_ERR_INVALID_ARG;
  std::vector<Digest> digests;
  std::vector<int32_t> hits;
  const int32_t nhit = prompt_hits(bm, tokens, num_tokens, digests, hits);
  const int64_t fresh = ((int64_t)num_tokens + bm->block_size - 1) / bm->block_size - nhit;
  int64_t idle = 0;
  for (int32_t b : hits) idle += bm->refcount[b] == 0;
  if (fresh + idle > bm->queue_len) return PA_ERR_OUT_OF_BLOCKS;
  for (int32_t b : hits) {
    bm->touch(b);
    s->table.push_back(b);
  }
  for (int64_t i = 0; i < fresh; ++i) s->table.push_back(bm->allocate());
  s->num_tokens = num_tokens;
  s->tokens.assign(tokens, tokens + num_tokens);
  s->chain = std::move(digests);
  for (size_t j = 0; j < s->chain.size(); ++j) bm->enter(s->table[j], s->chain[j]);
  *num_cached_tokens = nhit * bm->block_size;
  return PA_OK;
}

int pa_bm_commit_tokens(pa_block_manager *bm, int64_t seq, const int32_t *ids, int32_t n) {
  if (bm == nullptr || n < 0 || (n > 0 && ids == nullptr)) return PA_ERR_INVALID_ARG;
  Sequence *s = bm->find(seq);
  if (s == nullptr) return PA_ERR_NO_SEQUENCE;
  if (s->on_host) return PA_ERR_SWAPPED;
  if ((int64_t)s->tokens.size() + n > s->num_tokens) return PA_ERR_INVALID_ARG;
  bm->commit(*s, ids, n);
  return PA_OK;
}

int64_t pa_bm_num_cached(const pa_block_manager *bm) { return bm ? (int64_t)bm->cached.size() : PA_ERR_INVALID_ARG; }

int pa_bm_block_digest(const pa_block_manager *bm, int32_t block, uint8_t *digest_out) {
  if (bm == nullptr || block < 0 || block >= bm->num_blocks || digest_out == nullptr) return PA_ERR_INVALID_ARG;
  if (!bm->has_digest[block]) return 0;
  std::memcpy(digest_out, bm->digest_of[block].data(), 32);
  return 1;
}

int pa_bm_set_host_pool(pa_block_manager *bm, int64_t num_host_blocks) {
  if (bm == nullptr || num_host_blocks < 0 || num_host_blocks > INT32_MAX) return PA_ERR_INVALID_ARG;
  for (const auto &kv : bm->seqs)
    if (kv.second.on_host) return PA_ERR_INVALID_ARG;  // host blocks in use
  bm->host_ref.assign(num_host_blocks, 0);
  bm->host_free.clear();
  for (int64_t h = 0; h < num_host_blocks; ++h) bm->host_free.push_back((int32_t)h);
  return PA_OK;
}

}  // extern "C"

namespace {
// Validate a swap group: known, distinct, all on the given side.
int swap_group(pa_block_manager *bm, const int64_t *seqs, int32_t n, bool on_host, std::vector<Sequence *> &ss) {
  if (n < 0 || (n > 0 && seqs == nullptr)) return PA_ERR_INVALID_ARG;
  ss.resize(n);
  std::unordered_set<int64_t> distinct;
  for (int32_t i = 0; i < n; ++i) {
    ss[i] = bm->find(seqs[i]);
    if (ss[i] == nullptr) return PA_ERR_NO_SEQUENCE;
    if (!distinct.insert(seqs[i]).second) return PA_ERR_INVALID_ARG;
    if (ss[i]->on_host != on_host) return on_host ? PA_ERR_INVALID_ARG : PA_ERR_SWAPPED;
  }
  return PA_OK;
}

// Move the group's tables to the other pool: the first holder of each block
// takes a fresh block there (one copy pair), later holders share it; then each
// sequence drops its references in the pool it left, last block first.
template <typename Alloc, typename Share, typename Release>
int32_t move_group(std::vector<Sequence *> &ss, Alloc alloc_dst, Share share_dst, Release release_src,
                   int32_t *src_out, int32_t *dst_out) {
  std::unordered_map<int32_t, int32_t> mapping;
  std::vector<std::vector<int32_t>> tables(ss.size());
  int32_t npairs = 0;
  for (size_t i = 0; i < ss.size(); ++i) {
    for (int32_t b : ss[i]->table) {
      auto it = mapping.find(b);
      if (it != mapping.end()) {
        share_dst(it->second);
        tables[i].push_back(it->second);
      } else {
        const int32_t d = alloc_dst();
        mapping.emplace(b, d);
        src_out[npairs] = b;
        dst_out[npairs] = d;
        ++npairs;
        tables[i].push_back(d);
      }
    }
  }
  for (size_t i = 0; i < ss.size(); ++i) {
    const std::vector<int32_t> &t = ss[i]->table;
    for (auto b = t.rbegin(); b != t.rend(); ++b) release_src(*b);
    ss[i]->table = std::move(tables[i]);
  }
  return npairs;
}

int64_t distinct_blocks(const std::vector<Sequence *> &ss) {
  std::unordered_set<int32_t> d;
  for (const Sequence *s : ss) d.insert(s->table.begin(), s->table.end());
  return (int64_t)d.size();
}
}  // namespace

extern "C" {

int pa_bm_swap_out(pa_block_manager *bm, const int64_t *seqs, int32_t n, int32_t *gpu_blocks_out,
                   int32_t *host_blocks_out, int32_t *num_pairs_out) {
  if (bm == nullptr || num_pairs_out == nullptr) return PA_ERR_INVALID_ARG;
  std::vector<Sequence *> ss;
  const int st = swap_group(bm, seqs, n, false, ss);
  if (st != PA_OK) return st;
  const int64_t need = distinct_blocks(ss);
  if (need > 0 && (gpu_blocks_out == nullptr || host_blocks_out == nullptr)) return PA_ERR_INVALID_ARG;
  if (need > (int64_t)bm->host_free.size()) return PA_ERR_OUT_OF_BLOCKS;
  *num_pairs_out = move_group(
      ss, [bm] { return bm->host_allocate(); }, [bm](int32_t h) { ++bm->host_ref[h]; },
      [bm](int32_t b) { bm->release(b, false); }, gpu_blocks_out, host_blocks_out);
  for (Sequence *s : ss) s->on_host = true;
  return PA_OK;
}

int pa_bm_swap_in(pa_block_manager *bm, const int64_t *seqs, int32_t n, int32_t *host_blocks_out,
                  int32_t *gpu_blocks_out, int32_t *num_pairs_out) {
  if (bm == nullptr || num_pairs_out == nullptr) return PA_ERR_INVALID_ARG;
  std::vector<Sequence *> ss;
  const int st = swap_group(bm, seqs, n, true, ss);
  if (st != PA_OK) return st;
  const int64_t need = distinct_blocks(ss);
  if (need > 0 && (gpu_blocks_out == nullptr || host_blocks_out == nullptr)) return PA_ERR_INVALID_ARG;
  if (need > bm->queue_len) return PA_ERR_OUT_OF_BLOCKS;
  *num_pairs_out = move_group(
      ss, [bm] { return bm->allocate(); }, [bm](int32_t b) { ++bm->refcount[b]; },
      [bm](int32_t h) { bm->host_release(h); }, host_blocks_out, gpu_blocks_out);
  for (Sequence *s : ss) s->on_host = false;
  return PA_OK;
}

int64_t pa_bm_num_free_host(const pa_block_manager *bm) {
  return bm ? (int64_t)bm->host_free.size() : PA_ERR_INVALID_ARG;
}

int pa_bm_sequence_on_host(const pa_block_manager *bm, int64_t seq) {
  if (bm == nullptr) return PA_ERR_INVALID_ARG;
  const Sequence *s = bm->find(seq);
  if (s == nullptr) return PA_ERR_NO_SEQUENCE;
  return s->on_host ? 1 : 0;
}

int32_t pa_bm_host_refcount(const pa_block_manager *bm, int32_t block) {
  if (bm == nullptr || block < 0 || block >= (int64_t)bm->host_ref.size()) return PA_ERR_INVALID_ARG;
  return bm->host_ref[block];
}

int64_t pa_bm_host_free_queue(const pa_block_manager *bm, int32_t *out, int64_t cap) {
  if (bm == nullptr || (out == nullptr && cap > 0)) return PA_ERR_INVALID_ARG;
  int64_t i = 0;
  for (int32_t h : bm->host_free) {
    if (i < cap) out[i] = h;
    ++i;
  }
  return i;
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
