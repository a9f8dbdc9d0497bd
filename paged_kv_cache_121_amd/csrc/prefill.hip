// Prefill / chunked-prefill attention over the paged cache for gfx950.
//
// What is computed ([HRL] section 9, prefill runs a prompt's tokens together;
// [TSS] "Next", chunked prefill takes a prompt a piece at a time; [HRL]
// section 8 for the formula): sequence s owns query rows
// query_start_loc[s] .. query_start_loc[s+1]-1, its last n_s positions, so
// row i sits at position p = context_lens[s] - n_s + i and attends causally
// over cached positions 0 .. p, found through the block table.
//
// Unlike decode this is a dense contraction, so it runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16).  One workgroup of 4 waves takes 64 query rows
// of one KV head: rows are (head of the group, token) pairs, head-major, so
// every row of the workgroup reads the same K/V.  K/V tiles of 64 keys are
// gathered through the block table into LDS (double-buffered, the next
// tile's global loads in flight while the current one is used), and each
// wave computes flash-attention style on its 16 rows:
//   S^T = K Q^T   A = K rows from LDS (ds_read_b128, XOR-swizzled rows so 16
//                 rows hit 16 different bank groups), B = Q^T held in
//                 registers.  The C layout of S^T gives every lane one row
//                 and four consecutive keys per 16-key sub-tile.
//   P V           A = P straight from those registers: the contraction's key
//                 order is permuted (slots 0-3 of a lane group are keys
//                 4g..4g+3 of one sub-tile, slots 4-7 the same keys of the
//                 next) and V's operand is built in the same order with the
//                 LDS transpose read ds_read_b64_tr_b16 from row-major V.
// P is split into bf16 high and low parts (two MFMAs), so rounding P costs
// about 2^-16 relative instead of 2^-9: a row attending over two keys would
// otherwise lose up to 2.4e-3.  Online softmax in log2 units with the
// hardware exp2, the running max raised lazily (threshold 8) as in decode.
// Keys past the context are written to LDS as zeros (never read from HBM),
// so padding slots cannot leak NaN through 0 * V.

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRows = 64;        // query rows per workgroup (16 per wave)
constexpr int kKeys = 64;        // keys per LDS tile
constexpr float kPfNegInf = -__builtin_inff();
constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfRescaleThreshold = 8.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float pf_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int D>
struct PfCfg {
  static constexpr int ROWB = D * 2;          // bytes per key row (bf16)
  static constexpr int NCH16 = D / 8;         // 16-byte chunks per row
  static constexpr int NCH8 = D / 4;          // 8-byte chunks per row
  static constexpr int TILEB = kKeys * ROWB;  // bytes of one K or V tile in LDS
  static constexpr int KC = D / 32;           // 32-dim steps of QK
  static constexpr int NT = D / 16;           // 16-dim output tiles of PV
  static constexpr int LOADS = kKeys * NCH16 / kPfThreads;  // 16-byte loads per thread per K (and V) tile
};

// LDS placement (bytes within a tile) of 16-byte chunk c of K row `key`:
// chunks are XOR-swizzled by the row so 16 rows read at one logical chunk
// land in 16 different bank groups.
template <int D>
__device__ __forceinline__ int k_lds(int key, int c) {
  return key * PfCfg<D>::ROWB + ((c ^ (key % PfCfg<D>::NCH16)) << 4);
}
// V rows are swizzled at 8-byte granularity by multiples of 4 chunks, so a
// 16-byte pair stays contiguous and the transpose read's 4-row groups spread
// over the banks.
template <int D>
__device__ __forceinline__ int v_lds8(int key, int c8) {
  return key * PfCfg<D>::ROWB + ((c8 ^ (4 * (key % (PfCfg<D>::NCH8 / 4)))) << 3);
}

template <int D, int B, int G>
__global__ void __launch_bounds__(kPfThreads)
prefill_kernel(const char *__restrict__ pool, int64_t num_blocks, int num_kv_heads, const char *__restrict__ q,
               float *__restrict__ out, const int32_t *__restrict__ query_start_loc,
               const int32_t *__restrict__ context_lens, const int32_t *__restrict__ tables,
               int max_blocks_per_seq, int num_q_heads, int total_tokens, int max_query_len, float scale_log2) {
  using C = PfCfg<D>;
  constexpr int QT = kRows / G;  // tokens per workgroup
  __shared__ __attribute__((aligned(16))) char s_k[2][C::TILEB];
  __shared__ __attribute__((aligned(16))) char s_v[2][C::TILEB];
  __shared__ int s_poison;

  const int qt = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, grp = lane >> 4;

  const int q0 = query_start_loc[s];
  const int n = query_start_loc[s + 1] - q0;
  const int ctx = context_lens[s];
  const bool bad = n < 0 || n > ctx || n > max_query_len || ctx > max_blocks_per_seq * B || q0 < 0 ||
                   (int64_t)q0 + n > total_tokens;
  if (!bad && qt * QT >= n) return;  // no rows of this sequence in this tile

  // this lane's row in the S^T layout (row r16 of the wave's 16)
  auto row_head = [&](int r) { return r / QT; };
  auto row_token = [&](int r) { return qt * QT + r % QT; };
  const int64_t hq0 = (int64_t)h * G;

  if (bad) {  // NaN rows for what this tile covers, inside the output
    if (q0 < 0 || n <= 0) return;
    for (int i = tid; i < kRows * D; i += kPfThreads) {
      const int r = i / D, d = i % D;
      const int64_t row = (int64_t)q0 + row_token(r);
      if (row_token(r) < n && row < total_tokens)
        out[(row * num_q_heads + hq0 + row_head(r)) * D + d] = __builtin_nanf("");
    }
    return;
  }

  const int my_r = wave * 16 + r16;
  const int my_t = row_token(my_r);
  const bool my_active = my_t < n;
  const int my_pos = my_active ? ctx - n + my_t : -1;

  // Q^T operand: lane holds Q[row r16][kc*32 + 8*grp .. +8] for every kc
  bf16x8_t qb[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (my_active) {
      const char *p = q + ((((int64_t)q0 + my_t) * num_q_heads + hq0 + row_head(my_r)) * D + kc * 32 + 8 * grp) * 2;
      v = *reinterpret_cast<const u32x4_t *>(p);
    }
    qb[kc] = as_bf16x8(v);
  }

  // key range this workgroup needs, and per-wave bounds for skipping/masking
  const int last_t = min(qt * QT + QT, n) - 1;
  const int kv_end = ctx - n + last_t + 1;  // keys 0 .. kv_end-1
  const int ntiles = (kv_end + kKeys - 1) / kKeys;
  int w_tmin = QT >= 16 ? (wave * 16) % QT : 0;
  int w_tmax = QT >= 16 ? w_tmin + 15 : QT - 1;
  w_tmin = qt * QT + w_tmin;
  w_tmax = min(qt * QT + w_tmax, n - 1);
  const bool wave_active = w_tmin <= w_tmax;
  const int w_pos_min = ctx - n + w_tmin;
  const int w_pos_max = ctx - n + w_tmax;

  if (tid == 0) s_poison = 0;

  // ---- global -> registers -> LDS for one tile of kKeys keys
  u32x4_t kr[C::LOADS], vr[C::LOADS];
  bool poisoned = false;
  const char *head_base = pool + (int64_t)h * B * C::ROWB;
  const int64_t kv_half = (int64_t)num_kv_heads * B * C::ROWB;  // K tile to V tile of one block
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = tid + i * kPfThreads;
      const int key = c / C::NCH16, ch = c % C::NCH16;
      const int j = t * kKeys + key;
      kr[i] = vr[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (j < ctx) {
        int b = tables[(int64_t)s * max_blocks_per_seq + j / B];
        if (b < 0 || (int64_t)b >= num_blocks) {
          poisoned = true;
          b = 0;
        }
        const char *p = head_base + (int64_t)b * 2 * kv_half + (j % B) * C::ROWB + ch * 16;
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p + kv_half));
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = tid + i * kPfThreads;
      const int key = c / C::NCH16, ch = c % C::NCH16;
      *reinterpret_cast<u32x4_t *>(&s_k[buf][k_lds<D>(key, ch)]) = kr[i];
      *reinterpret_cast<u32x4_t *>(&s_v[buf][v_lds8<D>(key, 2 * ch)]) = vr[i];
    }
  };

  // ---- per-row state: running max (log2 units), partial sum of this lane's
  // keys, and the output tile O[4*grp + jj][16*nt + r16]
  float m = kPfNegInf, lpart = 0.0f;
  f32x4_t o[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) o[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute_tile = [&](int t, int buf) {
    const int k0 = t * kKeys;
    if (!wave_active || k0 > w_pos_max) return;  // every key of the tile is after every row
    const char *kt_lds = s_k[buf];
    // S^T sub-tiles: sacc[kt] = K[16kt .. +16] Q^T
    f32x4_t sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const int key = 16 * kt + r16;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(&kt_lds[k_lds<D>(key, kc * 4 + grp)]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qb[kc], sacc[kt], 0, 0, 0);
      }
    }
    // scores of row r16, keys k0 + 16kt + 4grp + jj
    const bool full = k0 + kKeys - 1 <= w_pos_min;  // no key of the tile is masked for any row
    float sc[4][4];
    float mx = kPfNegInf;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = k0 + 16 * kt + 4 * grp + jj;
        float v = sacc[kt][jj] * scale_log2;
        if (!full && key > my_pos) v = kPfNegInf;
        sc[kt][jj] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const bool upd = mn > m + kPfRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
      const float alpha = upd ? pf_exp2(m - mn) : 1.0f;
      if (upd) m = mn;
      lpart *= alpha;
      // O rows are 4*grp + jj: fetch those rows' factors
      float ar[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ar[jj] = __shfl(alpha, 4 * grp + jj);
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o[nt][jj] *= ar[jj];
    }
    const float ms = m == kPfNegInf ? 0.0f : m;
    // P = exp2(s - m), split into bf16 high and low parts, in the permuted key order
    bf16x8_t ph[2], pl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float pv = pf_exp2(sc[2 * ks + half][jj] - ms);
          lpart += pv;
          const __bf16 hi = (__bf16)pv;
          ph[ks][4 * half + jj] = hi;
          pl[ks][4 * half + jj] = (__bf16)(pv - (float)hi);
        }
    // O += P V: V operand by transpose reads, keys in the same permuted order
    const char *vt_lds = s_v[buf];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        i16x4_t lo4, hi4;
        {
          const int key = 32 * ks + 4 * grp + r16 / 4;
          lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t *)(vt_lds + v_lds8<D>(key, 4 * nt + (r16 & 3))));
        }
        {
          const int key = 32 * ks + 16 + 4 * grp + r16 / 4;
          hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t *)(vt_lds + v_lds8<D>(key, 4 * nt + (r16 & 3))));
        }
        const bf16x8_t vb = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[ks], vb, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[ks], vb, o[nt], 0, 0, 0);
      }
    }
  };

  // ---- main loop over key tiles
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);
    compute_tile(t, t & 1);
    if (more) store_tile((t + 1) & 1);
    __syncthreads();
  }
  if (poisoned) s_poison = 1;
  __syncthreads();
  const bool seq_poisoned = s_poison != 0;

  // ---- normalise and store: row totals, then each O row divided by its total
  float lrow = lpart + __shfl_xor(lpart, 16);
  lrow += __shfl_xor(lrow, 32);
  const float inv = lrow > 0.0f ? 1.0f / lrow : 0.0f;
  float inv_r[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) inv_r[jj] = __shfl(inv, 4 * grp + jj);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int r = wave * 16 + 4 * grp + jj;
    const int tok = row_token(r);
    if (tok >= n) continue;
    float *dst = out + (((int64_t)q0 + tok) * num_q_heads + hq0 + row_head(r)) * D + r16;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
      dst[16 * nt] = seq_poisoned ? __builtin_nanf("") : o[nt][jj] * inv_r[jj];
  }
}

template <int D, int B, int G>
hipError_t prefill_one(const PrefillArgs &a, hipStream_t stream) {
  constexpr int QT = kRows / G;
  const dim3 grid((a.max_query_len + QT - 1) / QT, a.pool.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((prefill_kernel<D, B, G>), grid, dim3(kPfThreads), 0, stream,
                     static_cast<const char *>(a.pool.base), a.pool.num_blocks, a.pool.num_kv_heads,
                     static_cast<const char *>(a.q), a.out, a.query_start_loc, a.context_lens, a.block_tables,
                     a.max_blocks_per_seq, a.num_q_heads, a.total_tokens, a.max_query_len, a.scale * kPfLog2e);
  return hipGetLastError();
}

template <int D, int B>
hipError_t prefill_group(const PrefillArgs &a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return prefill_one<D, B, 1>(a, stream);
    case 2: return prefill_one<D, B, 2>(a, stream);
    case 4: return prefill_one<D, B, 4>(a, stream);
    case 8: return prefill_one<D, B, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t prefill_block(const PrefillArgs &a, int group, hipStream_t stream) {
  switch (a.pool.block_size) {
    case 16: return prefill_group<D, 16>(a, group, stream);
    case 32: return prefill_group<D, 32>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int block_size, int group) {
  return dtype == PA_BF16 && (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  const int group = a.num_q_heads / a.pool.num_kv_heads;
  if (a.pool.head_dim == 128) return prefill_block<128>(a, group, stream);
  if (a.pool.head_dim == 64) return prefill_block<64>(a, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
