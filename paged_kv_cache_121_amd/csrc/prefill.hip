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
// (v_mfma_f32_16x16x32_bf16).  One workgroup of 4 waves takes 128 query rows
// of one KV head (32 per wave, two 16-row groups sharing every K and V
// operand read): rows are (head of the group, token) pairs, head-major, so
// every row of the workgroup reads the same K/V.  K/V tiles of 64 keys are
// gathered through the block table into LDS (double-buffered, the next
// tile's global loads in flight while the current one is used), and each
// wave computes flash-attention style on its rows:
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

#ifndef PA_PREFILL_ROW_GROUPS
#define PA_PREFILL_ROW_GROUPS 1
#endif

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
// 16-row groups per wave: every K or V operand read from LDS feeds RG
// matrix-core instructions, so LDS traffic per flop falls as 1/RG.
constexpr int kRG = PA_PREFILL_ROW_GROUPS;
constexpr int kRows = 16 * kRG * kPfWaves;  // query rows per workgroup
constexpr int kKeys = 64;                    // keys per LDS tile
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

// Max / sum over the four 16-lane groups of the wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap permutes: with both operands the same value,
// permlane16_swap yields the values of lanes (l & ~16, l | 16) and
// permlane32_swap those of (l & ~32, l | 32) -- VALU only, no LDS round trip.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

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

// Two waves per SIMD: the register budget that lets two workgroups share a
// compute unit (their LDS fits as well), so one's loads overlap the other's math.
template <int D, int B, int G>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
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

  // rows of this wave: 16*kRG consecutive rows starting at wave*16*kRG;
  // lane (r16, grp) owns row wave*16*kRG + 16*rg + r16 of group rg
  int my_pos[kRG];
  bool my_active[kRG];
  bf16x8_t qb[kRG][C::KC];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const int r = wave * 16 * kRG + 16 * rg + r16;
    const int t = row_token(r);
    my_active[rg] = t < n;
    my_pos[rg] = my_active[rg] ? ctx - n + t : -1;
    // Q^T operand: lane holds Q[row][kc*32 + 8*grp .. +8] for every kc
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (my_active[rg]) {
        const char *p = q + ((((int64_t)q0 + t) * num_q_heads + hq0 + row_head(r)) * D + kc * 32 + 8 * grp) * 2;
        v = *reinterpret_cast<const u32x4_t *>(p);
      }
      qb[rg][kc] = as_bf16x8(v);
    }
  }

  // key range this workgroup needs, and per-wave bounds for skipping/masking
  const int last_t = min(qt * QT + QT, n) - 1;
  const int kv_end = ctx - n + last_t + 1;  // keys 0 .. kv_end-1
  const int ntiles = (kv_end + kKeys - 1) / kKeys;
  constexpr int WR = 16 * kRG;  // rows per wave
  int w_tmin = QT >= WR ? (wave * WR) % QT : 0;
  int w_tmax = QT >= WR ? w_tmin + WR - 1 : QT - 1;
  w_tmin = qt * QT + w_tmin;
  w_tmax = min(qt * QT + w_tmax, n - 1);
  const bool wave_active = w_tmin <= w_tmax;
  const int w_pos_min = ctx - n + w_tmin;
  const int w_pos_max = ctx - n + w_tmax;

  if (tid == 0) s_poison = 0;

  // ---- global -> registers -> LDS for one tile of kKeys keys.  The tile's
  // block ids are uniform (scalar loads, validated once); every lane then
  // issues its K/V loads unconditionally at in-bounds addresses (keys past
  // the sequence read block 0 and are replaced by zeros), so no load waits
  // on a per-lane table read and no branch splits the wave.
  // A tile spans NBT whole blocks (B <= kKeys) or a kKeys-key slice of one
  // block (B > kKeys).
  constexpr int NBT = B <= kKeys ? kKeys / B : 1;
  static_assert(B % 4 == 0 && (B <= kKeys ? kKeys % B == 0 : B % kKeys == 0), "block size");
  u32x4_t kr[C::LOADS], vr[C::LOADS];
  bool poisoned = false;
  const int seq_blocks = (ctx + B - 1) / B;
  const char *head_base = pool + (int64_t)h * B * C::ROWB;
  const int64_t kv_half = (int64_t)num_kv_heads * B * C::ROWB;  // K tile to V tile of one block
  const int32_t *table_row = tables + (int64_t)s * max_blocks_per_seq;
  auto load_tile = [&](int t) {
    int blk[NBT];
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      const int jb = B <= kKeys ? t * NBT + i : t / (B / kKeys);
      int b = jb < seq_blocks ? table_row[jb] : 0;
      b = __builtin_amdgcn_readfirstlane(b);
      if (b < 0 || (int64_t)b >= num_blocks) {
        poisoned = true;
        b = 0;
      }
      blk[i] = b;
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = tid + i * kPfThreads;
      const int key = c / C::NCH16, ch = c % C::NCH16;
      int b = blk[0];
      int row_in_block;
      if constexpr (B <= kKeys) {
        const int slot = key / B;  // uniform per i for D = 128 and B >= 16
#pragma unroll
        for (int k = 1; k < NBT; ++k) b = slot == k ? blk[k] : b;
        row_in_block = key % B;
      } else {
        row_in_block = (t % (B / kKeys)) * kKeys + key;
      }
      const char *p = head_base + (int64_t)b * 2 * kv_half + row_in_block * C::ROWB + ch * 16;
      const bool valid = t * kKeys + key < ctx;
      const u32x4_t kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
      const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p + kv_half));
      const u32x4_t zero = {0u, 0u, 0u, 0u};
      kr[i] = valid ? kv : zero;
      vr[i] = valid ? vv : zero;
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
  // keys, and the output tiles O[4*grp + jj][16*nt + r16] of each row group
  float m[kRG], lpart[kRG];
  f32x4_t o[kRG][C::NT];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    m[rg] = kPfNegInf;
    lpart[rg] = 0.0f;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) o[rg][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Per-lane LDS byte offsets of the operand reads for sub-tile 0; the
  // sub-tile, key-step and buffer offsets are compile-time constants that
  // fold into the instructions' immediate offsets (the swizzle term depends
  // only on the lane because 16kt, 32ks and 16 are multiples of its period).
  int k_base[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) k_base[kc] = k_lds<D>(r16, kc * 4 + grp);
  int v_base[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) v_base[nt] = v_lds8<D>(4 * grp + r16 / 4, 4 * nt + (r16 & 3));

  auto compute_tile = [&](int t, auto buf_tag) {
    constexpr int buf = decltype(buf_tag)::value;
    const int k0 = t * kKeys;
    if (!wave_active || k0 > w_pos_max) return;  // every key of the tile is after every row
    const char *kt_lds = s_k[buf];
    // S^T sub-tiles: sacc[rg][kt] = K[16kt .. +16] Q_rg^T; each K operand serves every row group
    f32x4_t sacc[kRG][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) sacc[rg][kt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(&kt_lds[k_base[kc] + 16 * kt * C::ROWB]);
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg)
          sacc[rg][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qb[rg][kc], sacc[rg][kt], 0, 0, 0);
      }
    }
    const bool full = k0 + kKeys - 1 <= w_pos_min;  // no key of the tile is masked for any row
    bf16x8_t ph[kRG][2], pl[kRG][2];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      // scores of this lane's row, keys k0 + 16kt + 4grp + jj
      float sc[4][4];
      float mx = kPfNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = k0 + 16 * kt + 4 * grp + jj;
          float v = sacc[rg][kt][jj] * scale_log2;
          if (!full && key > my_pos[rg]) v = kPfNegInf;
          sc[kt][jj] = v;
          mx = fmaxf(mx, v);
        }
      mx = group_max(mx);
      const float mn = fmaxf(m[rg], mx);
      const bool upd = mn > m[rg] + kPfRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(upd) != 0) {
        const float alpha = upd ? pf_exp2(m[rg] - mn) : 1.0f;
        if (upd) m[rg] = mn;
        lpart[rg] *= alpha;
        // O rows are 4*grp + jj: fetch those rows' factors
        float ar[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ar[jj] = __shfl(alpha, 4 * grp + jj);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) o[rg][nt][jj] *= ar[jj];
      }
      const float ms = m[rg] == kPfNegInf ? 0.0f : m[rg];
      // P = exp2(s - m), split into bf16 high and low parts, in the permuted key order
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float pv = pf_exp2(sc[2 * ks + half][jj] - ms);
            lpart[rg] += pv;
            const __bf16 hi = (__bf16)pv;
            ph[rg][ks][4 * half + jj] = hi;
            pl[rg][ks][4 * half + jj] = (__bf16)(pv - (float)hi);
          }
    }
    // O += P V: V operand by transpose reads, keys in the same permuted order; each serves every row group
    const char *vt_lds = s_v[buf];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i16x4_t lo4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vt_lds + v_base[nt] + 32 * ks * C::ROWB));
        const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t *)(vt_lds + v_base[nt] + (32 * ks + 16) * C::ROWB));
        const bf16x8_t vb = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) {
          o[rg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[rg][ks], vb, o[rg][nt], 0, 0, 0);
          o[rg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[rg][ks], vb, o[rg][nt], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop over key tiles, unrolled by two so each half uses a fixed
  // LDS buffer (its offsets are immediates)
  using buf0 = std::integral_constant<int, 0>;
  using buf1 = std::integral_constant<int, 1>;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) load_tile(t + 1);
    compute_tile(t, buf0{});
    if (t + 1 < ntiles) store_tile(1);
    __syncthreads();
    if (t + 1 >= ntiles) break;
    if (t + 2 < ntiles) load_tile(t + 2);
    compute_tile(t + 1, buf1{});
    if (t + 2 < ntiles) store_tile(0);
    __syncthreads();
  }
  if (poisoned) s_poison = 1;
  __syncthreads();
  const bool seq_poisoned = s_poison != 0;

  // ---- normalise and store: row totals, then each O row divided by its total
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const float lrow = group_sum(lpart[rg]);
    const float inv = lrow > 0.0f ? 1.0f / lrow : 0.0f;
    float inv_r[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) inv_r[jj] = __shfl(inv, 4 * grp + jj);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = wave * 16 * kRG + 16 * rg + 4 * grp + jj;
      const int tok = row_token(r);
      if (tok >= n) continue;
      float *dst = out + (((int64_t)q0 + tok) * num_q_heads + hq0 + row_head(r)) * D + r16;
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
        dst[16 * nt] = seq_poisoned ? __builtin_nanf("") : o[rg][nt][jj] * inv_r[jj];
    }
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
    case 4: return prefill_group<D, 4>(a, group, stream);
    case 8: return prefill_group<D, 8>(a, group, stream);
    case 16: return prefill_group<D, 16>(a, group, stream);
    case 32: return prefill_group<D, 32>(a, group, stream);
    case 64: return prefill_group<D, 64>(a, group, stream);
    case 128: return prefill_group<D, 128>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int block_size, int group) {
  const bool b_ok = block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32 ||
                    block_size == 64 || block_size == 128;
  return dtype == PA_BF16 && (head_dim == 64 || head_dim == 128) && b_ok &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  const int group = a.num_q_heads / a.pool.num_kv_heads;
  if (a.pool.head_dim == 128) return prefill_block<128>(a, group, stream);
  if (a.pool.head_dim == 64) return prefill_block<64>(a, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
