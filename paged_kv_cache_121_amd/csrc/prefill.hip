// Prefill / chunked-prefill attention over the paged cache for gfx950.
//
// What is computed ([HRL] section 9, prefill runs a prompt's tokens together;
// [TSS] "Next", chunked prefill takes a prompt a piece at a time; [HRL]
// section 8 for the formula): sequence s owns query rows
// query_start_loc[s] .. query_start_loc[s+1]-1, its last n_s positions, so
// row i sits at position p = context_lens[s] - n_s + i and attends causally
// over cached positions 0 .. p, found through the block table.
//
// Unlike decode this is a dense contraction, so it runs on the matrix cores.
// One workgroup of 4 waves takes 64 query rows of one KV head (16 per wave):
// rows are (head of the GQA group, token) pairs, head-major, so every row of
// the workgroup reads the same K/V.  K/V tiles of 64 keys are gathered
// through the block table into LDS, and each wave computes flash-attention
// style on its 16 rows:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16; A = K rows from LDS (ds_read_b128,
//                 XOR-swizzled rows so 16 rows hit 16 different bank groups),
//                 B = Q^T held in registers.  The C layout of S^T gives every
//                 lane one row and four consecutive keys per 16-key sub-tile.
//   P V           v_mfma_f32_16x16x32_f16; A = P straight from those registers
//                 (the contraction's key order is permuted: slots 0-3 of a
//                 lane group are keys 4g..4g+3 of one sub-tile, slots 4-7 the
//                 same keys of the next), V's operand built in the same order
//                 with the LDS transpose read ds_read_b64_tr_b16.
// Numerics: P is rounded to fp16 (relative 2^-11; bf16's 2^-9 could cost a
// row over two keys more than 2e-3) and V is stored in LDS as fp16, an exact
// conversion of bf16 for |v| < 65504 (larger values saturate).  The row sums
// come from the matrix cores too, as P times a block of ones, so they weigh
// exactly the rounded P the output uses.  Online softmax in log2 units with
// the hardware exp2; the scale multiplies inside the exp2 argument (one fma)
// and the running maximum is taken on unscaled scores, raised lazily
// (threshold 8) as in decode.
// Pipeline: K runs two tiles ahead of the softmax and V one, so while a wave
// turns tile t's scores into probabilities the matrix cores already compute
// tile t+1's scores; one barrier per tile orders the LDS reuse.  Keys past
// the context are written to LDS as zeros (never read from HBM), so padding
// slots cannot leak NaN through 0 * V.  Workgroups take the heaviest row
// tiles first (causal rows late in a prompt see the most keys).

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kXcds = 8;  // accelerator complex dies (each with its own L2)
constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRows = kPrefillRows;  // query rows per workgroup (16 per wave)
static_assert(kRows == 16 * kPfWaves, "16 rows per wave");
constexpr int kKeys = 64;             // keys per LDS tile
constexpr float kPfNegInf = -__builtin_inff();
constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfRescaleThreshold = 8.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float pf_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Max / min over the four 16-lane groups of the wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap permutes: with both operands the same value,
// permlane16_swap yields the values of lanes (l & ~16, l | 16) and
// permlane32_swap those of (l & ~32, l | 32) -- VALU only, no LDS round trip.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_min(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D>
struct PfCfg {
  static constexpr int ROWB = D * 2;          // bytes per key row (bf16)
  static constexpr int NCH16 = D / 8;         // 16-byte chunks per row
  static constexpr int NCH8 = D / 4;          // 8-byte chunks per row
  static constexpr int TILEB = kKeys * ROWB;  // bytes of one K or V tile in LDS
  static constexpr int KC = D / 32;           // 32-dim steps of QK
  static constexpr int NT = D / 16;           // 16-dim output tiles of PV
  static constexpr int LOADS = kKeys * NCH16 / kPfThreads;  // 16-byte loads per thread per K (or V) tile
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
               int max_blocks_per_seq, int num_q_heads, int total_tokens, int max_query_len, float scale_log2,
               int num_row_tiles, int num_seqs) {
  using C = PfCfg<D>;
  constexpr int QT = kRows / G;  // tokens per workgroup
  __shared__ __attribute__((aligned(16))) char s_k[2][C::TILEB];
  __shared__ __attribute__((aligned(16))) char s_v[2][C::TILEB];
  __shared__ int s_poison;

  // Work order: (sequence, KV head) pairs one after another, each pair's row
  // tiles heaviest first (causal rows late in a prompt see the most keys).
  // Workgroups are handed to the 8 XCDs in turn, so workgroup L runs on XCD
  // L % 8; XCD x takes the x-th eighth of the work list in order, and the
  // workgroups resident on one XCD at a time walk the same pair's K/V together
  // through its own L2.
  const int total = num_row_tiles * num_kv_heads * num_seqs;
  const int per_xcd = (int)gridDim.x / kXcds;
  const int w = ((int)blockIdx.x % kXcds) * per_xcd + (int)blockIdx.x / kXcds;
  if (w >= total) return;
  const int pair = w / num_row_tiles;
  const int qt = num_row_tiles - 1 - (w - pair * num_row_tiles);
  const int s = pair / num_kv_heads, h = pair - s * num_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, grp = lane >> 4;

  const int q0 = query_start_loc[s];
  const int n = query_start_loc[s + 1] - q0;
  const int ctx = context_lens[s];
  const bool bad = n < 0 || n > ctx || n > max_query_len || ctx > max_blocks_per_seq * B || q0 < 0 ||
                   (int64_t)q0 + n > total_tokens;
  if (!bad && qt * QT >= n) return;  // no rows of this sequence in this tile

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

  // ---- this lane's row in the S^T layout: row wave*16 + r16; Q^T operand in registers
  // A negative scale is applied as |scale| on -Q (an exact sign flip), so the
  // row maximum is always taken on the largest raw score.  A zero scale is
  // applied as the smallest normal float: every probability stays within
  // 1e-36 of uniform, and masked keys still get exactly zero.
  const uint32_t qsign = scale_log2 < 0.0f ? 0x80008000u : 0u;
  const float cs = scale_log2 == 0.0f ? 1.17549435e-38f : fabsf(scale_log2);
  int my_pos;
  bf16x8_t qb[C::KC];
  {
    const int r = wave * 16 + r16;
    const int t = row_token(r);
    my_pos = t < n ? ctx - n + t : -1;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (t < n) {
        const char *p = q + ((((int64_t)q0 + t) * num_q_heads + hq0 + row_head(r)) * D + kc * 32 + 8 * grp) * 2;
        v = *reinterpret_cast<const u32x4_t *>(p);
        v ^= qsign;
      }
      qb[kc] = as_bf16x8(v);
    }
  }

  // ---- tiles: the workgroup needs keys 0 .. kv_end-1; this wave's rows stop at w_pos_max
  const int last_t = min(qt * QT + QT, n) - 1;
  const int kv_end = ctx - n + last_t + 1;
  const int ntiles = (kv_end + kKeys - 1) / kKeys;
  int w_tmin = QT >= 16 ? (wave * 16) % QT : 0;
  int w_tmax = QT >= 16 ? w_tmin + 15 : QT - 1;
  w_tmin = qt * QT + w_tmin;
  w_tmax = min(qt * QT + w_tmax, n - 1);
  const int w_pos_min = ctx - n + w_tmin;
  const int w_pos_max = ctx - n + w_tmax;
  const int w_last_tile = w_tmin <= w_tmax ? w_pos_max / kKeys : -1;  // tiles beyond are masked for every row

  if (tid == 0) s_poison = 0;

  // ---- global -> registers -> LDS.  A tile spans NBT whole blocks (B <= 64)
  // or a 64-key slice of one block (B > 64).  Block ids are uniform scalar
  // loads, validated; every lane issues its loads unconditionally at
  // in-bounds addresses.  When one load instruction's KPL keys sit in one
  // block (KPL <= B) its block address is uniform, so only the lane's row
  // offset is per lane.  Keys past the context (last tile only) become zeros.
  constexpr int NBT = B <= kKeys ? kKeys / B : 1;
  constexpr int KPL = kPfThreads / C::NCH16;  // keys per load instruction
  static_assert(B % 4 == 0 && (B <= kKeys ? kKeys % B == 0 : B % kKeys == 0), "block size");
  const int lkey = tid / C::NCH16, lch = tid % C::NCH16;
  const int seq_blocks = (ctx + B - 1) / B;
  const char *head_base = pool + (int64_t)h * B * C::ROWB;
  const int64_t kv_half = (int64_t)num_kv_heads * B * C::ROWB;  // K tile to V tile of one block
  const int32_t *table_row = tables + (int64_t)s * max_blocks_per_seq;
  bool poisoned = false;
  u32x4_t kr[C::LOADS], vr[C::LOADS];

  auto load_part = [&](int t, int64_t part_off, u32x4_t (&dst)[C::LOADS]) {
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
    const char *ptr[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int key = i * KPL + lkey;
      int b, row;
      if constexpr (B > kKeys) {
        b = blk[0];
        row = (t % (B / kKeys)) * kKeys + key;
      } else if constexpr (KPL <= B) {
        b = blk[(i * KPL) / B];
        row = (i * KPL) % B + lkey;
      } else {
        const int slot = key / B;
        b = blk[0];
#pragma unroll
        for (int k = 1; k < NBT; ++k) b = slot == k ? blk[k] : b;
        row = key % B;
      }
      ptr[i] = head_base + (int64_t)b * 2 * kv_half + part_off + row * C::ROWB + lch * 16;
    }
    if ((t + 1) * kKeys <= ctx) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) dst[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(ptr[i]));
    } else {
      const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(ptr[i]));
        dst[i] = t * kKeys + i * KPL + lkey < ctx ? x : zero;
      }
    }
  };
  auto store_k = [&](char *buf) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      *reinterpret_cast<u32x4_t *>(&buf[k_lds<D>(i * KPL + lkey, lch)]) = kr[i];
  };
  auto store_v = [&](char *buf) {  // as fp16
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      u32x4_t vh;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        vh[w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(vr[i][w] << 16),
                                                                        __uint_as_float(vr[i][w] & 0xffff0000u)));
      *reinterpret_cast<u32x4_t *>(&buf[v_lds8<D>(i * KPL + lkey, 2 * lch)]) = vh;
    }
  };

  // ---- per-row state: running max (log2 units) of this lane's S row, and
  // the output tiles O[4*grp + jj][16*nt + r16] with their row sums
  float m = kPfNegInf;
  f32x4_t o[C::NT], osum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) o[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  f16x8_t ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (_Float16)1.0f;

  // Per-lane LDS byte offsets of the operand reads; sub-tile, key-step and
  // buffer offsets fold into the instructions' immediate offsets.
  int k_base[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) k_base[kc] = k_lds<D>(r16, kc * 4 + grp);
  int v_base[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) v_base[nt] = v_lds8<D>(4 * grp + r16 / 4, 4 * nt + (r16 & 3));

  // S^T of tile t: sacc[kt] = K[16kt .. +16] Q^T (raw, unscaled)
  auto qk = [&](const char *kt_lds, f32x4_t (&sacc)[4]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(&kt_lds[k_base[kc] + 16 * kt * C::ROWB]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qb[kc], sacc[kt], 0, 0, 0);
      }
    }
  };
  // Softmax, first half: mask tile t's raw scores in place (diagonal tiles
  // only), take each row's maximum and raise the running maximum, rescaling
  // O and the row sums when it moves by more than the threshold (rare).
  auto row_max = [&](int t, f32x4_t (&sacc)[4]) {
    const int k0 = t * kKeys;
    if (k0 + kKeys - 1 > w_pos_min) {  // some key of the tile lies after some row
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (k0 + 16 * kt + 4 * grp + jj > my_pos) sacc[kt][jj] = kPfNegInf;
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(sacc[2][0], sacc[2][1]), fmaxf(sacc[2][2], sacc[2][3])),
                         fmaxf(fmaxf(sacc[3][0], sacc[3][1]), fmaxf(sacc[3][2], sacc[3][3]))));
    const float mt = group_max(mx) * cs;  // this tile's row maximum, log2 units (-inf if fully masked)
    const float mn = fmaxf(m, mt);
    const bool upd = mn > m + kPfRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
      const float alpha = upd ? pf_exp2(m - mn) : 1.0f;
      if (upd) m = mn;
      // O rows are 4*grp + jj: fetch those rows' factors
      float ar[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ar[jj] = __shfl(alpha, 4 * grp + jj);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        osum[jj] *= ar[jj];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) o[nt][jj] *= ar[jj];
      }
    }
  };
  // Softmax, second half, and O += P V(t): P = exp2(cs * s - m) in fp16 (the
  // permuted key order), row sums P 1 and the V products on the matrix cores.
  auto exp_pv = [&](const f32x4_t (&sacc)[4], const char *vt_lds) {
    const float nms = m == kPfNegInf ? 0.0f : -m;
    f16x8_t ph[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          ph[ks][4 * half + jj] = (_Float16)pf_exp2(__builtin_fmaf(sacc[2 * ks + half][jj], cs, nms));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) osum = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[ks], ones, osum, 0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i16x4_t lo4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vt_lds + v_base[nt] + 32 * ks * C::ROWB));
        const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t *)(vt_lds + v_base[nt] + (32 * ks + 16) * C::ROWB));
        const f16x8_t vb = __builtin_bit_cast(f16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[ks], vb, o[nt], 0, 0, 0);
      }
    }
  };

  // ---- pipeline.  Prologue: K(0), V(0), K(1) in LDS; V(1), K(2) in flight; S(0) computed.
  // Iteration t: S(t+1) from K(t+1) || softmax(t), PV(t); store K(t+2) over K(t)'s
  // buffer and V(t+1) over V(t-1)'s; barrier; load V(t+2), K(t+3).
  load_part(0, 0, kr);
  load_part(0, kv_half, vr);
  store_k(s_k[0]);
  store_v(s_v[0]);
  if (ntiles > 1) {
    load_part(1, 0, kr);
    store_k(s_k[1]);
  }
  __syncthreads();
  if (ntiles > 1) load_part(1, kv_half, vr);
  if (ntiles > 2) load_part(2, 0, kr);
  f32x4_t sA[4], sB[4];
  if (w_last_tile >= 0) qk(s_k[0], sA);

  auto step = [&](int t, auto bt, f32x4_t (&s_cur)[4], f32x4_t (&s_next)[4]) {
    constexpr int b = decltype(bt)::value;
    if (t <= w_last_tile) {
      row_max(t, s_cur);
      // one branch-free stretch: tile t+1's scores (from a stale buffer, unused,
      // past the last tile) beside tile t's probabilities and V products
      qk(s_k[1 - b], s_next);
      exp_pv(s_cur, s_v[b]);
    }
    if (t + 2 < ntiles) store_k(s_k[b]);
    if (t + 1 < ntiles) store_v(s_v[1 - b]);
    __syncthreads();
    if (t + 2 < ntiles) load_part(t + 2, kv_half, vr);
    if (t + 3 < ntiles) load_part(t + 3, 0, kr);
  };
  using buf0 = std::integral_constant<int, 0>;
  using buf1 = std::integral_constant<int, 1>;
  for (int t = 0; t < ntiles; t += 2) {
    step(t, buf0{}, sA, sB);
    if (t + 1 >= ntiles) break;
    step(t + 1, buf1{}, sB, sA);
  }
  if (poisoned) s_poison = 1;
  __syncthreads();
  const bool seq_poisoned = s_poison != 0;

  // ---- normalise and store: lane holds rows 4*grp + jj, columns 16*nt + r16
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int r = wave * 16 + 4 * grp + jj;
    const int tok = row_token(r);
    if (tok >= n) continue;
    const float inv = osum[jj] > 0.0f ? 1.0f / osum[jj] : 0.0f;
    float *dst = out + (((int64_t)q0 + tok) * num_q_heads + hq0 + row_head(r)) * D + r16;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) dst[16 * nt] = seq_poisoned ? __builtin_nanf("") : o[nt][jj] * inv;
  }
}

template <int D, int B, int G>
hipError_t prefill_one(const PrefillArgs &a, hipStream_t stream) {
  constexpr int QT = kRows / G;
  const int row_tiles = (a.max_query_len + QT - 1) / QT;
  const int64_t total = (int64_t)row_tiles * a.pool.num_kv_heads * a.num_seqs;
  const dim3 grid((unsigned)((total + kXcds - 1) / kXcds * kXcds));
  hipLaunchKernelGGL((prefill_kernel<D, B, G>), grid, dim3(kPfThreads), 0, stream,
                     static_cast<const char *>(a.pool.base), a.pool.num_blocks, a.pool.num_kv_heads,
                     static_cast<const char *>(a.q), a.out, a.query_start_loc, a.context_lens, a.block_tables,
                     a.max_blocks_per_seq, a.num_q_heads, a.total_tokens, a.max_query_len, a.scale * kPfLog2e,
                     row_tiles, a.num_seqs);
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
