// Prefill / chunked-prefill attention over the paged cache for gfx950.
// Citation keys ([HRL], [VIBE], [TSS], ...) name the source pages listed with
// their titles at the top of include/pa.h.
//
// What is computed ([HRL] section 9, prefill runs a prompt's tokens together;
// [TSS] "Next", chunked prefill takes a prompt a piece at a time; [HRL]
// section 8 for the formula): sequence s owns query rows
// query_start_loc[s] .. query_start_loc[s+1]-1, its last n_s positions, so
// row i sits at position p = context_lens[s] - n_s + i and attends causally
// over cached positions 0 .. p, found through the block table.
//
// Unlike decode this is a dense contraction, so it runs on the matrix cores.
// One workgroup of 8 waves takes 256 query rows of one KV head (32 per wave,
// two 16-row groups sharing every K and V operand read): rows are (head of
// the GQA group, token) pairs, head-major, so every row of the workgroup
// reads the same K/V, and each K/V tile is loaded once for 8 waves (one
// workgroup per CU at two waves per SIMD).  K/V tiles of 64 keys go from HBM
// straight into LDS (global_load_lds_dwordx4, no registers on the way),
// double-buffered, and each wave computes flash-attention style on its rows,
// its matrix-core work and its softmax in alternate half-phases, out of step
// with the other wave of its SIMD (the ping-pong at the tile loop):
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16; A = K rows from LDS (ds_read_b128,
//                 XOR-swizzled rows so 16 rows hit 16 different bank groups),
//                 B = Q^T held in registers.  The C layout of S^T gives every
//                 lane one row and four consecutive keys per 16-key sub-tile.
//   P V           v_mfma_f32_16x16x32_bf16 twice, P = P_hi + P_lo; A = those
//                 parts straight from the registers (the contraction's key
//                 order is permuted: slots 0-3 of a lane group are keys
//                 4g..4g+3 of one sub-tile, slots 4-7 the same keys of the
//                 next), V's operand built in the same order from the stored
//                 bf16 with the LDS transpose read ds_read_b64_tr_b16.
// Numerics: V is used exactly as stored (bf16, its whole range).  P in fp32
// is split into P_hi (P with its low 16 bits cleared, a bf16) and P_lo =
// bf16(P - P_hi) (the difference is exact in fp32 and below 2^-7 P), so
// P_hi + P_lo is within 2^-15 P of P; one bf16 part alone (2^-8) could cost
// a row over two keys more than 2e-3.  The row sums come from the matrix
// cores too, as P_hi + P_lo times a block of ones, so they weigh exactly the
// P the output uses.  Online softmax in log2 units
// with the hardware exp2; the scale multiplies inside the exp2 argument (one
// fma) and the running maximum is taken on unscaled scores, raised lazily
// (threshold 8) as in decode.  Workgroups take each (sequence, head) pair's
// heaviest row tiles first and each XCD takes a contiguous run of the work,
// so the workgroups resident on one XCD share K/V in its L2.

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kXcds = 8;  // accelerator complex dies (each with its own L2)
constexpr int kPfWaves = kPrefillWaves;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRG = kPrefillRowGroups;  // 16-row groups per wave
constexpr int kRows = kPrefillRows;      // query rows per workgroup
static_assert(kRows == 16 * kRG * kPfWaves, "16 * kRG rows per wave");
constexpr int kKeys = 64;             // keys per LDS tile
constexpr int kVAhead = 4;            // P.V operand reads in flight ahead of their MFMAs
constexpr float kPfNegInf = -__builtin_inff();
constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfRescaleThreshold = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float pf_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Maximum over the four 16-lane groups of the wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap permutes: with both operands the same value,
// permlane16_swap yields the values of lanes (l & ~16, l | 16) and
// permlane32_swap those of (l & ~32, l | 32) -- VALU only, no LDS round trip.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

// Two waves per SIMD (at most 256 registers each): a workgroup's 8 waves fill
// the four SIMDs of a compute unit twice, so while one wave of a SIMD waits on
// LDS, memory or the barrier, the other can issue.
template <int D, int B, int G>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(const char *__restrict__ pool, int64_t num_blocks, int num_kv_heads, const char *__restrict__ q,
               float *__restrict__ out, const int32_t *__restrict__ query_start_loc,
               const int32_t *__restrict__ context_lens, const int32_t *__restrict__ tables,
               int max_blocks_per_seq, int num_q_heads, int total_tokens, int max_query_len, float scale_log2,
               int num_row_tiles, int num_seqs) {
  using C = PfCfg<D>;
  constexpr int QT = kRows / G;  // tokens per workgroup
  // Separate LDS objects per buffer: the compiler can then see that a
  // direct-to-LDS load into one buffer does not touch the other, and does not
  // make the next tile's reads wait for it.
  __shared__ __attribute__((aligned(16))) char s_k0[C::TILEB];
  __shared__ __attribute__((aligned(16))) char s_k1[C::TILEB];
  __shared__ __attribute__((aligned(16))) char s_v0[C::TILEB];
  __shared__ __attribute__((aligned(16))) char s_v1[C::TILEB];
  char *const s_k[2] = {s_k0, s_k1};
  char *const s_v[2] = {s_v0, s_v1};

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

  auto row_head = [&](int r) __attribute__((always_inline)) { return r / QT; };
  auto row_token = [&](int r) __attribute__((always_inline)) { return qt * QT + r % QT; };
  const int64_t hq0 = (int64_t)h * G;

  if (bad) {
    // NaN rows for the tokens this tile covers, inside the output; the last
    // row tile also takes every token past the grid's tiles (n_s may exceed
    // max_query_len, which sized the grid)
    if (q0 < 0 || n <= 0) return;
    const int64_t lim = min((int64_t)n, (int64_t)total_tokens - q0);  // tokens inside the output
    const int64_t t0 = (int64_t)qt * QT;
    const int64_t t1 = qt == num_row_tiles - 1 ? lim : min(lim, t0 + QT);
    for (int64_t i = tid; i < (t1 - t0) * G * D; i += kPfThreads) {
      const int64_t tok = t0 + i / (G * D);
      const int hd = (int)(i % (G * D));
      out[((q0 + tok) * num_q_heads + hq0) * D + hd] = __builtin_nanf("");
    }
    return;
  }

  // ---- this lane's rows in the S^T layout: row wave*16*kRG + 16*rg + r16; Q^T operands in registers
  // A negative scale is applied as |scale| on -Q (an exact sign flip), so the
  // row maximum is always taken on the largest raw score.  A zero scale is
  // applied as the smallest normal float: every probability stays within
  // 1e-36 of uniform, and masked keys still get exactly zero.
  const uint32_t qsign = scale_log2 < 0.0f ? 0x80008000u : 0u;
  const float cs = scale_log2 == 0.0f ? 1.17549435e-38f : fabsf(scale_log2);
  // Every lane loads (rows past the chunk read its last row, in bounds) and
  // zeroes afterwards, so all the loads are in flight at once rather than
  // each waited inside its own branch.
  int my_pos[kRG];
  bf16x8_t qb[kRG][C::KC];
  u32x4_t qv[kRG][C::KC];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const int r = wave * 16 * kRG + 16 * rg + r16;
    const int t = row_token(r);
    my_pos[rg] = t < n ? ctx - n + t : -1;
    const int tc = min(t, n - 1);
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
      qv[rg][kc] = *reinterpret_cast<const u32x4_t *>(
          q + ((((int64_t)q0 + tc) * num_q_heads + hq0 + row_head(r)) * D + kc * 32 + 8 * grp) * 2);
  }
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const bool live = my_pos[rg] >= 0;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      const u32x4_t v = qv[rg][kc] ^ qsign;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      qb[rg][kc] = as_bf16x8(live ? v : z);
    }
  }

  // ---- tiles: the workgroup needs keys 0 .. kv_end-1; this wave's rows stop at w_pos_max
  const int last_t = min(qt * QT + QT, n) - 1;
  const int kv_end = ctx - n + last_t + 1;
  const int ntiles = (kv_end + kKeys - 1) / kKeys;
  constexpr int WR = 16 * kRG;  // rows per wave
  int w_tmin = QT >= WR ? (wave * WR) % QT : 0;
  int w_tmax = QT >= WR ? w_tmin + WR - 1 : QT - 1;
  w_tmin = qt * QT + w_tmin;
  w_tmax = min(qt * QT + w_tmax, n - 1);
  const int w_pos_min = ctx - n + w_tmin;
  const int w_pos_max = ctx - n + w_tmax;
  const int w_last_tile = w_tmin <= w_tmax ? w_pos_max / kKeys : -1;  // tiles beyond are masked for every row

  // ---- global -> LDS.  A tile spans NBT whole blocks (B <= 64) or a 64-key
  // slice of one block (B > 64).  Block ids are uniform scalar loads,
  // validated; every wave reads all of a tile's ids, so the poison flag is the
  // same in every wave of the workgroup.
  constexpr int NBT = B <= kKeys ? kKeys / B : 1;
  static_assert(B % 4 == 0 && (B <= kKeys ? kKeys % B == 0 : B % kKeys == 0), "block size");
  const int seq_blocks = (ctx + B - 1) / B;
  const char *head_base = pool + (int64_t)h * B * C::ROWB;
  const int64_t kv_half = (int64_t)num_kv_heads * B * C::ROWB;  // K tile to V tile of one block
  const int32_t *table_row = tables + (int64_t)s * max_blocks_per_seq;
  const int num_blocks32 = (int)num_blocks;  // at most INT32_MAX (checked by the host)
  bool poisoned = false;

  // K and V go straight from global memory into LDS (global_load_lds_dwordx4:
  // each instruction writes 1 KiB, lane l's 16 bytes at l * 16).  Waves 4-7
  // (the loaders) issue every load of a tile: instruction i of loader lw fills
  // tile rows RPI*(4i+lw) .. +RPI-1; lane l writes slot l % NCH16 of row
  // RPI*(4i+lw) + l / NCH16, and loads the chunk its tile's swizzle puts in
  // that slot (K: 16-byte XOR swizzle, V: v_lds8).  The loaders start a tile
  // in their vector half, so the matrix-core waves 0-3 are not held up behind
  // a CU's worth of loads queueing for the texture path at the tile's start
  // (1-2.5 % faster than every wave loading its own rows).  Keys past the context
  // are loaded from wherever their rows fall (the last block's tail, or block
  // 0 past the table's used entries): their scores are masked before any use
  // and zero_v_tail overwrites their values with zeros (a zero probability
  // times a NaN would still be NaN), so whatever those rows hold never
  // reaches the output.
  constexpr int RPI = 1024 / C::ROWB;  // key rows per instruction
  const int dl_row = lane / C::NCH16, dl_slot = lane % C::NCH16;
  // The chunk that lands in LDS slot `slot` of tile row `row`: the inverse of
  // k_lds (16-byte XOR by row % NCH16) or of v_lds8 (which moves 16-byte
  // chunk c to slot c ^ 2 (row % (NCH8 / 4))).
  auto src_chunk = [&](int row, int slot, bool is_v) __attribute__((always_inline)) {
    return is_v ? slot ^ (2 * (row % (C::NCH8 / 4))) : slot ^ (row % C::NCH16);
  };
  // this lane's byte offset inside an instruction's RPI rows
  constexpr int kLoaders = kPfWaves / 2;               // waves 4-7
  constexpr int LPW = C::LOADS * kPfWaves / kLoaders;  // load instructions per loader per tile
  const int lw = wave % kLoaders;
  uint32_t lane_off_k[LPW], lane_off_v[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = RPI * (kLoaders * i + lw) + dl_row;
    lane_off_k[i] = dl_row * C::ROWB + (src_chunk(row, dl_slot, false) << 4);
    lane_off_v[i] = dl_row * C::ROWB + (src_chunk(row, dl_slot, true) << 4);
  }
  // block ids of tile t (scalar loads; fetched a tile ahead of their use)
  auto fetch_ids = [&](int t, int (&ids)[NBT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      const int jb = B <= kKeys ? t * NBT + i : t / (B / kKeys);
      ids[i] = __builtin_amdgcn_readfirstlane(jb < seq_blocks ? table_row[jb] : 0);
    }
  };
  // Every wave checks the tile's block ids (an invalid id poisons its rows);
  // only a loader (`issue`) starts the loads.
  auto load_lds = [&](int t, const int (&ids)[NBT], int64_t part_off, bool is_v, char *buf, bool issue)
                      __attribute__((always_inline)) {
    int blk[NBT];
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      int b = ids[i];
      if (b < 0 || b >= num_blocks32) {
        poisoned = true;
        b = 0;
      }
      blk[i] = b;
    }
    if (!issue) return;
    if constexpr (RPI <= B) {
      // Every instruction's RPI rows lie in one block, so its address is a
      // uniform base (scalar registers) plus this lane's fixed offset.  Rows
      // past the context read whatever the block holds there: their scores
      // are masked, and zero_v_tail zeroes their values.
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int row0 = RPI * (kLoaders * i + lw);  // uniform
        int b, rib0;
        if constexpr (B > kKeys) {
          b = blk[0];
          rib0 = (t % (B / kKeys)) * kKeys + row0;
        } else {
          const int slot = row0 / B;
          b = blk[0];
#pragma unroll
          for (int k = 1; k < NBT; ++k) b = slot == k ? blk[k] : b;
          rib0 = row0 % B;
        }
        const uint64_t base = (uint64_t)(head_base + (int64_t)b * 2 * kv_half + part_off + (int64_t)rib0 * C::ROWB);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
        const char *sbase = reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
        const uint32_t off = is_v ? lane_off_v[i] : lane_off_k[i];
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(sbase + off),
                                         (__attribute__((address_space(3))) void *)(buf + (kLoaders * i + lw) * 1024),
                                         16, 0, 0);
      }
    } else {
      // an instruction spans two blocks (64-dim rows, 4-token blocks): per-lane
      // addresses; rows past the context read the last real row
      const int last_row = ctx - 1 - t * kKeys;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int row = RPI * (kLoaders * i + lw) + dl_row;
        const int chunk = src_chunk(row, dl_slot, is_v);
        const int src_row = min(row, last_row);
        const int slot = src_row / B;
        int b = blk[0];
#pragma unroll
        for (int k = 1; k < NBT; ++k) b = slot == k ? blk[k] : b;
        const char *src = head_base + (int64_t)b * 2 * kv_half + part_off + (src_row % B) * C::ROWB + chunk * 16;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(buf + (kLoaders * i + lw) * 1024),
                                         16, 0, 0);
      }
    }
  };
  // Rows of V tile t past the context hold whatever their source rows held
  // (padding may be NaN); each loader lane overwrites the 16 bytes its own
  // loads put there with zeros.  Only the tile where the context ends has such
  // rows (uniform test); a loader calls it after its loads of the tile have
  // landed.
  auto zero_v_tail = [&](char *buf, int t) __attribute__((always_inline)) {
    const int vrows = ctx - t * kKeys;  // rows of the tile inside the context (uniform)
    if (vrows < kKeys) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int row = RPI * (kLoaders * i + lw) + dl_row;
        if (row >= vrows)
          *reinterpret_cast<u32x4_t *>(&buf[(kLoaders * i + lw) * 1024 + lane * 16]) = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  // The LDS writes of this wave's loads are done (a barrier after this publishes them).
  auto wait_lds_loads = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // ---- per-row state: running max (log2 units) of this lane's S row, and
  // the output tiles O[4*grp + jj][16*nt + r16] with their row sums
  float m[kRG];
  f32x4_t o[kRG][C::NT], osum[kRG];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    m[rg] = kPfNegInf;
    osum[rg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) o[rg][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const bf16x8_t ones = as_bf16x8(u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});  // bf16 1.0

  // Per-lane LDS byte offsets of the operand reads; sub-tile, key-step and
  // buffer offsets fold into the instructions' immediate offsets.
  int k_base[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) k_base[kc] = k_lds<D>(r16, kc * 4 + grp);
  int v_base[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) v_base[nt] = v_lds8<D>(4 * grp + r16 / 4, 4 * nt + (r16 & 3));

  // S^T of tile t: sacc[rg][kt] = K[16kt .. +16] Q_rg^T (raw, unscaled); each K operand serves every row group.
  // The 32-dim steps run outermost, so the MFMAs that accumulate into one
  // score tile are 8 apart (measured 0.5 % faster than tile by tile).
  auto qk = [&](const char *kt_lds, f32x4_t (&sacc)[kRG][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) sacc[rg][kt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // The K operands of step kc+1 are read while step kc's MFMAs run (order
    // pinned: step 0's reads, then per step the next step's 4 reads and this
    // step's 4 kRG MFMAs).
    u32x4_t ka[2][4];
    auto rdk = [&](int kc, u32x4_t (&a)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) a[kt] = *reinterpret_cast<const u32x4_t *>(&kt_lds[k_base[kc] + 16 * kt * C::ROWB]);
    };
    rdk(0, ka[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // step 0's reads first
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      if (kc + 1 < C::KC) rdk(kc + 1, ka[(kc + 1) & 1]);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg)
          sacc[rg][kt] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[kc & 1][kt]), qb[rg][kc], sacc[rg][kt], 0, 0, 0);
      if (kc + 1 < C::KC) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * kRG, 0);                 // MFMAs
    }
  };
  // Softmax, first half: mask tile t's raw scores in place (diagonal tiles
  // only), take each row's maximum and raise the running maximum, rescaling
  // O and the row sums when it moves by more than the threshold (rare).
  auto row_max = [&](int t, f32x4_t (&sacc)[kRG][4]) __attribute__((always_inline)) {
    const int k0 = t * kKeys;
    float mnew[kRG];
    bool upd[kRG];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      if (k0 + kKeys - 1 > w_pos_min) {  // some key of the tile lies after some row
        const int lim = my_pos[rg] - k0 - 4 * grp;  // key k0 + 4*grp + c is visible iff c <= lim
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (16 * kt + jj > lim) sacc[rg][kt][jj] = kPfNegInf;
      }
      // NaN-propagating maximum: no operand quieting, and pairs fuse into v_maximum3
      float mx = __builtin_elementwise_maximum(sacc[rg][0][0], sacc[rg][0][1]);
      mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(sacc[rg][0][2], sacc[rg][0][3]));
#pragma unroll
      for (int kt = 1; kt < 4; ++kt) {
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(sacc[rg][kt][0], sacc[rg][kt][1]));
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(sacc[rg][kt][2], sacc[rg][kt][3]));
      }
      const float mt = group_max(mx) * cs;  // this tile's row maximum, log2 units (-inf if fully masked)
      mnew[rg] = __builtin_elementwise_maximum(m[rg], mt);
      upd[rg] = mnew[rg] > m[rg] + kPfRescaleThreshold;
    }
    // one wave-uniform branch for all row groups (rare)
    bool any_upd = false;
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) any_upd = any_upd || upd[rg];
    if (__builtin_amdgcn_ballot_w64(any_upd) != 0) {
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) {
        const float alpha = upd[rg] ? pf_exp2(m[rg] - mnew[rg]) : 1.0f;
        if (upd[rg]) m[rg] = mnew[rg];
        // O rows are 4*grp + jj: fetch those rows' factors
        float ar[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ar[jj] = __shfl(alpha, 4 * grp + jj);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          osum[rg][jj] *= ar[jj];
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) o[rg][nt][jj] *= ar[jj];
        }
      }
    }
  };
  // Softmax, second half: P = exp2(cs * s - m) in fp32 (the permuted key
  // order), split into bf16 parts P_hi + P_lo (P_hi the truncation, P_lo the
  // rounded remainder).  Their row sums P 1 are taken with P.V, on the matrix
  // cores, so the vector half ends with its last vector instruction.
  auto make_p = [&](const f32x4_t (&sacc)[kRG][4], bf16x8_t (&ph)[kRG][2], bf16x8_t (&pl)[kRG][2])
                    __attribute__((always_inline)) {
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      const float nms = m[rg] == kPfNegInf ? 0.0f : -m[rg];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t hi, lo;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int jp = 0; jp < 2; ++jp) {
            // slots 4 half + 2 jp, +1: keys jj = 2 jp, 2 jp + 1 of sub-tile 2 ks + half
            const float p0 = pf_exp2(__builtin_fmaf(sacc[rg][2 * ks + half][2 * jp], cs, nms));
            const float p1 = pf_exp2(__builtin_fmaf(sacc[rg][2 * ks + half][2 * jp + 1], cs, nms));
            const uint32_t b0 = __float_as_uint(p0) & 0xFFFF0000u, b1 = __float_as_uint(p1) & 0xFFFF0000u;
            hi[2 * half + jp] = b1 | (b0 >> 16);
            const bf16x2_t r = {(__bf16)(p0 - __uint_as_float(b0)), (__bf16)(p1 - __uint_as_float(b1))};
            lo[2 * half + jp] = __builtin_bit_cast(uint32_t, r);
          }
        ph[rg][ks] = as_bf16x8(hi);
        pl[rg][ks] = as_bf16x8(lo);
      }
    }
  };
  // O += P V and the row sums += P 1: P_hi then P_lo against each operand.
  auto pv = [&](const bf16x8_t (&ph)[kRG][2], const bf16x8_t (&pl)[kRG][2], const char *vt_lds)
                __attribute__((always_inline)) {
    // V operands are read kVAhead steps before the MFMAs that use them, and
    // the schedule is pinned to (4 reads of later steps, 8 MFMAs of this step
    // pair) so the reads' latency overlaps the matrix work (left to itself the
    // scheduler waits on each step's reads just before its MFMAs).
    constexpr int NS = 2 * C::NT;  // (nt, ks) steps, ks outermost: consecutive steps feed different output tiles
    bf16x8_t vq[kVAhead];
    auto rdv = [&](int st) __attribute__((always_inline)) {
      const int nt = st % C::NT, ks = st / C::NT;
      const i16x4_t lo4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vt_lds + v_base[nt] + 32 * ks * C::ROWB));
      const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t *)(vt_lds + v_base[nt] + (32 * ks + 16) * C::ROWB));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int st = 0; st < kVAhead; ++st) vq[st] = rdv(st);
    // the row sums P 1 (they need no V operand, so they run while the first reads land)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) {
        osum[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[rg][ks], ones, osum[rg], 0, 0, 0);
        osum[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[rg][ks], ones, osum[rg], 0, 0, 0);
      }
    // Steps go in pairs (output tiles nt, nt+1 of one key half): the P_hi
    // and P_lo products into one tile are 2 kRG MFMAs apart.
#pragma unroll
    for (int st = 0; st < NS; st += 2) {
      const int nt = st % C::NT, ks = st / C::NT;
      const bf16x8_t vb0 = vq[st % kVAhead], vb1 = vq[(st + 1) % kVAhead];
      if (st + kVAhead < NS) vq[st % kVAhead] = rdv(st + kVAhead);
      if (st + 1 + kVAhead < NS) vq[(st + 1) % kVAhead] = rdv(st + 1 + kVAhead);
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg)
        o[rg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[rg][ks], vb0, o[rg][nt], 0, 0, 0);
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg)
        o[rg][nt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[rg][ks], vb1, o[rg][nt + 1], 0, 0, 0);
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg)
        o[rg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[rg][ks], vb0, o[rg][nt], 0, 0, 0);
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg)
        o[rg][nt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[rg][ks], vb1, o[rg][nt + 1], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);      // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * kRG, 0);  // MFMAs
    }
  };

  // ---- ping-pong.  Waves w and w + 4 share a SIMD (a workgroup's waves go
  // to its CU's four SIMDs in turn).  Each wave alternates a matrix-core half
  // (scores of tile t, P.V and row sums of tile t-1) and a vector half (row
  // maxima and probabilities of tile t); waves 4-7 run one half-phase behind
  // waves 0-3, so while one wave of a SIMD feeds the matrix cores the other
  // runs its softmax, instead of both meeting in the same phase.  The
  // matrix-core halves run at raised wave priority, so the arbiter gives an
  // MFMA the issue slot before the other wave's vector instruction (2 %
  // measured).  Every half-phase ends in a barrier.  Wave group 0 runs M(u)
  // in half-phase 2u and V(u) in 2u+1; group 1 (the loaders) runs V(u-1) in
  // half-phase 2u, starting it with the loads of K(u+1) (buffer (u+1) % 2) and
  // V(u) (buffer u % 2), and M(u) in 2u+1.  The barrier that ends half-phase
  // 2u already waits for those loads (its release covers direct-to-LDS
  // writes), so they land before the loaders' M(u) reads LDS; a bare barrier
  // there, letting them land during M(u), measured 0-6 % slower, and a third
  // buffer pair (loads a tile earlier) gained nothing.  K(u) and V(u-1) are
  // read in M(u) only, so their buffers are free after half-phase 2u+1.
  const int n_compute = min(ntiles, w_last_tile + 1);  // tiles with work for this wave (uniform)
  const int grp1 = wave >= kPfWaves / 2;
  int ids_k[NBT], ids_v[NBT];
  fetch_ids(0, ids_v);
  load_lds(0, ids_v, 0, false, s_k[0], grp1);
  if (ntiles > 1) fetch_ids(1, ids_k);
  wait_lds_loads();
  __syncthreads();
  f32x4_t sc[kRG][4];
  bf16x8_t ph[kRG][2], pl[kRG][2];
  // M(u): scores of tile u, P.V and row sums of tile u-1 (matrix cores)
  auto m_half = [&](int u, auto ub) __attribute__((always_inline)) {
    constexpr int UB = decltype(ub)::value;  // u % 2
    __builtin_amdgcn_s_setprio(1);
    if (u < n_compute) qk(s_k[UB], sc);
    if (u >= 1 && u - 1 < n_compute) pv(ph, pl, s_v[1 - UB]);
    __builtin_amdgcn_s_setprio(0);
  };
  // V(t): row maxima and probabilities of tile t (vector ALU)
  auto v_half = [&](int t) __attribute__((always_inline)) {
    if (t >= 0 && t < n_compute) {
      row_max(t, sc);
      make_p(sc, ph, pl);
    }
  };
  // half-phases 2u and 2u+1 for wave group WG
  auto tile2 = [&](int u, auto ub, auto g) __attribute__((always_inline)) {
    constexpr int UB = decltype(ub)::value;
    constexpr int WG = decltype(g)::value;
    if (u + 1 < ntiles) load_lds(u + 1, ids_k, 0, false, s_k[1 - UB], WG == 1);
    if (u < ntiles) load_lds(u, ids_v, kv_half, true, s_v[UB], WG == 1);
    // The next tiles' block ids (scalar loads) are fetched at the head of the
    // vector half, which has no LDS waits for them to hold up, so they have
    // landed by the barrier that ends the tile (its release waits for every
    // scalar load in flight).
    auto next_ids = [&]() __attribute__((always_inline)) {
      if (u + 2 < ntiles) fetch_ids(u + 2, ids_k);
      if (u + 1 < ntiles) fetch_ids(u + 1, ids_v);
    };
    if constexpr (WG == 0) {
      m_half(u, ub);
    } else {
      next_ids();
      v_half(u - 1);
    }
    __syncthreads();
    if constexpr (WG == 0) {
      next_ids();
      v_half(u);
    } else {
      m_half(u, ub);
    }
    wait_lds_loads();
    if (WG == 1 && u < ntiles) zero_v_tail(s_v[UB], u);
    __syncthreads();
  };
  using b0 = std::integral_constant<int, 0>;
  using b1 = std::integral_constant<int, 1>;
  auto run = [&](auto g) __attribute__((always_inline)) {
    int u = 0;
    for (; u + 1 <= ntiles; u += 2) {
      tile2(u, b0{}, g);
      tile2(u + 1, b1{}, g);
    }
    if (u <= ntiles) tile2(u, b0{}, g);
  };
  if (grp1)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});
  const bool seq_poisoned = poisoned;

  // ---- normalise and store: lane holds rows 4*grp + jj of each group, columns 16*nt + r16
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = wave * 16 * kRG + 16 * rg + 4 * grp + jj;
      const int tok = row_token(r);
      if (tok >= n) continue;
      const float inv = osum[rg][jj] > 0.0f ? 1.0f / osum[rg][jj] : 0.0f;
      float *dst = out + (((int64_t)q0 + tok) * num_q_heads + hq0 + row_head(r)) * D + r16;
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
        dst[16 * nt] = seq_poisoned ? __builtin_nanf("") : o[rg][nt][jj] * inv;
    }
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
