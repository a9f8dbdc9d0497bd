// Paged decode attention for gfx950 (CDNA4, wave64).
// Citation keys ([HRL], [VIBE], [TSS], ...) name the source pages listed with
// their titles at the top of include/pa.h.
//
// What is computed ([HRL] section 8; [VIBE] vLLM procedure step 5): for every
// sequence s and query head hq, out = softmax(scale * q K^T) V over the
// sequence's context_lens[s] cached tokens, where token t of the sequence
// lives in physical block table[s][t / B] at offset t % B.
//
// Work decomposition
//   one workgroup per (partition p, KV head h, sequence s), in a
//   one-dimensional grid ordered so each XCD gets an equal share of the
//   (sequence, head) pairs.  A workgroup of kWaves (4 or 8, chosen per launch)
//   wavefronts serves all G = Hq / Hkv query heads of KV head h, so each K/V
//   byte is read from HBM once per step.  The workgroup owns the blocks
//   [p * part, (p + 1) * part) of the sequence; wave w takes the workgroup's
//   blocks w, w + kWaves, ...
//
// Lane layout (16 lanes per token)
//   A (block, head) K or V tile is [B][D] contiguous, so a token's row is
//   D * elem bytes = 16 lanes x VEC bytes.  Per load step a wavefront reads
//   64 x VEC contiguous bytes = 4 tokens; lane l holds dims
//   (l % 16) * EPL ... of token 4 * step + l / 16.  The four 16-lane rows of
//   the wave are four independent online-softmax streams (each sees every
//   fourth token) that are merged once at the end of the partition.
//
// QK: each lane forms partial dots over its EPL dims for all G heads (bf16:
//   v_dot2 on packed pairs, exact products with fp32 accumulation), then a
//   DPP reduce-scatter inside each 16-lane row leaves lane l holding the full
//   scores of heads sigma(l) ... sigma(l) + HPL - 1.  The query registers are
//   loaded in a lane-dependent head order (register r holds head r ^ sigma(l))
//   so every exchange step is uniform across lanes: no selects.
//   Groups of 8 over bf16 pools take their scores from the matrix cores
//   instead, with their own lane layout (described at the kernel, "MQ").
// Softmax: scores are kept in log2 units (scale * log2 e folded in) and
//   exponentiated with the hardware exp2.  The running max is raised only
//   when a score exceeds it by more than kRescaleThreshold, so the rescale
//   of the accumulators is rare; the normalisation divides it out exactly.
// PV: each lane accumulates o[head][its EPL dims] for all G heads, taking each
//   token's probabilities from the lanes of its quad with a DPP broadcast.
// Masking: tokens at or past the context length get score -inf and value 0
//   (selected, never multiplied), so poisoned padding cannot leak in.
// Split context: when a sequence spans more than one partition, every
//   partition writes (max, sum, unnormalised output) to the workspace and a
//   second kernel combines the partitions of each (sequence, head) in
//   partition order.  The kernel boundary makes the partials visible without
//   device-wide fences.  The combination order depends only on logical
//   positions, so results are identical under any physical placement.

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "pa_internal.h"

namespace pa {
namespace {

// Partitions of kMidPartitionMin..kShortPartitionTokens tokens (mixed batches
// of many pairs) take 8-wave workgroups and 8-token stages on the grid; groups
// of 8 take 8-token stages up to kShortPartitionTokens.
constexpr int kShortPartitionTokens = 2048;
constexpr int kMidPartitionMin = 1024;
constexpr int kXcds = 8;  // XCDs of the chip; workgroup L is dispatched to XCD L % 8
constexpr float kRescaleThreshold = 8.0f;     // log2 units the running max may lag
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

struct bf16_tag {};

// DPP controls (gfx9 encoding): quad permutations and 16-lane row rotations.
constexpr int kQuadXor1 = 0xB1;  // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int quad_bcast(int k) { return k * 0x55; }  // [k,k,k,k]

// Every control used here (quad permutes, row rotates) reads a valid lane of
// the same 16-lane row for every lane, and all rows and banks are written, so
// the "old" operand is never used: bound_ctrl lets the compiler drop it and
// fold the permute into the instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int NW>
struct Frag {
  uint32_t w[NW];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename V, bool NT>
__device__ __forceinline__ V load_vec(const char *p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
  return *reinterpret_cast<const V *>(p);
}

template <int NW, bool NT = false>
__device__ __forceinline__ void load_frag(Frag<NW> &f, const char *p) {
  if constexpr (NW == 2) {
    const u32x2 x = load_vec<u32x2, NT>(p);
    f.w[0] = x.x;
    f.w[1] = x.y;
  } else if constexpr (NW == 4) {
    const u32x4 x = load_vec<u32x4, NT>(p);
    f.w[0] = x.x;
    f.w[1] = x.y;
    f.w[2] = x.z;
    f.w[3] = x.w;
  } else {
    static_assert(NW == 8, "8, 16 or 32 bytes per lane per token");
    const u32x4 x = load_vec<u32x4, NT>(p);
    const u32x4 y = load_vec<u32x4, NT>(p + 16);
    f.w[0] = x.x;
    f.w[1] = x.y;
    f.w[2] = x.z;
    f.w[3] = x.w;
    f.w[4] = y.x;
    f.w[5] = y.y;
    f.w[6] = y.z;
    f.w[7] = y.w;
  }
}

// Widen one lane's EPL stored elements to fp32 (bf16: low half first).
template <typename T, int NW, int EPL>
__device__ __forceinline__ void widen(const Frag<NW> &f, float (&x)[EPL]) {
  if constexpr (std::is_same_v<T, float>) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = __uint_as_float(f.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      x[2 * i] = __uint_as_float(f.w[i] << 16);
      x[2 * i + 1] = __uint_as_float(f.w[i] & 0xFFFF0000u);
    }
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Partial dot of one lane's EPL dims: query (held as stored words) . key.
template <typename T, int NW>
__device__ __forceinline__ float partial_dot(const Frag<NW> &qw, const Frag<NW> &kw) {
  float acc = 0.0f;
  if constexpr (std::is_same_v<T, float>) {
#pragma unroll
    for (int i = 0; i < NW; ++i) acc = fmaf(__uint_as_float(qw.w[i]), __uint_as_float(kw.w[i]), acc);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw.w[i]),
                                            __builtin_bit_cast(bf16x2_t, kw.w[i]), acc, false);
  }
  return acc;
}

// Reduce-scatter of G partial dots across the 16 lanes of a row.  On entry
// a[r] is this lane's partial for head r ^ sigma(lane), sigma(l) =
// (l % QS) * HPL.  On exit a[t], t < HPL, is the full dot for head
// sigma(lane) + t.  Split steps pair lanes differing in one quad bit; the
// remaining bits are summed with rotations (all lanes then agree).
template <int G>
__device__ __forceinline__ void reduce_heads(float (&a)[G]) {
  if constexpr (G == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += dpp<kQuadXor2>(a[k + 4]);
#pragma unroll
    for (int k = 0; k < 2; ++k) a[k] += dpp<kQuadXor1>(a[k + 2]);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      a[k] += dpp<kRowRor4>(a[k]);
      a[k] += dpp<kRowRor8>(a[k]);
    }
  } else if constexpr (G == 4) {
    a[0] += dpp<kQuadXor2>(a[2]);
    a[1] += dpp<kQuadXor2>(a[3]);
    a[0] += dpp<kQuadXor1>(a[1]);
    a[0] += dpp<kRowRor4>(a[0]);
    a[0] += dpp<kRowRor8>(a[0]);
  } else if constexpr (G == 2) {
    a[0] += dpp<kQuadXor1>(a[1]);
    a[0] += dpp<kQuadXor2>(a[0]);
    a[0] += dpp<kRowRor4>(a[0]);
    a[0] += dpp<kRowRor8>(a[0]);
  } else {
    static_assert(G == 1, "group size 1, 2, 4 or 8");
    a[0] += dpp<kQuadXor1>(a[0]);
    a[0] += dpp<kQuadXor2>(a[0]);
    a[0] += dpp<kRowRor4>(a[0]);
    a[0] += dpp<kRowRor8>(a[0]);
  }
}

// Value of head hh (held by quad lane hh / HPL in register hh % HPL) in every lane.
template <int G, int HPL>
__device__ __forceinline__ float head_value(const float (&v)[HPL], int hh) {
  if constexpr (G == 1) {
    return v[0];
  } else {
    const int k = hh / HPL, t = hh % HPL;
    switch (k) {
      case 0: return dpp<quad_bcast(0)>(v[t]);
      case 1: return dpp<quad_bcast(1)>(v[t]);
      case 2: return dpp<quad_bcast(2)>(v[t]);
      default: return dpp<quad_bcast(3)>(v[t]);
    }
  }
}

// Matrix-core layout (groups of 8, bf16): every lane gets the value held by
// lane hh of its 16-lane row (DPP row_newbcast).
__device__ __forceinline__ float row_lane_value(float v, int hh) {
  switch (hh) {
    case 0: return dpp<0x150>(v);
    case 1: return dpp<0x151>(v);
    case 2: return dpp<0x152>(v);
    case 3: return dpp<0x153>(v);
    case 4: return dpp<0x154>(v);
    case 5: return dpp<0x155>(v);
    case 6: return dpp<0x156>(v);
    default: return dpp<0x157>(v);
  }
}

// Per-head value hh in every lane, for either lane layout.
template <int G, int HPL, bool MQ>
__device__ __forceinline__ float head_bcast(const float (&v)[HPL], int hh) {
  if constexpr (MQ) return row_lane_value(v[0], hh);
  else return head_value<G, HPL>(v, hh);
}

// Partitions a sequence of length L spans (0 when its outputs are set by
// the first partition alone: empty or invalid context).  Both kernels use
// this one definition.
__device__ __forceinline__ int partitions_of(int L, int max_context_len, int max_tokens_per_row,
                                             int part_tokens) {
  if (L < 0 || L > max_context_len || L > max_tokens_per_row) return -1;  // invalid: NaN rows
  if (L == 0) return 0;
  return (L + part_tokens - 1) / part_tokens;
}

template <typename T, int D, int B, int G, int CH>
struct Cfg {
  static constexpr int kElem = std::is_same_v<T, float> ? 4 : 2;
  static constexpr int EPL = D / 16;             // elements per lane per token
  static constexpr int VEC = EPL * kElem;        // bytes per lane per token
  static constexpr int NW = VEC / 4;             // 32-bit words per lane per token
  static constexpr int QS = G < 4 ? G : 4;       // quad lanes that own distinct heads
  static constexpr int HPL = G / QS;             // heads owned per lane
  // A pipeline stage is CH consecutive tokens (STEPS load steps of 4).  Large blocks hold CPB
  // stages; small blocks (B = 4, 8) are grouped R to a stage.  A "unit" is
  // the span a wave takes at a time: one block, or R consecutive blocks.
  static constexpr int STEPS = CH / 4;
  static constexpr int R = B < CH ? CH / B : 1;    // blocks per unit
  static constexpr int CPB = B < CH ? 1 : B / CH;  // pipeline stages per unit
  static constexpr int UNIT = R * B;                       // tokens per unit
  static constexpr int64_t ROW = (int64_t)D * kElem;
  static constexpr int64_t TILE = (int64_t)B * ROW;
  static constexpr int64_t CHUNK = (int64_t)CH * ROW;
  static constexpr int64_t STEP = 64 * VEC;      // bytes per load step (4 tokens)
};

// NT: K/V loads carry the non-temporal hint.  K/V are read once per step, so
// streaming them keeps them from displacing reusable lines in L2; measured on
// the Qwen3-8B batch-64 layer it raised decode bandwidth from 5.8 to 6.4
// TB/s.  Batches whose sequences share blocks want the normal policy instead
// (the later readers of a shared block hit in L2).
//
// MQ: the scores come from the matrix cores (bf16, groups of 8, blocks of 16
// tokens or more; 16-token stages).  Per stage, S^T = K Q^T is one
// v_mfma_f32_16x16x32_bf16 per 32 dims: A = K with lane (g, c) = (lane / 16,
// lane % 16) holding token c, dims 32k + 8g ...; B = Q^T with that lane
// holding head c (zero for c >= G) at the same dims.  The result leaves lane
// (g, c) the scores of tokens 4g .. 4g + 3 for head c, so lane (g, c) runs the
// online softmax of head c over stream g (tokens 4g .. 4g + 3 of every
// stage).  V keeps the vector layout with the token order matched: at load
// step i row r holds token 4r + i, and takes head hh's probability and
// rescale factor from lane hh of its row.
// LIST: the workgroups walk a work list (skewed batches) instead of taking one
// (pair, partition) each from the grid; a separate instantiation, so the
// grid kernels keep their register budget.
template <typename T, int D, int B, int G, int CH, int W, bool NT, bool MQ, bool LIST>
__global__ void __launch_bounds__(64 * W)
decode_kernel(const char *__restrict__ pool, int64_t num_blocks, int num_kv_heads,
              const char *__restrict__ q, float *__restrict__ out, const int32_t *__restrict__ tables,
              int max_blocks_per_seq, const int32_t *__restrict__ context_lens, int num_q_heads,
              float scale_log2, int max_context_len, int part_blocks, int max_parts, int num_pairs,
              float *__restrict__ ws_o, float *__restrict__ ws_ml, const int32_t *__restrict__ items,
              const int32_t *__restrict__ n_items, int32_t *__restrict__ next_item) {
  using C = Cfg<T, D, B, G, CH>;
  constexpr int kWaves = W;  // wavefronts per workgroup
  constexpr int kThreads = 64 * W;
  constexpr int EPL = C::EPL, NW = C::NW, CPB = C::CPB, R = C::R;
  constexpr int NS = C::STEPS;
  constexpr int HPL = MQ ? 1 : C::HPL, QS = MQ ? G : C::QS;
  constexpr int KC = D / 32;           // MQ: matrix-core steps per stage (32 dims each)
  constexpr int KW = MQ ? 4 : NW;      // K words per lane per load
  constexpr int KN = MQ ? KC : NS;     // K loads per stage
  static_assert(B % 4 == 0 && (B < CH ? CH % B == 0 : B % CH == 0), "block size");
  static_assert(!MQ || (!std::is_same_v<T, float> && G == 8 && CH == 16 && B >= CH), "matrix-core layout");

  // Partition length cap in blocks (the host routes longer partitions to the
  // grid launch).
  constexpr int kTblCap = LIST ? kMaxListPartitionBlocks : kMaxPartitionBlocks;
  __shared__ int s_tbl[kTblCap];
  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_bad[kWaves];

  // One-dimensional grid (see the dispatch at the end).  Workgroup wg runs on
  // XCD wg % kXcds; each XCD takes an equal share of the (sequence, KV head)
  // pairs, first partition 0 of each, then partition 1 of each, and so on.
  // In a batch of mixed lengths most pairs have one partition, so the
  // workgroups that exit at once all sit at the end of the dispatch order
  // instead of in a regular pattern among the working ones (measured: with
  // the partition index fastest, an even partition count crowded the work
  // onto a fraction of the compute units, up to 2.7x slower).
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int row = lane >> 4, col = lane & 15;

  // One (sequence-and-KV-head pair, partition) work item; a return ends the item.
  auto run_item = [&](const int pair, const int p) __attribute__((always_inline)) {
  const int h = pair % num_kv_heads, s = pair / num_kv_heads;

  // ---- loads that do not depend on the context length go out first, so
  // their latency overlaps that of the length itself: the queries (register
  // r holds head r ^ sigma(lane), dims col*EPL ...) and, for partition 0 --
  // which every valid context has -- the partition's block ids.
  const int64_t head_row0 = ((int64_t)s * num_q_heads + (int64_t)h * G);  // first query/output row
  Frag<KW> qf[MQ ? KC : G];
  if constexpr (MQ) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qf[kc] = Frag<KW>{};
      if (col < G) load_frag<KW>(qf[kc], q + ((head_row0 + col) * D + 32 * kc + 8 * row) * C::kElem);
    }
  } else {
    const int sigma = (lane % QS) * HPL;
#pragma unroll
    for (int r = 0; r < G; ++r)
      load_frag<NW>(qf[r], q + ((head_row0 + (r ^ sigma)) * D + col * EPL) * C::kElem);
  }
  // Table entries staged per thread; up to two are loaded early (in
  // registers), any further ones (grid partitions of more than 2 kThreads
  // blocks, i.e. small blocks) once the length is known, straight into LDS.
  constexpr int kTblPerThread = (kTblCap + kThreads - 1) / kThreads;
  constexpr int kTblEarly = kTblPerThread < 2 ? kTblPerThread : 2;
  const int blk_begin = p * part_blocks;
  const int32_t *trow = tables + (int64_t)s * max_blocks_per_seq + blk_begin;
  int tb[kTblEarly];
#pragma unroll
  for (int k = 0; k < kTblEarly; ++k) tb[k] = 0;
  if (p == 0) {
    const int n = min(part_blocks, max_blocks_per_seq);
#pragma unroll
    for (int k = 0; k < kTblEarly; ++k)
      if (tid + k * kThreads < n) tb[k] = trow[tid + k * kThreads];
  }

  const int L = context_lens[s];
  const int part_tokens = part_blocks * B;
  const int np = partitions_of(L, max_context_len, max_blocks_per_seq * B, part_tokens);
  const int nparts = np < 1 ? 1 : np;
  if (p >= nparts) return;

  if (np < 0) {
    for (int i = tid; i < G * D; i += kThreads) out[head_row0 * D + i] = __builtin_nanf("");
    return;
  }

  // ---- stage this partition's block ids in LDS (validated; an invalid id
  // reads block 0 and poisons the workgroup's output)
  const int seq_blocks = (L + B - 1) / B;
  const int nblk = min(part_blocks, seq_blocks - blk_begin);
  // The last unit of a sequence of small blocks may reach past its blocks:
  // those entries read block 0 (in bounds) and all their tokens are masked.
  // Partitions hold whole units, so nunits * R <= part_blocks.
  const int nunits = (nblk + R - 1) / R;
  bool bad = false;
  auto stage = [&](int i, int b) {
    if (i < nunits * R) {
      if (i >= nblk) b = 0;
      if (b < 0 || (int64_t)b >= num_blocks) {
        bad = true;
        b = 0;
      }
      s_tbl[i] = b;
    }
  };
#pragma unroll
  for (int k = 0; k < kTblEarly; ++k) {
    const int i = tid + k * kThreads;
    stage(i, p == 0 ? tb[k] : i < nblk ? trow[i] : 0);
  }
  if constexpr (kTblPerThread > kTblEarly) {
#pragma unroll 1
    for (int i = tid + kTblEarly * kThreads; i < nunits * R; i += kThreads) stage(i, i < nblk ? trow[i] : 0);
  }
  const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;  // all lanes take part
  if (lane == 0) s_bad[wave] = wave_bad;
  __syncthreads();

  float m[HPL], lsum[HPL], o[G][EPL];
#pragma unroll
  for (int t = 0; t < HPL; ++t) {
    m[t] = kNegInf;
    lsum[t] = 0.0f;
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.0f;

  // The partition's stages of CH tokens (up to the last that holds a token of
  // the context) are dealt to the waves in turn: wave w takes stages w,
  // w + kWaves, ...  With blocks longer than a stage the waves thus share a
  // block instead of taking whole blocks (33 blocks of 128 tokens over 4
  // waves would leave one wave a ninth block).
  static_assert(C::UNIT == CPB * CH, "a unit is CPB stages: stage g starts at token g * CH");
  const int part_len = min(L - blk_begin * B, nunits * C::UNIT);  // tokens of this partition
  const int nstages = (part_len + CH - 1) / CH;
  const int nch = nstages > wave ? (nstages - wave + kWaves - 1) / kWaves : 0;
  const char *kv_head_base = pool + (int64_t)h * C::TILE;
  const int64_t v_off = (int64_t)num_kv_heads * C::TILE;
  const int lane_off = lane * C::VEC;

  auto issue = [&](int ci, Frag<KW> (&kf)[KN], Frag<NW> (&vf)[NS]) {
    const int g = wave + ci * kWaves;  // this stage's index in the partition
    const int unit = g / CPB;
    if constexpr (MQ) {
      // K: token col, bytes 64 kc + 16 row of its row; V: token 4 row + i, dims col * EPL ...
      const int sub = g % CPB;
      const int phys = __builtin_amdgcn_readfirstlane(s_tbl[unit]);
      const char *cp = kv_head_base + (int64_t)phys * (2 * v_off) + sub * C::CHUNK;
      const char *kp = cp + col * C::ROW + 16 * row;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) load_frag<KW, NT>(kf[kc], kp + 64 * kc);
      const char *vp = cp + v_off + 4 * row * C::ROW + col * C::VEC;
#pragma unroll
      for (int i = 0; i < NS; ++i) load_frag<NW, NT>(vf[i], vp + i * C::ROW);
    } else if constexpr (R == 1) {
      const int sub = g % CPB;
      const int phys = __builtin_amdgcn_readfirstlane(s_tbl[unit]);
      const char *kp = kv_head_base + (int64_t)phys * (2 * v_off) + sub * C::CHUNK + lane_off;
#pragma unroll
      for (int j = 0; j < NS; ++j) load_frag<NW, NT>(kf[j], kp + j * C::STEP);
#pragma unroll
      for (int j = 0; j < NS; ++j) load_frag<NW, NT>(vf[j], kp + v_off + j * C::STEP);
    } else {
      // load step j (4 tokens) lies in block 4j / B of the unit, at row 4j % B
      const char *kp[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int phys = __builtin_amdgcn_readfirstlane(s_tbl[unit * R + (4 * j) / B]);
        kp[j] = kv_head_base + (int64_t)phys * (2 * v_off) + ((4 * j) % B) * C::ROW + lane_off;
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) load_frag<NW, NT>(kf[j], kp[j]);
#pragma unroll
      for (int j = 0; j < NS; ++j) load_frag<NW, NT>(vf[j], kp[j] + v_off);
    }
  };
  // (each layout's body is instantiated only for its own kernels)
  auto process_mq = [&](int ci, const auto &kf, const auto &vf) {
    if constexpr (MQ) {
      const int tok0 = blk_begin * B + (wave + ci * kWaves) * CH;
      const bool partial = tok0 + CH > L;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kc].w),
                                                      __builtin_bit_cast(bf16x8_t, qf[kc].w), acc, 0, 0, 0);
      // lane (row, col): scores of tokens tok0 + 4 row + i for head col
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = (!partial || tok0 + 4 * row + i < L) ? acc[i] * scale_log2 : kNegInf;
      const float cm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      const float mn = fmaxf(m[0], cm);
      const bool upd = mn > m[0] + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(upd) != 0) {
        const float alpha[1] = {upd ? fast_exp2(m[0] - mn) : 1.0f};
        lsum[0] *= alpha[0];
        m[0] = upd ? mn : m[0];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float a = head_bcast<G, HPL, MQ>(alpha, hh);
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[hh][e] *= a;
        }
      }
      const float ms = m[0] == kNegInf ? 0.0f : m[0];
      float pr[4][1];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i][0] = fast_exp2(sc[i] - ms);
      lsum[0] += (pr[0][0] + pr[1][0]) + (pr[2][0] + pr[3][0]);
      // PV: load step i holds token 4 row + i in row `row`
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        float v[EPL];
        widen<T, NW, EPL>(vf[i], v);
        if (partial && !(tok0 + 4 * row + i < L)) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[e] = 0.0f;
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pb = head_bcast<G, HPL, MQ>(pr[i], hh);
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(pb, v[e], o[hh][e]);
        }
      }
    }
  };
  auto process_vec = [&](int ci, const auto &kf, const auto &vf) {
    const int tok0 = blk_begin * B + (wave + ci * kWaves) * CH;
    const bool partial = tok0 + CH > L;
    // QK for the 4 tokens this row sees in the chunk
    float sc[NS][HPL];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float a[G];
#pragma unroll
      for (int r = 0; r < G; ++r) a[r] = partial_dot<T, NW>(qf[r], kf[j]);
      reduce_heads<G>(a);
      const bool valid = !partial || (tok0 + 4 * j + row < L);
#pragma unroll
      for (int t = 0; t < HPL; ++t) sc[j][t] = valid ? a[t] * scale_log2 : kNegInf;
    }
    // online softmax with a lazily raised running max
    bool upd[HPL];
    float m_new[HPL];
    bool any_upd = false;
#pragma unroll
    for (int t = 0; t < HPL; ++t) {
      float cm = sc[0][t];
#pragma unroll
      for (int j = 1; j < NS; ++j) cm = fmaxf(cm, sc[j][t]);
      const float mn = fmaxf(m[t], cm);
      upd[t] = mn > m[t] + kRescaleThreshold;
      m_new[t] = upd[t] ? mn : m[t];
      any_upd |= upd[t];
    }
    if (__builtin_amdgcn_ballot_w64(any_upd) != 0) {
      float alpha[HPL];
#pragma unroll
      for (int t = 0; t < HPL; ++t) {
        alpha[t] = upd[t] ? fast_exp2(m[t] - m_new[t]) : 1.0f;
        lsum[t] *= alpha[t];
        m[t] = m_new[t];
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float a = head_value<G, HPL>(alpha, hh);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] *= a;
      }
    }
    float pr[NS][HPL];
#pragma unroll
    for (int t = 0; t < HPL; ++t) {
      const float ms = m[t] == kNegInf ? 0.0f : m[t];
#pragma unroll
      for (int j = 0; j < NS; ++j) pr[j][t] = fast_exp2(sc[j][t] - ms);
      float ps = pr[0][t];
#pragma unroll
      for (int j = 1; j < NS; ++j) ps += pr[j][t];
      lsum[t] += ps;
    }
    // PV
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float v[EPL];
      widen<T, NW, EPL>(vf[j], v);
      if (partial && !(tok0 + 4 * j + row < L)) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[e] = 0.0f;
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pb = head_value<G, HPL>(pr[j], hh);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(pb, v[e], o[hh][e]);
      }
    }
  };
  auto process = [&](int ci, const Frag<KW> (&kf)[KN], const Frag<NW> (&vf)[NS]) {
    if constexpr (MQ) process_mq(ci, kf, vf);
    else process_vec(ci, kf, vf);
  };

  // ---- main loop: double-buffered K/V chunks, two per iteration with no
  // exit in between.  Every load is issued unconditionally (the prefetch past
  // the end re-reads the last chunk, an L2 hit), so the compiler's wait
  // counts at each use cover exactly the loads issued before it: each
  // process() waits for its own chunk while the next one is in flight.
  // One chunk is in flight ahead of the one being processed (measured on the
  // Qwen3-8B batch-64 layer: two ahead was 3 % slower and cost 20 more VGPRs).
  if (nch > 0) {
    Frag<KW> kA[KN];
    Frag<NW> vA[NS];
    Frag<KW> kB[KN];
    Frag<NW> vB[NS];
    const int last = nch - 1;
    issue(0, kA, vA);
    int ci = 0;
    for (; ci < last; ci += 2) {
      issue(ci + 1, kB, vB);
      process(ci, kA, vA);
      issue(min(ci + 2, last), kA, vA);
      process(ci + 1, kB, vB);
    }
    if (ci == last) process(ci, kA, vA);
  }

  // ---- merge the four row streams of this wave (partners lane ^ 16, lane ^ 32)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    float a1[HPL], a2[HPL];
#pragma unroll
    for (int t = 0; t < HPL; ++t) {
      const float m2 = __shfl_xor(m[t], off);
      const float l2 = __shfl_xor(lsum[t], off);
      const float M = fmaxf(m[t], m2);
      const float Ms = M == kNegInf ? 0.0f : M;
      a1[t] = fast_exp2(m[t] - Ms);
      a2[t] = fast_exp2(m2 - Ms);
      lsum[t] = a1[t] * lsum[t] + a2[t] * l2;
      m[t] = M;
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float b1 = head_bcast<G, HPL, MQ>(a1, hh);
      const float b2 = head_bcast<G, HPL, MQ>(a2, hh);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o2 = __shfl_xor(o[hh][e], off);
        o[hh][e] = b1 * o[hh][e] + b2 * o2;
      }
    }
  }

  // ---- merge the waves through LDS
  if (row == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][hh][col * EPL + e] = o[hh][e];
  }
  if (lane < QS) {
#pragma unroll
    for (int t = 0; t < HPL; ++t) {
      s_m[wave][lane * HPL + t] = m[t];
      s_l[wave][lane * HPL + t] = lsum[t];
    }
  }
  __syncthreads();
  bool poisoned = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) poisoned |= s_bad[w] != 0;
  for (int i = tid; i < G * D; i += kThreads) {
    const int hh = i / D, d = i - hh * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][hh]);
    const float Ms = M == kNegInf ? 0.0f : M;
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = fast_exp2(s_m[w][hh] - Ms);
      num += a * s_o[w][hh][d];
      den += a * s_l[w][hh];
    }
    if (poisoned) num = den = M = __builtin_nanf("");
    if (nparts == 1) {
      out[(head_row0 + hh) * D + d] = den > 0.0f ? num / den : (poisoned ? num : 0.0f);
    } else {
      const int64_t prow = (head_row0 + hh) * max_parts + p;
      ws_o[prow * D + d] = num;
      if (d == 0) {
        ws_ml[prow * 2] = M;
        ws_ml[prow * 2 + 1] = den;
      }
    }
  }
  };

  if constexpr (!LIST) {
    // The grid holds one workgroup per (pair, partition).  Streaming loads
    // (no shared blocks), vector scores: XCD x takes the x-th eighth of the
    // pairs in order, so the KV heads of a sequence -- the 4 KiB tiles that
    // make up each of its 64 KiB blocks -- are read together by one XCD (1 %
    // faster than head by head on the Qwen3-8B batch-64 layer).  Otherwise
    // XCD x takes pairs x, x + 8, ..., i.e. KV head x of every sequence at 8
    // KV heads: with blocks shared by several sequences (cached loads) the
    // sharers of a block then read it through one L2 (4 % faster than by
    // sequence on a shared prefix), and the matrix-core kernel's few long
    // partitions measured no better by sequence.
    constexpr bool kBySequence = NT && !MQ;
    const int wg = blockIdx.x, xcd = wg % kXcds, j = wg / kXcds;
    const int per_xcd = (num_pairs + kXcds - 1) / kXcds;
    const int pair = kBySequence ? xcd * per_xcd + (j % per_xcd) : (j % per_xcd) * kXcds + xcd;
    const int p = j / per_xcd;
    if (pair < num_pairs) run_item(pair, p);
  } else {
    // Work list (skewed batches of many pairs): the items with work, longest
    // first.  A grid of resident workgroups takes item blockIdx.x first, then
    // the next untaken one from a counter (grid + the counter's old value),
    // fetched while the current item runs.  Every workgroup leaves the loop
    // once the index passes the item count, which it reads once.
    __shared__ int s_next_item;
    const int n = __builtin_amdgcn_readfirstlane(*n_items);
    int i = blockIdx.x;
    while (i < n) {
      int grabbed = 0;
      if (tid == 0) grabbed = atomicAdd(next_item, 1);
      const int it = __builtin_amdgcn_readfirstlane(items[i]);
      const int pair = it / max_parts;
      run_item(pair, it - pair * max_parts);
      if (tid == 0) s_next_item = (int)gridDim.x + grabbed;
      __syncthreads();
      i = s_next_item;
      __syncthreads();  // every thread has read it before thread 0 writes the next
    }
  }
}

// The work list of a decode call over a skewed batch: every (pair,
// partition) item that has work -- one per partition a sequence spans, a
// single one for an empty or invalid context (it writes that sequence's
// zero or NaN rows) -- sorted longest first (a counting sort on the item's
// length in 1/256ths of a partition), all KV heads of a (sequence,
// partition) next to each other from a multiple of the head count.  One
// workgroup; the order inside a length class follows atomics and does not
// matter (every item writes its own outputs, and the partitions of a
// sequence are combined in partition order).  Also resets the counter the
// decode's workgroups take items from.
constexpr int kListThreads = 1024;
constexpr int kListBuckets = 256;

__device__ __forceinline__ int item_bucket(int L, int np, int p, int part_tokens) {
  if (np < 1) return 0;  // empty or invalid context: writes its rows only
  const int len = min(part_tokens, L - p * part_tokens);
  return (int)((int64_t)len * (kListBuckets - 1) / part_tokens);
}

__global__ void __launch_bounds__(kListThreads)
worklist_kernel(const int32_t *__restrict__ context_lens, int num_seqs, int num_kv_heads, int max_context_len,
                int max_tokens_per_row, int part_tokens, int max_parts, int32_t *__restrict__ items,
                int32_t *__restrict__ n_items, int32_t *__restrict__ next_item) {
  __shared__ int s_count[kListBuckets];
  __shared__ int s_next[kListBuckets];
  const int tid = threadIdx.x;
  for (int b = tid; b < kListBuckets; b += kListThreads) s_count[b] = 0;
  __syncthreads();
  // a sequence's partitions before its last are full (the longest class), so
  // each sequence takes at most two atomics per pass
  for (int s = tid; s < num_seqs; s += kListThreads) {
    const int L = context_lens[s];
    const int np = partitions_of(L, max_context_len, max_tokens_per_row, part_tokens);
    if (np > 1) atomicAdd(&s_count[kListBuckets - 1], np - 1);
    atomicAdd(&s_count[item_bucket(L, np, max(np, 1) - 1, part_tokens)], 1);
  }
  __syncthreads();
  // start of each length class, longest first: an exclusive scan of the
  // classes in descending order, one class per thread of the first 4 waves
  static_assert(kListBuckets == 4 * 64, "four waves scan the classes");
  __shared__ int s_wave_sum[4];
  int c = 0, incl = 0;
  if (tid < kListBuckets) {
    c = s_count[kListBuckets - 1 - tid] * num_kv_heads;
    incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if ((tid & 63) >= off) incl += y;
    }
    if ((tid & 63) == 63) s_wave_sum[tid >> 6] = incl;
  }
  __syncthreads();
  if (tid < kListBuckets) {
    int before = 0;
    for (int w = 0; w < (tid >> 6); ++w) before += s_wave_sum[w];
    s_next[kListBuckets - 1 - tid] = before + incl - c;
    if (tid == kListBuckets - 1) {
      *n_items = before + incl;
      *next_item = 0;
    }
  }
  __syncthreads();
  for (int s = tid; s < num_seqs; s += kListThreads) {
    const int L = context_lens[s];
    const int np = partitions_of(L, max_context_len, max_tokens_per_row, part_tokens);
    const int last = max(np, 1) - 1;
    if (np > 1) {
      const int at = atomicAdd(&s_next[kListBuckets - 1], (np - 1) * num_kv_heads);
      for (int p = 0; p < last; ++p)
        for (int h = 0; h < num_kv_heads; ++h)
          items[at + p * num_kv_heads + h] = (s * num_kv_heads + h) * max_parts + p;
    }
    const int at = atomicAdd(&s_next[item_bucket(L, np, last, part_tokens)], num_kv_heads);
    for (int h = 0; h < num_kv_heads; ++h) items[at + h] = (s * num_kv_heads + h) * max_parts + last;
  }
}

// Combine the partitions of (sequence, query head) rows.  Both forms take
// the maximum over partitions, then the weighted sums in partition order with
// the loads of 8 partitions issued together, so the result depends only on
// logical positions and is the same bits in both; rows of sequences that fit
// one partition were written by the decode itself and are skipped.
//
// combine_kernel: one workgroup of D threads per row, thread d holding dim d
// (the maximum: thread d reads partitions d, d + D, ..., then a workgroup
// reduction).  For calls with few rows, each spread over its own compute unit.
template <int D>
__global__ void __launch_bounds__(D)
combine_kernel(const float *__restrict__ ws_o, const float *__restrict__ ws_ml, float *__restrict__ out,
               const int32_t *__restrict__ context_lens, int num_q_heads, int max_context_len,
               int max_tokens_per_row, int part_tokens, int max_parts) {
  constexpr int kCombineWaves = D / 64;
  constexpr int kBatch = 8;
  __shared__ float s_max[kCombineWaves];
  const int hq = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int np = partitions_of(context_lens[s], max_context_len, max_tokens_per_row, part_tokens);
  if (np <= 1) return;
  const int64_t row = (int64_t)s * num_q_heads + hq;
  const float *ml = ws_ml + row * max_parts * 2;
  const float *o = ws_o + row * max_parts * D + d;
  float M = kNegInf;
  for (int p = d; p < np; p += D) M = fmaxf(M, ml[2 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((d & 63) == 0) s_max[d >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) M = fmaxf(M, s_max[w]);
  const float Ms = M == kNegInf ? 0.0f : M;
  float num = 0.0f, den = 0.0f;
  int p = 0;
  for (; p + kBatch <= np; p += kBatch) {
    float mv[kBatch], lv[kBatch], ov[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      mv[k] = ml[2 * (p + k)];
      lv[k] = ml[2 * (p + k) + 1];
      ov[k] = o[(int64_t)(p + k) * D];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float a = fast_exp2(mv[k] - Ms);
      num += a * ov[k];
      den += a * lv[k];
    }
  }
  for (; p < np; ++p) {
    const float a = fast_exp2(ml[2 * p] - Ms);
    num += a * o[(int64_t)p * D];
    den += a * ml[2 * p + 1];
  }
  out[row * D + d] = num / den;
}

// combine_many_kernel: one wave per row, four rows per workgroup, lane l
// holding dims DPL*l .. DPL*l + DPL-1 (the maximum: lane l reads partitions
// l, l + 64, ..., then a wave reduction).  For calls with many rows, most of
// which (in a skewed batch) need no combining: 4x fewer workgroups to
// dispatch than one per row (1 % of a call over 512 x 32 rows; with few rows
// it is 2-3 % slower than combine_kernel).
constexpr int kCombineRows = 4;
constexpr int64_t kCombineManyRows = 4096;

template <int D>
__global__ void __launch_bounds__(64 * kCombineRows)
combine_many_kernel(const float *__restrict__ ws_o, const float *__restrict__ ws_ml, float *__restrict__ out,
                    const int32_t *__restrict__ context_lens, int num_seqs, int num_q_heads, int max_context_len,
                    int max_tokens_per_row, int part_tokens, int max_parts) {
  constexpr int DPL = D / 64;
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kCombineRows + (threadIdx.x >> 6);
  if (row >= (int64_t)num_seqs * num_q_heads) return;
  const int s = (int)(row / num_q_heads);
  const int np = partitions_of(context_lens[s], max_context_len, max_tokens_per_row, part_tokens);
  if (np <= 1) return;
  const float *ml = ws_ml + row * max_parts * 2;
  const float *o = ws_o + row * max_parts * D + lane * DPL;
  float M = kNegInf;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[2 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float Ms = M == kNegInf ? 0.0f : M;
  float num[DPL], den = 0.0f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) num[e] = 0.0f;
  int p = 0;
  for (; p + kBatch <= np; p += kBatch) {
    float mv[kBatch], lv[kBatch], ov[kBatch][DPL];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      mv[k] = ml[2 * (p + k)];
      lv[k] = ml[2 * (p + k) + 1];
#pragma unroll
      for (int e = 0; e < DPL; ++e) ov[k][e] = o[(int64_t)(p + k) * D + e];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float a = fast_exp2(mv[k] - Ms);
#pragma unroll
      for (int e = 0; e < DPL; ++e) num[e] += a * ov[k][e];
      den += a * lv[k];
    }
  }
  for (; p < np; ++p) {
    const float a = fast_exp2(ml[2 * p] - Ms);
#pragma unroll
    for (int e = 0; e < DPL; ++e) num[e] += a * o[(int64_t)p * D + e];
    den += a * ml[2 * p + 1];
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[row * D + lane * DPL + e] = num[e] / den;
}

// The one rule for which launches take their scores from the matrix cores.
constexpr bool matrix_core_scores(bool bf16, int group, int block_size) {
  return bf16 && group == 8 && block_size >= 16;
}

// Workgroups of `kernel` (with `threads` threads) resident on the whole
// device at once: the grid of a work-list launch.
int resident_workgroups(const void *kernel, int threads) {
  static std::mutex mu;
  static std::map<std::pair<const void *, int>, int> cache;  // (kernel, device) -> workgroups
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(kernel, dev);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int n = per_cu * cus / kXcds * kXcds;
  cache[key] = n;
  return n;
}

template <typename T, int D, int B, int G>
hipError_t launch_one(const DecodeArgs &a, hipStream_t stream) {
  const int pairs = a.num_seqs * a.pool.num_kv_heads;
  const int64_t grid_items = (int64_t)((pairs + kXcds - 1) / kXcds) * kXcds * a.num_partitions;
  // Work shape per launch (measured on MI355X; see the partition choice):
  // - groups up to 4: 4-waves workgroups with 4-token stages (less in flight
  //   per wave; short contexts reach their first score sooner: up to 27 %
  //   faster on 128-token contexts, the same on long ones), except partitions
  //   of 1,024-2,048 tokens -- the many-pair mixed batches -- which take 8 waves
  //   and 8-token stages on the grid (4-6 % faster there; 4 % slower on
  //   4,096-token partitions, 39 % slower on 256-token ones); a work-list
  //   launch keeps 4-wave workgroups, twice as many items in flight per
  //   compute unit (0.9 % faster on 512 lognormal contexts);
  // - groups of 8 carry twice the arithmetic per token: bf16 pools with
  //   blocks of 16 or more take their scores from the matrix cores
  //   (16-token stages); otherwise 8-token stages up to 2,048-token
  //   partitions, 16-token stages for the long partitions of a few long
  //   sequences.
  const bool listed = a.items != nullptr;
  auto pick = [&](auto ch, auto w, auto mq) {
    constexpr int CH = decltype(ch)::value, W = decltype(w)::value;
    constexpr bool MQ = decltype(mq)::value;
    if (listed)
      return a.stream_loads ? decode_kernel<T, D, B, G, CH, W, true, MQ, true>
                            : decode_kernel<T, D, B, G, CH, W, false, MQ, true>;
    return a.stream_loads ? decode_kernel<T, D, B, G, CH, W, true, MQ, false>
                          : decode_kernel<T, D, B, G, CH, W, false, MQ, false>;
  };
  using vec = std::false_type;
  using ch4 = std::integral_constant<int, 4>;
  using ch8 = std::integral_constant<int, 8>;
  using ch16 = std::integral_constant<int, 16>;
  using w4 = std::integral_constant<int, 4>;
  using w8 = std::integral_constant<int, 8>;
  const int part_tokens = a.partition_blocks * B;
  const bool mid = part_tokens >= kMidPartitionMin && part_tokens <= kShortPartitionTokens;
  auto kernel = pick(ch4{}, w4{}, vec{});
  int waves = 4;
  if constexpr (matrix_core_scores(!std::is_same_v<T, float>, G, B)) {
    kernel = pick(ch16{}, w4{}, std::true_type{});
  } else if constexpr (G > 4) {
    kernel = part_tokens <= kShortPartitionTokens ? pick(ch8{}, w4{}, vec{}) : pick(ch16{}, w4{}, vec{});
  } else if (mid && !listed) {
    kernel = pick(ch8{}, w8{}, vec{});
    waves = 8;
  }
  int64_t grid = grid_items;
  if (a.items != nullptr) {
    const int resident = resident_workgroups(reinterpret_cast<const void *>(kernel), 64 * waves);
    if (resident <= 0) return hipErrorInvalidValue;
    grid = std::min<int64_t>(grid_items, resident);
    hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(kListThreads), 0, stream, a.context_lens, a.num_seqs,
                       a.pool.num_kv_heads, a.max_context_len, a.max_blocks_per_seq * B, a.partition_blocks * B,
                       a.num_partitions, a.items, a.n_items, a.next_item);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64 * waves), 0, stream,
                     static_cast<const char *>(a.pool.base), a.pool.num_blocks, a.pool.num_kv_heads,
                     static_cast<const char *>(a.q), a.out, a.block_tables, a.max_blocks_per_seq,
                     a.context_lens, a.num_q_heads, a.scale * kLog2e, a.max_context_len, a.partition_blocks,
                     a.num_partitions, pairs, a.ws_o, a.ws_ml, a.items, a.n_items, a.next_item);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions == 1) return e;
  const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
  if (rows >= kCombineManyRows)
    hipLaunchKernelGGL((combine_many_kernel<D>), dim3((unsigned)((rows + kCombineRows - 1) / kCombineRows)),
                       dim3(64 * kCombineRows), 0, stream, a.ws_o, a.ws_ml, a.out, a.context_lens, a.num_seqs,
                       a.num_q_heads, a.max_context_len, a.max_blocks_per_seq * B, a.partition_blocks * B,
                       a.num_partitions);
  else
    hipLaunchKernelGGL((combine_kernel<D>), dim3(a.num_q_heads, a.num_seqs), dim3(D), 0, stream, a.ws_o, a.ws_ml,
                       a.out, a.context_lens, a.num_q_heads, a.max_context_len, a.max_blocks_per_seq * B,
                       a.partition_blocks * B, a.num_partitions);
  return hipGetLastError();
}

template <typename T, int D, int B>
hipError_t dispatch_group(const DecodeArgs &a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<T, D, B, 1>(a, stream);
    case 2: return launch_one<T, D, B, 2>(a, stream);
    case 4: return launch_one<T, D, B, 4>(a, stream);
    case 8: return launch_one<T, D, B, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t dispatch_block(const DecodeArgs &a, int group, hipStream_t stream) {
  switch (a.pool.block_size) {
    case 4: return dispatch_group<T, D, 4>(a, group, stream);
    case 8: return dispatch_group<T, D, 8>(a, group, stream);
    case 16: return dispatch_group<T, D, 16>(a, group, stream);
    case 32: return dispatch_group<T, D, 32>(a, group, stream);
    case 64: return dispatch_group<T, D, 64>(a, group, stream);
    case 128: return dispatch_group<T, D, 128>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t dispatch_dim(const DecodeArgs &a, int group, hipStream_t stream) {
  switch (a.pool.head_dim) {
    case 64: return dispatch_block<T, 64>(a, group, stream);
    case 128: return dispatch_block<T, 128>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_matrix_core_scores(int dtype, int group, int block_size) {
  return matrix_core_scores(dtype == PA_BF16, group, block_size);
}

bool decode_supported(int dtype, int head_dim, int block_size, int group) {
  return (dtype == PA_F32 || dtype == PA_BF16) && (head_dim == 64 || head_dim == 128) &&
         (block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64 ||
          block_size == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  const int group = a.num_q_heads / a.pool.num_kv_heads;
  if (a.pool.dtype == PA_BF16) return dispatch_dim<bf16_tag>(a, group, stream);
  if (a.pool.dtype == PA_F32) return dispatch_dim<float>(a, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
