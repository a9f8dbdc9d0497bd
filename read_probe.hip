// HBM read-rate probe for gfx950, used by bench.py --read-ceiling to measure
// the practical ceiling beside the decode kernel's rate: how fast one MI355X
// reads a buffer in pieces of a given size taken in a given order (in order,
// or randomly placed like the physical blocks of a paged KV cache), with the
// decode kernel's access style -- 16-byte non-temporal loads, one wavefront
// load covering 1 KiB contiguous -- and, in order, with direct-to-LDS loads.
// Built into libpa_probe.so, apart from the library; nothing in the
// paged-attention path uses it.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;     // 4 waves: one 4 KiB chunk per load round
constexpr int64_t kChunk = 4096;  // bytes one workgroup load round covers

// Chunk c of the walk lies in piece order[c / per_piece] at chunk c % per_piece
// of that piece.  Workgroup g takes chunks g, g + G, ...; U chunks' loads are
// issued before any is used.  The XOR of everything read goes to sink so no
// load can be dropped.
template <int U>
__global__ void __launch_bounds__(kThreads)
read_kernel(const char *__restrict__ base, const int32_t *__restrict__ order, int64_t per_piece,
            int64_t num_chunks, uint32_t *__restrict__ sink) {
  const int64_t G = gridDim.x;
  const int lane_off = threadIdx.x * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t c0 = blockIdx.x; c0 < num_chunks; c0 += G * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * G;
      const int64_t cc = c < num_chunks ? c : c0;  // past the end: re-read the first chunk
      const int64_t piece = order[cc / per_piece];
      const char *p = base + (piece * per_piece + cc % per_piece) * kChunk + lane_off;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// The same in-order walk with direct-to-LDS loads (global_load_lds_dwordx4,
// the prefill kernel's path): each wave moves its 1 KiB of a chunk into a
// ring of kRing chunks in LDS and keeps U chunks' loads in flight (waits for
// at most U - 1 outstanding after each issue).  Nothing reads the ring until
// the end, when each thread sends one word of it to sink.
constexpr int kRing = 8;

template <int U>
__global__ void __launch_bounds__(kThreads)
read_lds_kernel(const char *__restrict__ base, int64_t num_chunks, uint32_t *__restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char ring[kRing * kChunk];
  const int64_t G = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr unsigned kWait = (0x7u << 4) | (0xFu << 8) | ((U - 1) & 0xFu) | (((U - 1) >> 4) << 14);
  int k = 0;
  for (int64_t c = blockIdx.x; c < num_chunks; c += G, ++k) {
    const char *src = base + c * kChunk + wave * 1024 + lane * 16;
    char *dst = ring + (k % kRing) * kChunk + wave * 1024;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(kWait);  // vmcnt(U - 1)
  }
  __builtin_amdgcn_s_waitcnt((0x7u << 4) | (0xFu << 8));  // vmcnt(0)
  __syncthreads();
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = *reinterpret_cast<const uint32_t *>(&ring[threadIdx.x * 16]);
}

}  // namespace

extern "C" {

// Reads num_pieces pieces of piece_bytes (a multiple of 4 KiB) from `base`
// (device memory, num_pieces * piece_bytes bytes) in the order `order`
// (int32 [num_pieces], a permutation of 0 .. num_pieces-1, device memory) with
// `grid` workgroups of 256 threads and `unroll` (1, 2, 4 or 8) 4 KiB chunks in
// flight per workgroup.  `sink` (device, grid * 256 uint32) receives a value
// per thread.  Enqueues one kernel on `stream`; returns 0, or -1 for invalid
// arguments (nothing launched), or -4 when the launch fails.
int pa_probe_read(const void *base, int64_t piece_bytes, const int32_t *order, int64_t num_pieces, int grid,
                  int unroll, uint32_t *sink, hipStream_t stream) {
  if (base == nullptr || order == nullptr || sink == nullptr || piece_bytes <= 0 || piece_bytes % kChunk != 0 ||
      num_pieces <= 0 || grid <= 0)
    return -1;
  const int64_t per_piece = piece_bytes / kChunk;
  const int64_t chunks = per_piece * num_pieces;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, static_cast<const char *>(base), order, per_piece, chunks, sink); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, static_cast<const char *>(base), order, per_piece, chunks, sink); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, static_cast<const char *>(base), order, per_piece, chunks, sink); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, dim3(grid), dim3(kThreads), 0, stream, static_cast<const char *>(base), order, per_piece, chunks, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Reads `bytes` (a multiple of 4 KiB) from `base` in order with direct-to-LDS
// loads, `grid` workgroups of 256 threads, `unroll` (2, 4, 8 or 16) chunks in
// flight per wave; `sink` (device, grid * 256 uint32) receives a value per
// thread.  Enqueues one kernel on `stream`; returns 0, -1 for invalid
// arguments (nothing launched), or -4 when the launch fails.
int pa_probe_read_lds(const void *base, int64_t bytes, int grid, int unroll, uint32_t *sink, hipStream_t stream) {
  if (base == nullptr || sink == nullptr || bytes <= 0 || bytes % kChunk != 0 || grid <= 0) return -1;
  const int64_t chunks = bytes / kChunk;
  const char *b = static_cast<const char *>(base);
  switch (unroll) {
    case 2: hipLaunchKernelGGL(read_lds_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, b, chunks, sink); break;
    case 4: hipLaunchKernelGGL(read_lds_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, b, chunks, sink); break;
    case 8: hipLaunchKernelGGL(read_lds_kernel<8>, dim3(grid), dim3(kThreads), 0, stream, b, chunks, sink); break;
    case 16: hipLaunchKernelGGL(read_lds_kernel<16>, dim3(grid), dim3(kThreads), 0, stream, b, chunks, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
