// Bandwidth ceilings of the GPU the decode kernels run on, measured with
// the same kind of loads they issue.  Not part of the decode library: the
// benchmark loads this small library on its own to report each kernel's
// fraction of what the memory system delivers in practice, next to its
// fraction of the nominal HBM peak.
//
//  * stream read: every byte of one buffer read once, in order, with
//    16-byte loads (each wave reads a contiguous 4 KiB chunk per step);
//  * block gather: a list of 4 KiB blocks at random places in a pool,
//    read in list order by waves that each walk their own contiguous part
//    of the list, several blocks in flight per wave: the access pattern of
//    paged decode (a block of 16 tokens of one KV head is 4 KiB of bf16 K
//    or V at head size 128).
//
// Loads are non-temporal (streamed past the caches) or normal, as chosen.
// Each wave folds what it read into one word that it stores, so that no
// load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paprobe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4 *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ unsigned fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Wave w reads the 4 KiB chunks w, w + nwaves, ... of the buffer, DEPTH
// chunks at a time.
template <bool NT, int DEPTH>
__global__ __launch_bounds__(64) void stream_read(const u32x4 *buf, int64_t chunks,
                                                  unsigned *sink) {
  const int lane = (int)threadIdx.x;
  const int64_t nw = gridDim.x;
  unsigned acc = 0;
  for (int64_t c0 = blockIdx.x; c0 < chunks; c0 += nw * DEPTH) {
    u32x4 v[DEPTH][4];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      const int64_t c = c0 + (int64_t)k * nw;
      const u32x4 *p = buf + c * 256 + lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[k][j] = c < chunks ? load16<NT>(p + 64 * j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= fold(v[k][j]);
  }
  sink[(int64_t)blockIdx.x * 64 + lane] = acc;
}

// Wave w reads list entries [n * w / nw, n * (w + 1) / nw) in order, DEPTH
// blocks in flight: block ids[i] is 4 KiB at pool + ids[i] * 4096.  An id
// outside [0, pool_blocks) reads block 0.
template <bool NT, int DEPTH>
__global__ __launch_bounds__(64) void block_gather(const u32x4 *pool, int64_t pool_blocks,
                                                   const int32_t *ids, int64_t n,
                                                   unsigned *sink) {
  const int lane = (int)threadIdx.x;
  const int64_t nw = gridDim.x, w = blockIdx.x;
  const int64_t i0 = n * w / nw, i1 = n * (w + 1) / nw;
  unsigned acc = 0;
  for (int64_t i = i0; i < i1; i += DEPTH) {
    u32x4 v[DEPTH][4];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      const bool ok = i + k < i1;
      const int64_t id = ok ? ids[i + k] : 0;
      const int64_t b = id >= 0 && id < pool_blocks ? id : 0;
      const u32x4 *p = pool + b * 256 + lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[k][j] = ok ? load16<NT>(p + 64 * j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= fold(v[k][j]);
  }
  sink[w * 64 + lane] = acc;
}

template <bool NT>
hipError_t launch_stream(const void *buf, int64_t bytes, unsigned *sink, int waves, int depth,
                         hipStream_t st) {
  const u32x4 *b = static_cast<const u32x4 *>(buf);
  const int64_t chunks = bytes / 4096;
  switch (depth) {
    case 1: hipLaunchKernelGGL((stream_read<NT, 1>), dim3(waves), dim3(64), 0, st, b, chunks, sink); break;
    case 2: hipLaunchKernelGGL((stream_read<NT, 2>), dim3(waves), dim3(64), 0, st, b, chunks, sink); break;
    case 4: hipLaunchKernelGGL((stream_read<NT, 4>), dim3(waves), dim3(64), 0, st, b, chunks, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool NT>
hipError_t launch_gather(const void *pool, int64_t nb, const int32_t *ids, int64_t n,
                         unsigned *sink, int waves, int depth, hipStream_t st) {
  const u32x4 *p = static_cast<const u32x4 *>(pool);
  switch (depth) {
    case 1: hipLaunchKernelGGL((block_gather<NT, 1>), dim3(waves), dim3(64), 0, st, p, nb, ids, n, sink); break;
    case 2: hipLaunchKernelGGL((block_gather<NT, 2>), dim3(waves), dim3(64), 0, st, p, nb, ids, n, sink); break;
    case 4: hipLaunchKernelGGL((block_gather<NT, 4>), dim3(waves), dim3(64), 0, st, p, nb, ids, n, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

extern "C" {

int32_t probe_stream_read(const void *buf, int64_t bytes, void *sink, int32_t waves,
                          int32_t depth, int32_t nontemporal, void *stream) {
  if (!buf || !sink || bytes < 4096 || bytes % 4096 != 0 || waves <= 0 || !aligned(buf, 16))
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned *s = static_cast<unsigned *>(sink);
  const hipError_t e = nontemporal ? launch_stream<true>(buf, bytes, s, waves, depth, st)
                                   : launch_stream<false>(buf, bytes, s, waves, depth, st);
  return e == hipSuccess ? 0 : -5;
}

int32_t probe_block_gather(const void *pool, int64_t pool_blocks, const int32_t *block_ids,
                           int64_t num_ids, void *sink, int32_t waves, int32_t depth,
                           int32_t nontemporal, void *stream) {
  if (!pool || !block_ids || !sink || pool_blocks <= 0 || num_ids <= 0 || waves <= 0 ||
      !aligned(pool, 16))
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned *s = static_cast<unsigned *>(sink);
  const hipError_t e =
      nontemporal ? launch_gather<true>(pool, pool_blocks, block_ids, num_ids, s, waves, depth, st)
                  : launch_gather<false>(pool, pool_blocks, block_ids, num_ids, s, waves, depth, st);
  return e == hipSuccess ? 0 : -5;
}

}  // extern "C"
