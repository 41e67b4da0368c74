// Companion kernels of the paged KV cache for gfx950.
//
//  * reshape_and_cache: each new token's K/V go into the slot its block table
//    gives it; a block is taken only when a sequence's growth needs one (dmarx
//    note-023, "Method"; crackai.dev, "How It Works").  A slot is
//    block * block_size + offset; negative slots are skipped.
//  * copy_blocks: the copy half of copy-on-write, giving a writer its own
//    copy of a shared block (note-023, "Concepts"; inferensys glossary,
//    second paragraph).  Whole blocks: K and V, all heads, all slots.
//  * swap_blocks: the same copy between two pools (device and pinned host
//    memory), for swapping preempted sequences out and back in (inferensys
//    glossary, third and fifth paragraphs).
//
// Both are bit copies.  Pool layout, x = 16 / element size (block_size a
// multiple of 16):
//   key   [num_blocks][Hkv][d / x][block_size][x]
//   value [num_blocks][Hkv][block_size / 16][d][16]
// Indices read from device memory (slots, pairs) are range-checked before
// use; out-of-range entries are skipped so a bad input can never fault.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One thread per (token, KV head, 16-byte feature chunk).  The key chunk is
// one 16-byte store (keys keep x features of a token together); the value
// chunk scatters to x rows of the token's [d][16] value group.
template <int ESZ>
__device__ __forceinline__ void reshape_one(const char *__restrict__ key,
                                            const char *__restrict__ value,
                                            char *__restrict__ key_cache,
                                            char *__restrict__ value_cache,
                                            const int64_t *__restrict__ slots, int num_tokens,
                                            int num_kv_heads, int head_dim, int block_size,
                                            int64_t num_blocks) {
  constexpr int X = 16 / ESZ;
  const int chunks = head_dim / X;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  if (gid >= total) return;
  const int c = (int)(gid % chunks);
  const int h = (int)((gid / chunks) % num_kv_heads);
  const int64_t tok = gid / ((int64_t)chunks * num_kv_heads);
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_blocks * block_size) return;
  const int64_t b = slot / block_size;
  const int o = (int)(slot % block_size);
  const int64_t src = ((tok * num_kv_heads + h) * head_dim + (int64_t)c * X) * ESZ;
  const int64_t head_base = (b * num_kv_heads + h) * (int64_t)head_dim * block_size;
  const u32x4 kv = *reinterpret_cast<const u32x4 *>(key + src);
  *reinterpret_cast<u32x4 *>(key_cache + (head_base + ((int64_t)c * block_size + o) * X) * ESZ) =
      kv;
  const u32x4 vv = *reinterpret_cast<const u32x4 *>(value + src);
  char *vdst =
      value_cache +
      (head_base + (int64_t)(o / 16) * head_dim * 16 + (int64_t)c * X * 16 + o % 16) * ESZ;
#pragma unroll
  for (int e = 0; e < X; ++e) {
    if (ESZ == 4) {
      *reinterpret_cast<unsigned *>(vdst + (int64_t)e * 16 * ESZ) = vv[e];
    } else {
      const unsigned w = vv[e >> 1];
      *reinterpret_cast<uint16_t *>(vdst + (int64_t)e * 16 * ESZ) =
          (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
  }
}

template <int ESZ>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const char *__restrict__ key, const char *__restrict__ value, char *__restrict__ key_cache,
    char *__restrict__ value_cache, const int64_t *__restrict__ slots, int num_tokens,
    int num_kv_heads, int head_dim, int block_size, int64_t num_blocks) {
  reshape_one<ESZ>(key, value, key_cache, value_cache, slots, num_tokens, num_kv_heads,
                   head_dim, block_size, num_blocks);
}

// Every layer's new tokens in one launch: grid.y = layer, each layer with
// its own inputs and pools (device arrays of pointers), the same slots.
template <int ESZ>
__global__ __launch_bounds__(256) void reshape_and_cache_layers_kernel(
    const char *const *keys, const char *const *values, char *const *key_caches,
    char *const *value_caches, const int64_t *__restrict__ slots, int num_tokens,
    int num_kv_heads, int head_dim, int block_size, int64_t num_blocks) {
  const int l = (int)blockIdx.y;
  reshape_one<ESZ>(keys[l], values[l], key_caches[l], value_caches[l], slots, num_tokens,
                   num_kv_heads, head_dim, block_size, num_blocks);
}

// Whole-block copies from (src_key, src_value) to (dst_key, dst_value); the
// pools may be the same (copy_blocks) or different, device or pinned host
// (swap_blocks).  Grid: x = 16-byte pieces of a block, y = pair, z = pool
// (0 key, 1 value).
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    char *dst_key, char *dst_value, const char *src_key, const char *src_value,
    const int64_t *__restrict__ pairs, int64_t block_bytes, int64_t src_blocks,
    int64_t dst_blocks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.y];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.y + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const char *sp = blockIdx.z == 0 ? src_key : src_value;
  char *dp = blockIdx.z == 0 ? dst_key : dst_value;
  const u32x4 *s = reinterpret_cast<const u32x4 *>(sp + src * block_bytes);
  u32x4 *d = reinterpret_cast<u32x4 *>(dp + dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    d[i] = s[i];
}

// copy_blocks over every layer: grid.z = 2 * layer + pool.
__global__ __launch_bounds__(256) void copy_blocks_layers_kernel(
    char *const *key_caches, char *const *value_caches, const int64_t *__restrict__ pairs,
    int64_t block_bytes, int64_t num_blocks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.y];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.y + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int l = (int)blockIdx.z >> 1;
  char *pool = (blockIdx.z & 1) ? value_caches[l] : key_caches[l];
  const u32x4 *s = reinterpret_cast<const u32x4 *>(pool + src * block_bytes);
  u32x4 *d = reinterpret_cast<u32x4 *>(pool + dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    d[i] = s[i];
}

}  // namespace

int launch_reshape_and_cache_layers(const void *const *keys, const void *const *values,
                                    void *const *key_caches, void *const *value_caches,
                                    int32_t num_layers, const int64_t *slots, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int64_t num_blocks, int32_t elem_bytes, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t threads = (int64_t)num_tokens * num_kv_heads * (head_dim * elem_bytes / 16);
  if (threads == 0 || num_layers == 0) return (int)hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX || num_layers > 65535) return (int)hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks, (unsigned)num_layers);
  const char *const *k = reinterpret_cast<const char *const *>(keys);
  const char *const *v = reinterpret_cast<const char *const *>(values);
  char *const *kc = reinterpret_cast<char *const *>(key_caches);
  char *const *vc = reinterpret_cast<char *const *>(value_caches);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(reshape_and_cache_layers_kernel<4>, grid, dim3(256), 0, st, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  else
    hipLaunchKernelGGL(reshape_and_cache_layers_kernel<2>, grid, dim3(256), 0, st, k, v, kc, vc,
                       slots, num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  return (int)hipGetLastError();
}

int launch_copy_blocks_layers(void *const *key_caches, void *const *value_caches,
                              int32_t num_layers, const int64_t *pairs, int32_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (num_layers > 32767) return (int)hipErrorInvalidConfiguration;
  const int64_t pieces = block_bytes / 16;
  const int64_t gx64 = (pieces + 255) / 256;
  const unsigned gx = (unsigned)(gx64 < 64 ? gx64 : 64);
  for (int32_t first = 0; first < num_pairs; first += 65535) {
    const int32_t n = num_pairs - first < 65535 ? num_pairs - first : 65535;
    hipLaunchKernelGGL(copy_blocks_layers_kernel, dim3(gx, (unsigned)n, 2 * (unsigned)num_layers),
                       dim3(256), 0, st, reinterpret_cast<char *const *>(key_caches),
                       reinterpret_cast<char *const *>(value_caches), pairs + 2 * (int64_t)first,
                       block_bytes, num_blocks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipSuccess;
}

int launch_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slots, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, int32_t elem_bytes, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t threads = (int64_t)num_tokens * num_kv_heads * (head_dim * elem_bytes / 16);
  if (threads == 0) return (int)hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return (int)hipErrorInvalidConfiguration;
  const char *k = static_cast<const char *>(key);
  const char *v = static_cast<const char *>(value);
  char *kc = static_cast<char *>(key_cache);
  char *vc = static_cast<char *>(value_cache);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(reshape_and_cache_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, k,
                       v, kc, vc, slots, num_tokens, num_kv_heads, head_dim, block_size,
                       num_blocks);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, k,
                       v, kc, vc, slots, num_tokens, num_kv_heads, head_dim, block_size,
                       num_blocks);
  return (int)hipGetLastError();
}

int launch_copy_blocks(void *dst_key, void *dst_value, const void *src_key,
                       const void *src_value, const int64_t *pairs, int32_t num_pairs,
                       int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks,
                       void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t pieces = block_bytes / 16;
  const int64_t gx64 = (pieces + 255) / 256;
  const unsigned gx = (unsigned)(gx64 < 64 ? gx64 : 64);
  // grid.y is limited to 65535: launch the pairs in chunks.
  for (int32_t first = 0; first < num_pairs; first += 65535) {
    const int32_t n = num_pairs - first < 65535 ? num_pairs - first : 65535;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, (unsigned)n, 2), dim3(256), 0, st,
                       static_cast<char *>(dst_key), static_cast<char *>(dst_value),
                       static_cast<const char *>(src_key), static_cast<const char *>(src_value),
                       pairs + 2 * (int64_t)first, block_bytes, src_blocks, dst_blocks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipSuccess;
}

}  // namespace pa
