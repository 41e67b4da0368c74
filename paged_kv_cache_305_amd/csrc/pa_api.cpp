// C ABI of the kernel calls: argument checks, workspace layout, optional deep
// validation (PA_VALIDATE=1), then the launches.  Nothing here synchronises
// unless PA_VALIDATE=1 asks for the integer inputs on the host.
#include <hip/hip_runtime_api.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(pa_dtype t) { return t == PA_FP32 ? 4 : (t == PA_BF16 ? 2 : 0); }

bool deep_validation() {
  const char *v = getenv("PA_VALIDATE");
  return v && v[0] == '1';
}

pa_status hip_fail(const char *what, int err) {
  return pa_fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

template <typename T>
pa_status to_host(std::vector<T> &dst, const T *src, size_t n, void *stream) {
  dst.resize(n);
  if (n == 0) return PA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // hipMemcpyDefault: src may be device memory or pinned host memory.
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDefault, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e == hipSuccess ? PA_OK : hip_fail("PA_VALIDATE copy", (int)e);
}

// True when the device can read and write p directly: device memory, or
// pinned host memory mapped at the same address (hipHostMalloc on ROCm).
// Pageable host memory -- which a kernel access would fault on -- is refused.
bool device_addressable(const void *p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the error the query leaves behind
    return false;
  }
  if (at.type == hipMemoryTypeDevice) return true;
  return at.type == hipMemoryTypeHost && at.devicePointer == p;
}

// Tracing hook (pa_set_timing_events): per calling thread, so that a thread
// that times its calls never adds events to another thread's.
thread_local void *g_ev_main[2] = {nullptr, nullptr};
thread_local void *g_ev_merge[2] = {nullptr, nullptr};

// Per-XCD tile shares of the balanced split.  Measured on MI355X: waves on
// even-numbered XCDs finish a fixed share 10-15% sooner than waves on
// odd-numbered ones, so equal shares leave the even XCDs idle at the end.
// A sweep of the even weight over 100..130 on two GPUs put the best
// decode time at 115 for both the 7B- and 70B-shaped batches.
constexpr int32_t kDefaultXcdWeights[8] = {115, 100, 115, 100, 115, 100, 115, 100};
// Process-wide; a setting is replaced and read as a whole under the mutex,
// so a call never mixes two settings.
std::mutex g_weights_mutex;
int32_t g_xcd_weights[8] = {115, 100, 115, 100, 115, 100, 115, 100};

int32_t partitions_for(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0) return 1;
  const int32_t n = (int32_t)(((int64_t)max_context_len + partition_size - 1) / partition_size);
  return n > 0 ? n : 1;
}

// Most waves a balanced launch may use on the current device: 32 per
// compute unit (the wave slots of a gfx950 CU).  0 if no device answers.
int32_t balanced_wave_bound() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus * 32;
}

// Partial rows a call needs (0: it writes every output row directly).  A
// balanced call is sized for the largest plan it can take on this device.
size_t partial_rows(int32_t num_seqs, const pa::HeadUnits &hu, int32_t max_context_len,
                    int32_t partition_size, int32_t wave_bound) {
  if (partition_size < 0) {
    pa::DecodeArgs a{};
    a.num_seqs = num_seqs;
    a.max_context_len = max_context_len;
    a.max_waves = wave_bound;
    a.flags = PA_DECODE_KV_REUSED;   // rows do not depend on the split; take the widest
    return pa::balanced_plan(a, hu.units, wave_bound).rows * hu.gu;
  }
  const int32_t parts = partitions_for(max_context_len, partition_size);
  if (parts <= 1) return 0;
  return (size_t)num_seqs * hu.units * parts * hu.gu;
}

}  // namespace

namespace pa {

void balance_weights(int32_t out[8]) {
  std::lock_guard<std::mutex> lock(g_weights_mutex);
  for (int i = 0; i < 8; ++i) out[i] = g_xcd_weights[i];
}

WorkspaceLayout workspace_layout(size_t rows, int32_t head_dim, size_t segments, size_t waves,
                                 size_t prefix_rows) {
  WorkspaceLayout w{rows, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (rows == 0 && prefix_rows == 0) return w;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.sum_off = up(rows * sizeof(float));
  w.acc_off = w.sum_off + up(rows * sizeof(float));
  w.seg_off = w.acc_off + up(rows * (size_t)head_dim * sizeof(float));
  w.cnt_off = w.seg_off + up(segments * 2 * sizeof(int32_t));
  w.wave_off = w.cnt_off + up(segments * sizeof(int32_t));
  w.pf_max_off = w.wave_off + up(waves * sizeof(int32_t));
  w.pf_sum_off = w.pf_max_off + up(prefix_rows * sizeof(float));
  w.pf_acc_off = w.pf_sum_off + up(prefix_rows * sizeof(float));
  w.total = w.pf_acc_off + up(prefix_rows * (size_t)head_dim * sizeof(float));
  return w;
}

PrefixPlan prefix_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t prefix_len, int cus) {
  PrefixPlan pl{0, 0, 0, 0, 0};
  if (prefix_len <= 0 || num_seqs <= 0 || num_kv_heads <= 0) return pl;
  const int tiles = prefix_len / 16;
  pl.rows = num_seqs * (num_q_heads / num_kv_heads);
  pl.row_blocks = (pl.rows + 16 * kPrefixRowTiles - 1) / (16 * kPrefixRowTiles);
  const int64_t per_chunk = (int64_t)pl.row_blocks * num_kv_heads;
  int64_t chunks = ((int64_t)cus * kPrefixWavesPerCU + per_chunk - 1) / per_chunk;
  if (chunks < 1) chunks = 1;
  if (chunks > tiles) chunks = tiles;
  pl.chunk_tiles = (int)((tiles + chunks - 1) / chunks);
  pl.chunks = (tiles + pl.chunk_tiles - 1) / pl.chunk_tiles;
  pl.partial_rows = (size_t)pl.chunks * num_kv_heads * pl.rows;
  return pl;
}

}  // namespace pa

extern "C" {

pa_status pa_set_balance_weights(const int32_t *weights, int32_t n) {
  pa_clear_error();
  if (weights == nullptr) {
    std::lock_guard<std::mutex> lock(g_weights_mutex);
    for (int i = 0; i < 8; ++i) g_xcd_weights[i] = kDefaultXcdWeights[i];
    return PA_OK;
  }
  if (n != 8)
    return pa_fail(PA_ERR_INVALID_ARG, "pa_set_balance_weights: expected 8 weights, got %d", n);
  for (int i = 0; i < 8; ++i)
    if (weights[i] < 1 || weights[i] > 1000)
      return pa_fail(PA_ERR_INVALID_ARG, "pa_set_balance_weights: weight %d = %d outside [1, 1000]",
                     i, weights[i]);
  std::lock_guard<std::mutex> lock(g_weights_mutex);
  for (int i = 0; i < 8; ++i) g_xcd_weights[i] = weights[i];
  return PA_OK;
}

pa_status pa_set_timing_events(void *main_start, void *main_end, void *merge_start,
                               void *merge_end) {
  pa_clear_error();
  g_ev_main[0] = main_start;
  g_ev_main[1] = main_end;
  g_ev_merge[0] = merge_start;
  g_ev_merge[1] = merge_end;
  return PA_OK;
}

int32_t pa_resolve_partition(int32_t partition_size, int32_t max_context_len) {
  if (partition_size != PA_PARTITION_AUTO) return partition_size;
  return max_context_len <= PA_AUTO_WHOLE_MAX_LEN ? 0 : PA_PARTITION_BALANCED;
}

size_t pa_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_context_len, int32_t partition_size,
                                          pa_dtype kv_dtype) {
  partition_size = pa_resolve_partition(partition_size, max_context_len);
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_context_len < 0 ||
      elem_bytes(kv_dtype) == 0)
    return 0;
  const pa::HeadUnits hu = pa::head_units(num_q_heads, num_kv_heads, kv_dtype);
  const int32_t bound = partition_size < 0 ? balanced_wave_bound() : 0;
  if (partition_size < 0 && bound == 0) return 0;
  return pa::workspace_layout(
             partial_rows(num_seqs, hu, max_context_len, partition_size, bound), head_dim,
             partition_size < 0 ? (size_t)num_seqs * hu.units : 0,
             partition_size < 0 ? (size_t)bound : 0)
      .total;
}

}  // extern "C"

namespace {

// Shared by pa_paged_attention_decode (new_key == nullptr) and
// pa_paged_attention_decode_append.
pa_status decode_call(const char *fn, void *out, const void *query, const void *key_cache,
                      const void *value_cache, const void *new_key, const void *new_value,
                      const int64_t *slot_mapping, const int64_t *cow_src,
                      const int32_t *block_tables,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                      float scale, int32_t partition_size, pa_dtype kv_dtype, pa_dtype out_dtype,
                      uint32_t flags, void *workspace, size_t workspace_bytes, void *stream,
                      int32_t prefix_len = 0, bool own_scratch = false) {
  const bool appending = new_key != nullptr || new_value != nullptr || slot_mapping != nullptr;
  partition_size = pa_resolve_partition(partition_size, max_context_len);
  if (num_seqs < 0) return pa_fail(PA_ERR_INVALID_ARG, "%s: num_seqs < 0", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return pa_fail(PA_ERR_INVALID_ARG,
                   "%s: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn,
                   num_q_heads, num_kv_heads);
  if (elem_bytes(kv_dtype) == 0 || elem_bytes(out_dtype) == 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: dtypes must be PA_FP32 or PA_BF16", fn);
  if (head_dim != 64 && head_dim != 128)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", fn, head_dim);
  if (block_size != 16 && block_size != 32 && block_size != 64)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (supported: 16, 32, 64)", fn,
                   block_size);
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq and num_blocks must be positive",
                   fn);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return pa_fail(PA_ERR_INVALID_ARG,
                   "%s: max_context_len %d outside [0, max_blocks_per_seq * block_size = %lld]",
                   fn, max_context_len, (long long)max_blocks_per_seq * block_size);
  if (partition_size > 0 && partition_size % block_size != 0)
    return pa_fail(PA_ERR_INVALID_ARG,
                   "%s: partition_size %d must be negative (balanced), 0, or a positive "
                   "multiple of block_size %d", fn, partition_size, block_size);
  if ((flags & ~PA_DECODE_KV_REUSED) != 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
  if (prefix_len != 0) {
    if (kv_dtype != PA_BF16)
      return pa_fail(PA_ERR_UNSUPPORTED, "%s: a shared prefix needs bf16 K/V (MFMA)", fn);
    if (prefix_len < 0 || prefix_len % block_size != 0 || prefix_len > max_context_len)
      return pa_fail(PA_ERR_INVALID_ARG, "%s: prefix_len %d must be a positive multiple of "
                     "block_size %d and <= max_context_len %d", fn, prefix_len, block_size,
                     max_context_len);
  }
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return pa_fail(PA_ERR_INVALID_ARG, "%s: out, query and pools must be 16-byte aligned", fn);
  if (appending) {
    if (!new_key || !new_value || !slot_mapping)
      return pa_fail(PA_ERR_INVALID_ARG, "%s: new_key, new_value and slot_mapping are all "
                     "needed", fn);
    if (!aligned16(new_key) || !aligned16(new_value))
      return pa_fail(PA_ERR_INVALID_ARG, "%s: new_key and new_value must be 16-byte aligned", fn);
  } else if (cow_src) {
    return pa_fail(PA_ERR_INVALID_ARG, "%s: cow_src needs the new tokens (slot_mapping)", fn);
  }

  const int32_t parts = partitions_for(max_context_len, partition_size);
  const pa::HeadUnits hu = pa::head_units(num_q_heads, num_kv_heads, kv_dtype);
  const int32_t bound = partition_size < 0 ? balanced_wave_bound() : 0;
  if (partition_size < 0 && bound == 0)
    return pa_fail(PA_ERR_HIP, "%s: cannot query the current device", fn);
  const pa::PrefixPlan pf = pa::prefix_plan(num_seqs, num_q_heads, num_kv_heads, prefix_len,
                                            bound / 32);
  const pa::WorkspaceLayout ws = pa::workspace_layout(
      partial_rows(num_seqs, hu, max_context_len, partition_size, bound), head_dim,
      partition_size < 0 ? (size_t)num_seqs * hu.units : 0,
      partition_size < 0 ? (size_t)bound : 0, pf.partial_rows);
  if (own_scratch && ws.total > 0) {
    // The library's device array stands in for the caller's workspace.
    if (ws.total > pa::kNoAllocScratchBytes)
      return pa_fail(PA_ERR_INVALID_ARG, "%s: these sizes need %zu bytes of scratch; the "
                     "library's array holds %zu (use pa_paged_attention_decode_append with a "
                     "workspace)", fn, ws.total, pa::kNoAllocScratchBytes);
    const int e = pa::noalloc_scratch(&workspace);
    if (e != 0) return hip_fail(fn, e);
    workspace_bytes = pa::kNoAllocScratchBytes;
  }
  if (ws.total > 0) {
    if (!workspace || workspace_bytes < ws.total)
      return pa_fail(PA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, got %zu", fn,
                     ws.total, workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace & 255u) != 0)
      return pa_fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  }

  if (deep_validation()) {
    std::vector<int32_t> lens, tabs;
    pa_status s = to_host(lens, context_lens, (size_t)num_seqs, stream);
    if (s == PA_OK)
      s = to_host(tabs, block_tables, (size_t)num_seqs * max_blocks_per_seq, stream);
    if (s != PA_OK) return s;
    for (int32_t i = 0; i < num_seqs; ++i) {
      if (lens[i] < 0 || lens[i] > max_context_len)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: context_lens[%d] = %d outside [0, %d]", fn, i,
                       lens[i], max_context_len);
      const int32_t used = (lens[i] + block_size - 1) / block_size;
      for (int32_t j = 0; j < used; ++j) {
        const int32_t b = tabs[(size_t)i * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks)
          return pa_fail(PA_ERR_INVALID_ARG, "%s: block_tables[%d][%d] = %d outside [0, %lld)",
                         fn, i, j, b, (long long)num_blocks);
      }
    }
    if (prefix_len > 0) {
      // Every sequence holds the prefix, in the same blocks as sequence 0.
      for (int32_t i = 0; i < num_seqs; ++i) {
        if (lens[i] < prefix_len)
          return pa_fail(PA_ERR_INVALID_ARG, "%s: context_lens[%d] = %d < prefix_len %d", fn, i,
                         lens[i], prefix_len);
        for (int32_t j = 0; j < prefix_len / block_size; ++j)
          if (tabs[(size_t)i * max_blocks_per_seq + j] != tabs[(size_t)j])
            return pa_fail(PA_ERR_INVALID_ARG, "%s: block_tables[%d][%d] differs from sequence "
                           "0's prefix block", fn, i, j);
      }
    }
    if (appending) {
      // Each new token must sit at its sequence's last position.
      std::vector<int64_t> slots;
      s = to_host(slots, slot_mapping, (size_t)num_seqs, stream);
      if (s != PA_OK) return s;
      for (int32_t i = 0; i < num_seqs; ++i) {
        if (slots[i] < 0) continue;
        const int32_t pos = lens[i] - 1;
        const int64_t want =
            pos < 0 ? -1
                    : (int64_t)tabs[(size_t)i * max_blocks_per_seq + pos / block_size] *
                              block_size + pos % block_size;
        if (slots[i] != want)
          return pa_fail(PA_ERR_INVALID_ARG, "%s: slot_mapping[%d] = %lld is not the slot of "
                         "position context_lens - 1 (%lld)", fn, i, (long long)slots[i],
                         (long long)want);
        if (pos < prefix_len)
          return pa_fail(PA_ERR_INVALID_ARG, "%s: sequence %d appends at position %d, inside "
                         "the shared prefix", fn, i, pos);
      }
      if (cow_src) {
        // A copy source is a block other than the slot's, and a sequence
        // that writes a new token into a copy source in place writes it at
        // the same offset as the sequence copying it (they shared the
        // partly filled block, so they had the same length).
        std::vector<int64_t> src;
        s = to_host(src, cow_src, (size_t)num_seqs, stream);
        if (s != PA_OK) return s;
        std::unordered_map<int64_t, int64_t> slot_of_block;   // block -> slot written in it
        for (int32_t i = 0; i < num_seqs; ++i)
          if (slots[i] >= 0) slot_of_block[slots[i] / block_size] = slots[i];
        for (int32_t i = 0; i < num_seqs; ++i) {
          if (src[i] < 0) continue;
          if (slots[i] < 0 || src[i] >= num_blocks || src[i] == slots[i] / block_size)
            return pa_fail(PA_ERR_INVALID_ARG, "%s: cow_src[%d] = %lld needs a new token and "
                           "must be another block of the pool", fn, i, (long long)src[i]);
          const auto w = slot_of_block.find(src[i]);
          if (w != slot_of_block.end() && w->second % block_size != slots[i] % block_size)
            return pa_fail(PA_ERR_INVALID_ARG, "%s: cow_src[%d] = %lld is written at another "
                           "offset by this call", fn, i, (long long)src[i]);
        }
      }
    }
  }

  pa::DecodeArgs a;
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.new_key = new_key;
  a.new_value = new_value;
  a.slots = slot_mapping;
  a.cow_src = cow_src;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.partition_size = partition_size;
  a.num_partitions = parts;
  a.max_waves = bound;
  a.kv_dtype = kv_dtype;
  a.out_dtype = out_dtype;
  a.flags = flags;
  char *wsb = static_cast<char *>(workspace);
  a.ws_max = ws.total ? reinterpret_cast<float *>(wsb + ws.max_off) : nullptr;
  a.ws_sum = ws.total ? reinterpret_cast<float *>(wsb + ws.sum_off) : nullptr;
  a.ws_acc = ws.total ? reinterpret_cast<float *>(wsb + ws.acc_off) : nullptr;
  a.seg_units = ws.total ? reinterpret_cast<int32_t *>(wsb + ws.seg_off) : nullptr;
  a.seg_cnt = ws.total ? reinterpret_cast<int32_t *>(wsb + ws.cnt_off) : nullptr;
  a.wave_segs = ws.total ? reinterpret_cast<int32_t *>(wsb + ws.wave_off) : nullptr;
  a.prefix_len = prefix_len;
  a.pf_max = pf.partial_rows ? reinterpret_cast<float *>(wsb + ws.pf_max_off) : nullptr;
  a.pf_sum = pf.partial_rows ? reinterpret_cast<float *>(wsb + ws.pf_sum_off) : nullptr;
  a.pf_acc = pf.partial_rows ? reinterpret_cast<float *>(wsb + ws.pf_acc_off) : nullptr;
  pa::balance_weights(a.xcd_weights);
  a.ev_main_start = g_ev_main[0];
  a.ev_main_end = g_ev_main[1];
  a.ev_merge_start = g_ev_merge[0];
  a.ev_merge_end = g_ev_merge[1];
  const int e = pa::launch_decode(a, stream);
  return e == 0 ? PA_OK : hip_fail(fn, e);
}

}  // namespace

extern "C" {

pa_status pa_paged_attention_decode(void *out, const void *query, const void *key_cache,
                                    const void *value_cache, const int32_t *block_tables,
                                    const int32_t *context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int64_t num_blocks, int32_t max_context_len, float scale,
                                    int32_t partition_size, pa_dtype kv_dtype, pa_dtype out_dtype,
                                    uint32_t flags, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  pa_clear_error();
  return decode_call("pa_paged_attention_decode", out, query, key_cache, value_cache, nullptr,
                     nullptr, nullptr, nullptr, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, kv_dtype, out_dtype, flags,
                     workspace, workspace_bytes, stream);
}

pa_status pa_paged_attention_decode_prefix(void *out, const void *query, void *key_cache,
                                           void *value_cache, const void *new_key,
                                           const void *new_value, const int64_t *slot_mapping,
                                           const int64_t *cow_src, const int32_t *block_tables,
                                           const int32_t *context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t max_blocks_per_seq, int64_t num_blocks,
                                           int32_t max_context_len, float scale,
                                           int32_t prefix_len, pa_dtype kv_dtype,
                                           pa_dtype out_dtype, uint32_t flags, void *workspace,
                                           size_t workspace_bytes, void *stream) {
  pa_clear_error();
  const char *fn = "pa_paged_attention_decode_prefix";
  if (prefix_len <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: prefix_len must be positive", fn);
  return decode_call(fn, out, query, key_cache, value_cache, new_key, new_value, slot_mapping,
                     cow_src, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                     PA_PARTITION_BALANCED, kv_dtype, out_dtype, flags, workspace,
                     workspace_bytes, stream, prefix_len);
}

size_t pa_paged_attention_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim,
                                                 int32_t max_context_len, int32_t prefix_len,
                                                 pa_dtype kv_dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_context_len < 0 ||
      prefix_len <= 0 || kv_dtype != PA_BF16)
    return 0;
  const pa::HeadUnits hu = pa::head_units(num_q_heads, num_kv_heads, kv_dtype);
  const int32_t bound = balanced_wave_bound();
  if (bound == 0) return 0;
  const pa::PrefixPlan pf = pa::prefix_plan(num_seqs, num_q_heads, num_kv_heads, prefix_len,
                                            bound / 32);
  return pa::workspace_layout(partial_rows(num_seqs, hu, max_context_len, -1, bound), head_dim,
                              (size_t)num_seqs * hu.units, (size_t)bound, pf.partial_rows)
      .total;
}

pa_status pa_paged_attention_decode_append(
    void *out, const void *query, void *key_cache, void *value_cache, const void *new_key,
    const void *new_value, const int64_t *slot_mapping, const int64_t *cow_src,
    const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, pa_dtype kv_dtype,
    pa_dtype out_dtype, uint32_t flags, void *workspace, size_t workspace_bytes, void *stream) {
  pa_clear_error();
  return decode_call("pa_paged_attention_decode_append", out, query, key_cache, value_cache,
                     new_key, new_value, slot_mapping, cow_src, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, scale, partition_size, kv_dtype, out_dtype,
                     flags, workspace, workspace_bytes, stream);
}

pa_status pa_paged_attention_decode_noalloc(
    void *out, const void *query, void *key_cache, void *value_cache, const void *new_key,
    const void *new_value, const int64_t *slot_mapping, const int64_t *cow_src,
    const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, pa_dtype kv_dtype, pa_dtype out_dtype, uint32_t flags,
    void *stream) {
  pa_clear_error();
  return decode_call("pa_paged_attention_decode_noalloc", out, query, key_cache, value_cache,
                     new_key, new_value, slot_mapping, cow_src, block_tables, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size,
                     kv_dtype, out_dtype, flags, nullptr, 0, stream, 0, true);
}

pa_status pa_reshape_and_cache(const void *key, const void *value, void *key_cache,
                               void *value_cache, const int64_t *slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, pa_dtype dtype, void *stream) {
  pa_clear_error();
  const char *fn = "pa_reshape_and_cache";
  const int esz = elem_bytes(dtype);
  if (esz == 0) return pa_fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_FP32 or PA_BF16", fn);
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: sizes must be positive (num_tokens >= 0)", fn);
  if ((head_dim * esz) % 16 != 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: head_dim * element size must be a multiple of 16",
                   fn);
  if (block_size % 16 != 0)   // values are stored in 16-token groups
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: block_size %d is not a multiple of 16", fn,
                   block_size);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return pa_fail(PA_ERR_INVALID_ARG, "%s: key, value and pools must be 16-byte aligned", fn);
  if (deep_validation()) {
    std::vector<int64_t> slots;
    pa_status s = to_host(slots, slot_mapping, (size_t)num_tokens, stream);
    if (s != PA_OK) return s;
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (slots[i] < 0) continue;
      if (slots[i] >= num_blocks * block_size)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: slot_mapping[%d] = %lld >= %lld", fn, i,
                       (long long)slots[i], (long long)(num_blocks * block_size));
      if (!seen.insert(slots[i]).second)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: slot %lld repeats", fn, (long long)slots[i]);
    }
  }
  const int e = pa::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
                                             num_tokens, num_kv_heads, head_dim, block_size,
                                             num_blocks, esz, stream);
  return e == 0 ? PA_OK : hip_fail(fn, e);
}

namespace {

// PA_VALIDATE: every per-layer pointer must be 16-byte aligned device memory.
pa_status check_layer_pointers(const char *fn, const void *const *arr, int32_t n,
                               const char *what, void *stream) {
  std::vector<uintptr_t> host;
  pa_status s = to_host(host, reinterpret_cast<const uintptr_t *>(arr), (size_t)n, stream);
  if (s != PA_OK) return s;
  for (int32_t l = 0; l < n; ++l) {
    const void *p = reinterpret_cast<const void *>(host[(size_t)l]);
    if (!p || !aligned16(p) || !device_addressable(p))
      return pa_fail(PA_ERR_INVALID_ARG, "%s: %s[%d] is not 16-byte aligned device memory", fn,
                     what, l);
  }
  return PA_OK;
}

}  // namespace

pa_status pa_reshape_and_cache_layers(const void *const *keys, const void *const *values,
                                      void *const *key_caches, void *const *value_caches,
                                      int32_t num_layers, const int64_t *slot_mapping,
                                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                                      void *stream) {
  pa_clear_error();
  const char *fn = "pa_reshape_and_cache_layers";
  const int esz = elem_bytes(dtype);
  if (esz == 0) return pa_fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_FP32 or PA_BF16", fn);
  if (num_layers < 0 || num_layers > 65535 || num_tokens < 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: bad sizes (num_layers in [0, 65535])", fn);
  if ((head_dim * esz) % 16 != 0 || block_size % 16 != 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: head_dim * element size and block_size must be "
                   "multiples of 16", fn);
  if (num_tokens == 0 || num_layers == 0) return PA_OK;
  if (!keys || !values || !key_caches || !value_caches || !slot_mapping)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (deep_validation()) {
    pa_status s = check_layer_pointers(fn, keys, num_layers, "keys", stream);
    if (s == PA_OK) s = check_layer_pointers(fn, values, num_layers, "values", stream);
    if (s == PA_OK)
      s = check_layer_pointers(fn, (const void *const *)key_caches, num_layers, "key_caches",
                               stream);
    if (s == PA_OK)
      s = check_layer_pointers(fn, (const void *const *)value_caches, num_layers,
                               "value_caches", stream);
    if (s != PA_OK) return s;
    std::vector<int64_t> slots;
    s = to_host(slots, slot_mapping, (size_t)num_tokens, stream);
    if (s != PA_OK) return s;
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (slots[i] < 0) continue;
      if (slots[i] >= num_blocks * block_size || !seen.insert(slots[i]).second)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: slot_mapping[%d] = %lld out of range or "
                       "repeated", fn, i, (long long)slots[i]);
    }
  }
  const int e = pa::launch_reshape_and_cache_layers(keys, values, key_caches, value_caches,
                                                    num_layers, slot_mapping, num_tokens,
                                                    num_kv_heads, head_dim, block_size,
                                                    num_blocks, esz, stream);
  return e == 0 ? PA_OK : hip_fail(fn, e);
}

pa_status pa_copy_blocks_layers(void *const *key_caches, void *const *value_caches,
                                int32_t num_layers, const int64_t *block_mapping,
                                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                                void *stream) {
  pa_clear_error();
  const char *fn = "pa_copy_blocks_layers";
  const int esz = elem_bytes(dtype);
  if (esz == 0) return pa_fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_FP32 or PA_BF16", fn);
  if (num_layers < 0 || num_layers > 32767 || num_pairs < 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: bad sizes (num_layers in [0, 32767])", fn);
  const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * esz;
  if (block_bytes % 16 != 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: block bytes must be a multiple of 16", fn);
  if (num_pairs == 0 || num_layers == 0) return PA_OK;
  if (!key_caches || !value_caches || !block_mapping)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (deep_validation()) {
    pa_status s = check_layer_pointers(fn, (const void *const *)key_caches, num_layers,
                                       "key_caches", stream);
    if (s == PA_OK)
      s = check_layer_pointers(fn, (const void *const *)value_caches, num_layers,
                               "value_caches", stream);
    if (s != PA_OK) return s;
    std::vector<int64_t> m;
    s = to_host(m, block_mapping, (size_t)num_pairs * 2, stream);
    if (s != PA_OK) return s;
    std::unordered_set<int64_t> srcs, dsts;
    for (int32_t i = 0; i < num_pairs; ++i) {
      for (int k = 0; k < 2; ++k)
        if (m[2 * i + k] < 0 || m[2 * i + k] >= num_blocks)
          return pa_fail(PA_ERR_INVALID_ARG, "%s: block_mapping[%d][%d] out of range", fn, i, k);
      srcs.insert(m[2 * i]);
      if (!dsts.insert(m[2 * i + 1]).second)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: destination %lld repeats", fn,
                       (long long)m[2 * i + 1]);
    }
    for (int64_t d : dsts)
      if (srcs.count(d))
        return pa_fail(PA_ERR_INVALID_ARG, "%s: block %lld is both a source and a destination",
                       fn, (long long)d);
  }
  const int e = pa::launch_copy_blocks_layers(key_caches, value_caches, num_layers,
                                              block_mapping, num_pairs, block_bytes, num_blocks,
                                              stream);
  return e == 0 ? PA_OK : hip_fail(fn, e);
}

pa_status pa_copy_blocks(void *key_cache, void *value_cache, const int64_t *block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype, void *stream) {
  pa_clear_error();
  const char *fn = "pa_copy_blocks";
  const int esz = elem_bytes(dtype);
  if (esz == 0) return pa_fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_FP32 or PA_BF16", fn);
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: sizes must be positive (num_pairs >= 0)", fn);
  const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * esz;
  if (block_bytes % 16 != 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: block bytes must be a multiple of 16", fn);
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_mapping)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned16(key_cache) || !aligned16(value_cache))
    return pa_fail(PA_ERR_INVALID_ARG, "%s: pools must be 16-byte aligned", fn);
  if (deep_validation()) {
    std::vector<int64_t> m;
    pa_status s = to_host(m, block_mapping, (size_t)num_pairs * 2, stream);
    if (s != PA_OK) return s;
    std::unordered_set<int64_t> srcs, dsts;
    for (int32_t i = 0; i < num_pairs; ++i) {
      for (int k = 0; k < 2; ++k)
        if (m[2 * i + k] < 0 || m[2 * i + k] >= num_blocks)
          return pa_fail(PA_ERR_INVALID_ARG, "%s: block_mapping[%d][%d] = %lld outside [0, %lld)",
                         fn, i, k, (long long)m[2 * i + k], (long long)num_blocks);
      srcs.insert(m[2 * i]);
      if (!dsts.insert(m[2 * i + 1]).second)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: destination %lld repeats", fn,
                       (long long)m[2 * i + 1]);
    }
    for (int64_t d : dsts)
      if (srcs.count(d))
        return pa_fail(PA_ERR_INVALID_ARG, "%s: block %lld is both a source and a destination",
                       fn, (long long)d);
  }
  const int e = pa::launch_copy_blocks(key_cache, value_cache, key_cache, value_cache,
                                       block_mapping, num_pairs, block_bytes, num_blocks,
                                       num_blocks, stream);
  return e == 0 ? PA_OK : hip_fail(fn, e);
}

pa_status pa_swap_blocks(void *dst_key_cache, void *dst_value_cache, const void *src_key_cache,
                         const void *src_value_cache, const int64_t *block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t src_num_blocks, int64_t dst_num_blocks,
                         pa_dtype dtype, void *stream) {
  pa_clear_error();
  const char *fn = "pa_swap_blocks";
  const int esz = elem_bytes(dtype);
  if (esz == 0) return pa_fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_FP32 or PA_BF16", fn);
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      src_num_blocks <= 0 || dst_num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: sizes must be positive (num_pairs >= 0)", fn);
  const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * esz;
  if (block_bytes % 16 != 0)
    return pa_fail(PA_ERR_UNSUPPORTED, "%s: block bytes must be a multiple of 16", fn);
  if (num_pairs == 0) return PA_OK;
  if (!dst_key_cache || !dst_value_cache || !src_key_cache || !src_value_cache || !block_mapping)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned16(dst_key_cache) || !aligned16(dst_value_cache) || !aligned16(src_key_cache) ||
      !aligned16(src_value_cache))
    return pa_fail(PA_ERR_INVALID_ARG, "%s: pools must be 16-byte aligned", fn);
  const void *ptrs[5] = {dst_key_cache, dst_value_cache, src_key_cache, src_value_cache,
                         block_mapping};
  const char *names[5] = {"dst_key_cache", "dst_value_cache", "src_key_cache",
                          "src_value_cache", "block_mapping"};
  for (int i = 0; i < 5; ++i)
    if (!device_addressable(ptrs[i]))
      return pa_fail(PA_ERR_INVALID_ARG, "%s: %s is neither device memory nor pinned host "
                     "memory the device can address", fn, names[i]);
  if (deep_validation()) {
    std::vector<int64_t> m;
    pa_status s = to_host(m, block_mapping, (size_t)num_pairs * 2, stream);
    if (s != PA_OK) return s;
    std::unordered_set<int64_t> dsts;
    for (int32_t i = 0; i < num_pairs; ++i) {
      if (m[2 * i] < 0 || m[2 * i] >= src_num_blocks || m[2 * i + 1] < 0 ||
          m[2 * i + 1] >= dst_num_blocks)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: pair %d = (%lld, %lld) outside the pools", fn,
                       i, (long long)m[2 * i], (long long)m[2 * i + 1]);
      if (!dsts.insert(m[2 * i + 1]).second)
        return pa_fail(PA_ERR_INVALID_ARG, "%s: destination %lld repeats", fn,
                       (long long)m[2 * i + 1]);
    }
  }
  const int e = pa::launch_copy_blocks(dst_key_cache, dst_value_cache, src_key_cache,
                                       src_value_cache, block_mapping, num_pairs, block_bytes,
                                       src_num_blocks, dst_num_blocks, stream);
  return e == 0 ? PA_OK : hip_fail(fn, e);
}

}  // extern "C"
