// Internal declarations shared by the library's translation units.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

// Record a formatted message for pa_last_error() and return `code`.
pa_status pa_fail(pa_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void pa_clear_error();

namespace pa {

// Shapes of one decode call, validated by the ABI layer before any launch.
struct DecodeArgs {
  void *out;
  const void *query, *key_cache, *value_cache;
  const int32_t *block_tables, *context_lens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int64_t num_blocks;
  int32_t max_context_len;
  float scale;
  int32_t partition_size;   // 0: one partition per sequence
  int32_t num_partitions;   // partitions of the longest sequence (grid extent)
  pa_dtype kv_dtype, out_dtype;
  float *ws_max, *ws_sum, *ws_acc;  // split-K partials, null when num_partitions <= 1
  void *ev_before_main, *ev_after_main;  // optional hipEvent_t pair around the main kernel
};

// Workspace carve-up shared by the size query and the decode call.
struct WorkspaceLayout {
  size_t max_off, sum_off, acc_off, total;
};
WorkspaceLayout workspace_layout(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t num_partitions);

// Kernel launchers (pa_decode.hip, pa_cache.hip); they return hipError_t as int.
int launch_decode(const DecodeArgs &a, void *stream);
int launch_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slots, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, int32_t elem_bytes, void *stream);
int launch_copy_blocks(void *key_cache, void *value_cache, const int64_t *pairs,
                       int32_t num_pairs, int64_t block_bytes, int64_t num_blocks, void *stream);

}  // namespace pa
