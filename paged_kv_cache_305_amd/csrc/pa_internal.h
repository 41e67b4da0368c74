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
  // Appending variant: new token per sequence and its slot (null otherwise).
  const void *new_key, *new_value;
  const int64_t *slots;
  const int64_t *cow_src;   // copy-on-write inside the launch (null: none)
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int64_t num_blocks;
  int32_t max_context_len;
  float scale;
  int32_t partition_size;   // > 0 fixed partitions, 0 whole segments, < 0 balanced
  int32_t num_partitions;   // fixed mode: partitions of the longest sequence
  int32_t max_waves;        // balanced mode: upper bound of the wave count
  pa_dtype kv_dtype, out_dtype;
  uint32_t flags;           // PA_DECODE_* bits
  float *ws_max, *ws_sum, *ws_acc;  // split partials, null when every row is written whole
  int32_t *seg_units;               // balanced mode: 2 ints per (sequence, head unit)
  int32_t *seg_cnt;                 // balanced mode: 1 int per (sequence, head unit)
  int32_t *wave_segs;               // balanced mode: 1 int per wave
  int32_t prefix_len;               // shared prefix tokens (0: none)
  float *pf_max, *pf_sum, *pf_acc;  // shared-prefix partials
  int32_t xcd_weights[8];           // balanced mode: relative tile share per XCD
  // Optional hipEvent_t pairs stamped with the main and merge kernels' own
  // start and end (pa_set_timing_events); null: none.
  void *ev_main_start, *ev_main_end, *ev_merge_start, *ev_merge_end;
};

// How query heads are grouped into head units (one wave's worth of heads).
struct HeadUnits {
  bool mfma;       // bf16 KV with G >= 2: MFMA body, one KV head per unit
  int head_tiles;  // 16-head tiles per KV head (MFMA), else 1
  int units;       // head units per sequence
  int gu;          // partial rows per piece: heads one unit holds
};
HeadUnits head_units(int32_t num_q_heads, int32_t num_kv_heads, pa_dtype kv_dtype);

// Balanced split: one contiguous, per-XCD weighted range of tiles per wave.
struct BalancedPlan {
  int waves, xsplit;
  int64_t id_stride;   // piece ids per sub-problem
  size_t rows;         // pieces in all sub-problems (partial rows = rows * gu)
};
// `resident`: waves the device holds at once for the kernel.
BalancedPlan balanced_plan(const DecodeArgs &a, int units, int resident);

// Shared prefix: its 16-token tiles split into `chunks` runs of
// `chunk_tiles`, one wave per (row block of kPrefixRowTiles * 16 rows,
// chunk, KV head); partial rows = chunks * num_kv_heads * rows.
#ifndef PA_PREFIX_ROW_TILES
#define PA_PREFIX_ROW_TILES 2
#endif
#ifndef PA_PREFIX_WAVES_PER_CU
#define PA_PREFIX_WAVES_PER_CU 3
#endif
constexpr int kPrefixRowTiles = PA_PREFIX_ROW_TILES;     // 16-row tiles per wave
constexpr int kPrefixWavesPerCU = PA_PREFIX_WAVES_PER_CU;
struct PrefixPlan {
  int chunks, chunk_tiles, rows, row_blocks;
  size_t partial_rows;
};
PrefixPlan prefix_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t prefix_len, int cus);

// Current per-XCD weights (pa_set_balance_weights).
void balance_weights(int32_t out[8]);

// Workspace carve-up shared by the size query and the decode call: `rows`
// partial rows, each a base-2 max, a sum and head_dim unnormalised outputs,
// then `segments` pairs of int32 (balanced mode's first/last owning wave).
struct WorkspaceLayout {
  size_t rows, max_off, sum_off, acc_off, seg_off, cnt_off, wave_off, pf_max_off, pf_sum_off,
      pf_acc_off, total;
};
// segments: balanced split's (sequence, head unit) pairs (2 + 1 ints each);
// waves: its most waves (1 int each).
WorkspaceLayout workspace_layout(size_t rows, int32_t head_dim, size_t segments,
                                 size_t waves, size_t prefix_rows = 0);

// The library's own device scratch for pa_paged_attention_decode_noalloc:
// a file-scope device array of this many bytes in pa_decode.hip, one copy
// per GPU, held until the process ends.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Device address of that array on the current device, looked up with
// hipGetSymbolAddress on the first call per device and kept; returns
// hipError_t as int.
int noalloc_scratch(void **ptr);

// Kernel launchers (pa_decode.hip, pa_cache.hip); they return hipError_t as int.
int launch_decode(const DecodeArgs &a, void *stream);
int launch_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slots, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, int32_t elem_bytes, void *stream);
int launch_reshape_and_cache_layers(const void *const *keys, const void *const *values,
                                    void *const *key_caches, void *const *value_caches,
                                    int32_t num_layers, const int64_t *slots, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int64_t num_blocks, int32_t elem_bytes, void *stream);
int launch_copy_blocks_layers(void *const *key_caches, void *const *value_caches,
                              int32_t num_layers, const int64_t *pairs, int32_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, void *stream);
int launch_copy_blocks(void *dst_key, void *dst_value, const void *src_key,
                       const void *src_value, const int64_t *pairs, int32_t num_pairs,
                       int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks, void *stream);

}  // namespace pa
