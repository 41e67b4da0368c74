/*
 * pagedattn.h -- C ABI of libpagedattn.so: paged decode attention for MI355X
 * (gfx950) and the block management around it.
 *
 * The method (dmarx anthology note-023 "Method"; crackai.dev summary of Kwon
 * et al., "How It Works"): each sequence's KV cache is cut into fixed-size
 * blocks of block_size tokens, a per-sequence block table maps logical block
 * index to physical block, and the attention kernel gathers K/V from those
 * scattered physical blocks.  A block is taken only when a sequence's growth
 * needs one and returned when the sequence ends; sequences with a common
 * prefix point at the same blocks, and a shared block is duplicated only
 * when one of its sharers writes to it.
 *
 * Conventions
 *  - Every call returns pa_status; PA_OK is 0, errors are negative.  On an
 *    error nothing is launched and no state changes; pa_last_error() gives a
 *    message for the calling thread.  No exception crosses this boundary.
 *  - Device pointers are caller-owned (for example PyTorch tensors),
 *    contiguous, and 16-byte aligned.  The library never allocates or frees
 *    device memory.
 *  - Kernel calls are asynchronous on `stream` (a hipStream_t passed as
 *    void*, NULL = the default stream) and never synchronise.
 *  - Cheap scalar checks always run.  With the environment variable
 *    PA_VALIDATE=1 the kernel calls also copy their integer inputs to the
 *    host (synchronously) and check every table entry, slot and pair.
 *
 * Pool layout (one layer; K and V in separate pools), x = 16 / element size:
 *    key   pool [num_blocks][num_kv_heads][head_dim / x][block_size][x]
 *    value pool [num_blocks][num_kv_heads][block_size / 16][head_dim][16]
 *  so every (block, KV head) chunk is block_size * head_dim contiguous
 *  elements; keys keep 16-byte runs of one token's features, values keep
 *  each feature's tokens together in groups of 16 (one group per 16-token
 *  tile the kernels read).  A slot is physical_block * block_size +
 *  offset_in_block.
 *
 * Allocator handles are library-owned host objects, not thread-safe, and
 * destroyed by the caller.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
#define PA_OK 0
#define PA_ERR_INVALID_ARG (-1)   /* bad pointer, size, range or alignment   */
#define PA_ERR_UNSUPPORTED (-2)   /* valid but not built: head_dim, block_size */
#define PA_ERR_OUT_OF_BLOCKS (-3) /* allocator pool exhausted                 */
#define PA_ERR_UNKNOWN_SEQ (-4)   /* allocator: no such sequence id           */
#define PA_ERR_HIP (-5)           /* a HIP runtime call failed                */

typedef int32_t pa_dtype;
#define PA_FP32 0
#define PA_BF16 1

/* partition_size of pa_paged_attention_decode: balanced split. */
#define PA_PARTITION_BALANCED (-1)
/* partition_size of pa_paged_attention_decode: one pass per (sequence, head)
 * when max_context_len <= PA_AUTO_WHOLE_MAX_LEN, else the balanced split
 * (pa_resolve_partition).  Below that length a single wave's chain is at most
 * 16 tiles, and skipping the split skips its merge launch. */
#define PA_PARTITION_AUTO (-2)
#define PA_AUTO_WHOLE_MAX_LEN 256

/* flags of pa_paged_attention_decode.
 * PA_DECODE_KV_REUSED: some physical blocks are read by more than one
 *   sequence in this call (a shared prefix).  The K/V loads then go through
 *   the caches so repeated reads hit, and a balanced split keeps each KV
 *   head on one XCD.  Without it every block is streamed past the caches
 *   (non-temporal loads), the fastest choice when each block is read once.
 *   Results are the same either way. */
#define PA_DECODE_KV_REUSED 1u

/* Message describing the last error on the calling thread ("" if none). */
const char *pa_last_error(void);

/* Library ABI version (major * 100 + minor). */
int32_t pa_version(void);

/* ------------------------------------------------------------------------
 * paged_attention_decode -- single-query attention of every sequence over
 * its cached tokens, read through its block table rather than from one
 * contiguous buffer (note-023 "Concepts", PagedAttention).  The result is plain softmax
 * attention; paging changes where the bytes come from, not the attention
 * computation (inferensys glossary "Paged Attention", fourth paragraph).
 *
 *  out            [num_seqs][num_q_heads][head_dim] in out_dtype (device, written)
 *  query          [num_seqs][num_q_heads][head_dim] in kv_dtype (device)
 *  key_cache      key pool, layout above, kv_dtype (device)
 *  value_cache    value pool, layout above, kv_dtype (device)
 *  block_tables   int32 [num_seqs][max_blocks_per_seq], row-major (device);
 *                 entry j of row i is the physical block of tokens
 *                 j*block_size .. (j+1)*block_size-1 of sequence i.  Entries
 *                 at or past ceil(L_i / block_size) are never read.
 *  context_lens   int32 [num_seqs] (device): L_i cached tokens of sequence i,
 *                 0 <= L_i <= max_context_len.  L_i = 0 gives a zero row.
 *  num_blocks     physical blocks in each pool (used by PA_VALIDATE checks).
 *  Query head h attends with KV head h / (num_q_heads / num_kv_heads)
 *  (grouped-query attention, inferensys glossary, GQA paragraph).
 *  scale          multiplies q.k before the softmax (usually 1/sqrt(head_dim)).
 *  max_context_len  host upper bound of every L_i; sizes the launch without
 *                 a device read.  Must be <= max_blocks_per_seq * block_size.
 *  partition_size how each sequence's context is split across waves; the
 *                 pieces are merged exactly by a log-sum-exp reduce:
 *                   > 0  a multiple of block_size: ceil(L_i / partition_size)
 *                        partitions of that many tokens;
 *                   0    no split, one pass per (sequence, head);
 *                   PA_PARTITION_AUTO (-2)  0 or balanced, by
 *                        max_context_len (pa_resolve_partition);
 *                   any other value < 0 (PA_PARTITION_BALANCED) balanced:
 *                        the tiles of all sequences are cut into one range
 *                        per wave the GPU holds at once, sized per XCD by
 *                        pa_set_balance_weights.
 *  flags          PA_DECODE_* bits (0: K/V streamed, each block read once).
 *  workspace      device scratch of at least
 *                 pa_paged_attention_workspace_bytes(...) bytes when that is
 *                 nonzero (caller-owned, contents need not be initialised;
 *                 the call's kernels reset what they count with).  Calls
 *                 that may overlap (other streams) need workspaces of their own.
 *  Supported: head_dim in {64, 128}, block_size in {16, 32, 64},
 *  kv_dtype/out_dtype in {PA_FP32, PA_BF16}; anything else returns
 *  PA_ERR_UNSUPPORTED.  bf16 outputs are rounded to nearest even.
 * ---------------------------------------------------------------------- */
pa_status pa_paged_attention_decode(void *out, const void *query, const void *key_cache,
                                    const void *value_cache, const int32_t *block_tables,
                                    const int32_t *context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int64_t num_blocks, int32_t max_context_len, float scale,
                                    int32_t partition_size, pa_dtype kv_dtype, pa_dtype out_dtype,
                                    uint32_t flags, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode_append -- one decode step's cache write and
 * attention in one launch: the same results as pa_reshape_and_cache(new_key,
 * new_value, key_cache, value_cache, slot_mapping, num_seqs, ...) followed by
 * pa_paged_attention_decode(...) on the same stream, pools and outputs
 * alike.  The new token of a sequence is the last of its context (the
 * caller has reserved it with pa_seq_append_slot, which allocates a block at
 * a block boundary and copies a shared block first; note-023 "Method" and
 * "Concepts").  The wave that loads the 16-token tile holding that position
 * puts the new token into the loaded registers, so the arithmetic is
 * exactly the unfused pair's; the slots are written by the launch's waves
 * after their reads, which saves the separate pass and its launch.
 *
 *  new_key, new_value  [num_seqs][num_kv_heads][head_dim] in kv_dtype (device)
 *  slot_mapping   int64 [num_seqs] (device).  For each i, either negative
 *                 (no new token: sequence i is attended as is) or the slot
 *                 of position context_lens[i] - 1 in block_tables row i,
 *                 in a block that no other sequence of the call reads or
 *                 writes (true of blocks from pa_seq_append_slot, whose
 *                 copy-on-write pair is copied first: by pa_copy_blocks,
 *                 or by this launch through cow_src).  PA_VALIDATE=1 checks the
 *                 position; a slot outside the pool is skipped like a
 *                 negative one.
 *  cow_src        NULL, or int64 [num_seqs] (device): copy-on-write inside
 *                 the launch (note-023, Concepts; inferensys glossary,
 *                 second paragraph: a shared block is copied when a sharer
 *                 writes).  cow_src[i] >= 0 is the block whose whole
 *                 contents (K and V, all heads and slots) sequence i's new
 *                 token block, slot_mapping[i] / block_size, takes before
 *                 the token is written: the pair (cow_src[i], that block)
 *                 that pa_seq_append_slot returned, which pa_copy_blocks
 *                 would otherwise copy first.  Sequence i's attention reads
 *                 the source in that block's place.  Another sequence of
 *                 the call may write its new token into a source block in
 *                 place only at the same offset (true of sharers of a partly
 *                 filled block, which have equal lengths).  Negative: no
 *                 copy.  PA_VALIDATE=1 checks each source and offset.
 *  Every other argument as in pa_paged_attention_decode (key_cache and
 *  value_cache are written here).
 * ---------------------------------------------------------------------- */
pa_status pa_paged_attention_decode_append(
    void *out, const void *query, void *key_cache, void *value_cache, const void *new_key,
    const void *new_value, const int64_t *slot_mapping, const int64_t *cow_src,
    const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, pa_dtype kv_dtype,
    pa_dtype out_dtype, uint32_t flags, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode_noalloc -- pa_paged_attention_decode_append with
 * no workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Every argument, result and error is as in
 * pa_paged_attention_decode_append, and new_key, new_value, slot_mapping
 * and cow_src may all be NULL (the plain pa_paged_attention_decode).  The
 * call's scratch (partial rows, merge counters, per-wave records) is a
 * device array the library holds, 64 MiB on each GPU it runs on, kept until
 * the process ends; the call allocates nothing.  Calls whose sizes need
 * more scratch than that (as pa_paged_attention_workspace_bytes reports)
 * return PA_ERR_INVALID_ARG before any launch; a 70B-shaped batch (256
 * sequences, 64/8 heads, head_dim 128, 4096 tokens) needs about 43 MB.  The
 * kernels reset what they count with, so the array needs no clearing, but
 * calls on one GPU share it: calls that may overlap on one GPU (other
 * streams) race and must not be made.
 * ---------------------------------------------------------------------- */
pa_status pa_paged_attention_decode_noalloc(
    void *out, const void *query, void *key_cache, void *value_cache, const void *new_key,
    const void *new_value, const int64_t *slot_mapping, const int64_t *cow_src,
    const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, pa_dtype kv_dtype, pa_dtype out_dtype, uint32_t flags,
    void *stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode_prefix -- the same attention when every sequence
 * starts with the same prefix_len tokens stored in the same physical blocks
 * (parallel samples or beam candidates of one prompt: inferensys glossary
 * "Paged Attention", second paragraph; the skillsintelligence glossary's
 * worked example of a 4,000-token prompt stored once for ten users).  The
 * prefix blocks are read once per KV head for all num_seqs * G query rows
 * (MFMA tiles), each sequence's own tokens after the prefix as in
 * pa_paged_attention_decode, and the two combined exactly by log-sum-exp.
 *
 *  prefix_len     positive multiple of block_size, <= every context_lens[i];
 *                 block_tables rows agree on their first prefix_len /
 *                 block_size entries (PA_VALIDATE=1 checks both).
 *  new_key, new_value, slot_mapping, cow_src
 *                 new tokens all NULL, or the step's new tokens and copies
 *                 exactly as in pa_paged_attention_decode_append (written
 *                 by this call).
 *                 A new token sits after the prefix (context_lens[i] >
 *                 prefix_len where slot_mapping[i] >= 0): its block is the
 *                 sequence's own.  PA_VALIDATE=1 checks this too.
 *  workspace      pa_paged_attention_prefix_workspace_bytes(...) bytes.
 *  Needs bf16 K/V (PA_ERR_UNSUPPORTED otherwise); other arguments as in
 *  pa_paged_attention_decode, with the balanced split.
 * ---------------------------------------------------------------------- */
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
                                           size_t workspace_bytes, void *stream);
size_t pa_paged_attention_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim,
                                                 int32_t max_context_len, int32_t prefix_len,
                                                 pa_dtype kv_dtype);

/* Tracing hook: while set, every pa_paged_attention_decode(_append,
 * _noalloc, _prefix) call made from the calling thread launches its main
 * attention kernel with the hipEvent_t pair (main_start, main_end) and its
 * log-sum-exp merge kernel, when it has one, with (merge_start,
 * merge_end): the runtime stamps each pair with that kernel's own start and
 * end time (hipExtLaunchKernel), so the elapsed time between a pair is
 * that kernel's duration.  Any of the four may be NULL (not stamped); pass
 * all NULL to stop.  On ROCm an end event delays the next launch on the
 * stream by several microseconds, so the span from the main kernel's start
 * to the merge kernel's end is best taken with only main_start and
 * merge_end set.  The events are caller-owned; the setting belongs to the
 * calling thread only (calls from other threads record nothing). */
pa_status pa_set_timing_events(void *main_start, void *main_end, void *merge_start,
                               void *merge_end);

/* Tile shares of the balanced split (partition_size < 0), one weight per XCD
 * in workgroup dispatch order (workgroup w runs on XCD w mod 8): each wave's
 * range of tiles is proportional to its XCD's weight.  Default
 * {115,100,115,100,115,100,115,100}: on MI355X, waves on even-numbered XCDs
 * stream 10-15% faster than waves on odd-numbered ones.  weights == NULL
 * restores the default; otherwise n must be 8 and each weight in [1, 1000].
 * Process-wide and thread-safe: each call uses one whole setting, the one
 * current when it was made.  Weights move the piece boundaries, so outputs may change in
 * their last bits (within the attention tolerance); for fixed weights,
 * sizes and lengths every call gives the same bits. */
pa_status pa_set_balance_weights(const int32_t *weights, int32_t n);

/* The split a decode call with this partition_size and max_context_len
 * runs: PA_PARTITION_AUTO gives 0 when max_context_len <=
 * PA_AUTO_WHOLE_MAX_LEN and PA_PARTITION_BALANCED otherwise; any other value
 * is returned as it is.  Host only, no device call. */
int32_t pa_resolve_partition(int32_t partition_size, int32_t max_context_len);

/* Bytes of workspace pa_paged_attention_decode (and _append) needs for these sizes on the
 * current device; 0 when every output row is written directly (no split).
 * Returns 0 for invalid arguments too (the decode call then reports them),
 * and for a balanced split when no device can be queried. */
size_t pa_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_context_len, int32_t partition_size,
                                          pa_dtype kv_dtype);

/* ------------------------------------------------------------------------
 * reshape_and_cache -- write each new token's K/V into its slot of the
 * pools: blocks are taken as a sequence grows, one token at a time
 * (note-023 "Method"; crackai.dev "How It Works", KV cache pages).  Bit
 * copy, no conversion.
 *
 *  key, value     [num_tokens][num_kv_heads][head_dim] in dtype (device)
 *  key_cache, value_cache  pools, layout above (device, written)
 *  slot_mapping   int64 [num_tokens] (device): block * block_size + offset;
 *                 a negative slot skips the token.  Slots must be
 *                 < num_blocks * block_size and distinct (a repeated slot is
 *                 a caller error; PA_VALIDATE=1 rejects it).
 *  block_size must be a multiple of 16 (PA_ERR_UNSUPPORTED otherwise).
 * ---------------------------------------------------------------------- */
pa_status pa_reshape_and_cache(const void *key, const void *value, void *key_cache,
                               void *value_cache, const int64_t *slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, pa_dtype dtype, void *stream);

/* ------------------------------------------------------------------------
 * copy_blocks -- the copy of copy-on-write: a sequence writing into a shared
 * block first gets a private duplicate (note-023 "Concepts", copy-on-write;
 * inferensys glossary, second paragraph).  Copies whole blocks, K and V,
 * every head and every slot.
 *
 *  block_mapping  int64 [num_pairs][2] (device): (src, dst) physical blocks.
 *                 A src may repeat; dsts must be distinct and not among the
 *                 srcs, so the result does not depend on order (PA_VALIDATE=1
 *                 rejects violations).  num_pairs = 0 is a no-op.
 * ---------------------------------------------------------------------- */
pa_status pa_copy_blocks(void *key_cache, void *value_cache, const int64_t *block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype, void *stream);

/* ------------------------------------------------------------------------
 * Every layer at once.  A model keeps one pair of pools per layer and
 * writes one new token per sequence into each of them per decode step; the
 * copy of copy-on-write applies to every layer too.  These calls do that in
 * one launch instead of one per layer.  key_caches, value_caches (and keys,
 * values) are device arrays of num_layers pointers, one per layer, each as
 * in the single-layer call (PA_VALIDATE=1 checks every pointer); all
 * layers share the shapes, the slots and the block mapping.
 * ---------------------------------------------------------------------- */
pa_status pa_reshape_and_cache_layers(const void *const *keys, const void *const *values,
                                      void *const *key_caches, void *const *value_caches,
                                      int32_t num_layers, const int64_t *slot_mapping,
                                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                                      void *stream);
pa_status pa_copy_blocks_layers(void *const *key_caches, void *const *value_caches,
                                int32_t num_layers, const int64_t *block_mapping,
                                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                                void *stream);

/* ------------------------------------------------------------------------
 * swap_blocks -- the copy half of swapping a preempted sequence's blocks to
 * host memory and back (inferensys glossary "Paged Attention", third and
 * fifth paragraphs; crackai.dev "How It Works", preemption and swapping).
 * Copies whole blocks, K and V, from one pool to another; either pool may
 * be device memory or pinned host memory the device can address (from
 * hipHostMalloc, e.g. a torch tensor with pin_memory=True), both in the
 * pool layout above with the same head count, head size and block size.
 * One launch for all pairs.
 *
 *  block_mapping  int64 [num_pairs][2], device-addressable: (block in src
 *                 pools, block in dst pools), as pa_seqs_swap_out/_in
 *                 return them.  dst blocks must be distinct.  Pairs with a
 *                 block outside [0, src_num_blocks) or [0, dst_num_blocks)
 *                 are skipped (PA_VALIDATE=1 rejects them).
 *  Every pointer is checked with hipPointerGetAttributes before the launch:
 *  pageable host memory gives PA_ERR_INVALID_ARG instead of a device fault.
 * ---------------------------------------------------------------------- */
pa_status pa_swap_blocks(void *dst_key_cache, void *dst_value_cache, const void *src_key_cache,
                         const void *src_value_cache, const int64_t *block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t src_num_blocks, int64_t dst_num_blocks,
                         pa_dtype dtype, void *stream);

/* ------------------------------------------------------------------------
 * Block allocator (host).  Free list, reference counts and copy-on-write
 * over a pool of num_blocks physical blocks (note-023 "Method" and
 * "Concepts"; inferensys glossary, first and second paragraphs; crackai.dev
 * "How It Works").  Policy where the pages leave it open:
 *  - the free list is a LIFO stack;
 *  - a finished sequence's blocks are pushed from its last logical block to
 *    its first, so its first block is the next one handed out (the
 *    skillsintelligence glossary's worked example: a finished request's
 *    blocks go to a newly arriving request in the following step);
 *  - a copy happens only when appending into a partially filled last block
 *    whose refcount is above 1; a full shared block is never copied;
 *  - every call is all-or-nothing: on an error the state is unchanged.
 * Sequence ids are arbitrary int64 values chosen by the caller.
 * ---------------------------------------------------------------------- */
typedef struct pa_allocator pa_allocator;

/* New allocator over num_blocks blocks of block_size tokens.  With
 * initial_free_order == NULL the first blocks handed out are 0, 1, 2, ...;
 * otherwise initial_free_order[0..num_blocks-1] (a permutation of
 * 0..num_blocks-1, copied) gives the order of the first hand-outs.  Returns
 * NULL on invalid arguments (see pa_last_error). */
pa_allocator *pa_allocator_create(int64_t num_blocks, int32_t block_size,
                                  const int32_t *initial_free_order);
void pa_allocator_destroy(pa_allocator *a);
int64_t pa_allocator_num_free(const pa_allocator *a);
int32_t pa_allocator_block_size(const pa_allocator *a);

/* A sequence holding num_tokens prompt tokens in ceil(num_tokens/block_size)
 * fresh blocks (refcount 1).  PA_ERR_INVALID_ARG if seq_id exists or
 * num_tokens < 0; PA_ERR_OUT_OF_BLOCKS if the pool cannot hold it. */
pa_status pa_seq_create(pa_allocator *a, int64_t seq_id, int64_t num_tokens);

/* child shares every block of parent (each refcount + 1) and its length:
 * parallel sampling and beam search share the prompt's blocks (inferensys
 * glossary, second paragraph; crackai.dev, copy-on-write sharing). */
pa_status pa_seq_fork(pa_allocator *a, int64_t parent_id, int64_t child_id);

/* Reserve position L (the sequence then holds L + 1 tokens) and return its
 * slot.  If L % block_size == 0 a fresh block is appended.  Otherwise, if
 * the last block is shared (refcount > 1), a fresh block dst replaces it in
 * this sequence's table, the old block src loses one reference, and
 * (*cow_src, *cow_dst) = (src, dst); else the write goes in place and both
 * are -1.  The caller must run pa_copy_blocks on every returned pair before
 * pa_reshape_and_cache writes the slot. */
pa_status pa_seq_append_slot(pa_allocator *a, int64_t seq_id, int64_t *slot, int64_t *cow_src,
                             int64_t *cow_dst);

/* Release a finished sequence: each block loses one reference and blocks
 * reaching zero return to the free list (last logical block first). */
pa_status pa_seq_free(pa_allocator *a, int64_t seq_id);

/* Copy the sequence's physical blocks (swap-space blocks while it is
 * swapped out) into out[0..capacity); *n_out gets the count.
 * PA_ERR_INVALID_ARG if capacity is too small (nothing written). */
pa_status pa_seq_block_table(const pa_allocator *a, int64_t seq_id, int32_t *out,
                             int32_t capacity, int32_t *n_out);

/* Tokens held by the sequence, or -1 if unknown. */
int64_t pa_seq_len(const pa_allocator *a, int64_t seq_id);

/* References to a physical block (0 = free), or -1 if out of range. */
int32_t pa_block_refcount(const pa_allocator *a, int32_t block);

/* Swap space: num_host_blocks blocks in host memory with their own LIFO free
 * list (first hand-outs 0, 1, 2, ...), replacing any previous swap space.
 * PA_ERR_INVALID_ARG while a sequence is swapped out. */
pa_status pa_allocator_set_swap_space(pa_allocator *a, int64_t num_host_blocks);
int64_t pa_allocator_num_free_host(const pa_allocator *a);
/* References to a swap-space block (0 = free), or -1 if out of range. */
int32_t pa_host_block_refcount(const pa_allocator *a, int32_t block);
/* 1 if the sequence is swapped out, 0 if resident, -1 if unknown. */
int32_t pa_seq_is_swapped(const pa_allocator *a, int64_t seq_id);

/* Preempt a group of resident sequences to the swap space (inferensys
 * glossary, third and fifth paragraphs).  The group's distinct device
 * blocks, in order of first appearance (sequences in the given order, each
 * table in logical order), each get one swap block; pairs[2k], pairs[2k+1]
 * = (device block, swap block) for pa_swap_blocks (host int64 array of
 * capacity pairs), *num_pairs their count.  Each device block loses the
 * group's references and returns to the free list at zero (in reverse order
 * of first appearance), so the caller must run the copy before reusing the
 * pool.  Blocks shared inside the group stay shared in the swap space.
 * While swapped, a sequence cannot be forked, appended to or put in a
 * table; pa_seq_free releases its swap blocks.  All-or-nothing:
 * PA_ERR_OUT_OF_BLOCKS if the swap space is too small, PA_ERR_INVALID_ARG
 * for a repeated, already swapped sequence or a small capacity. */
pa_status pa_seqs_swap_out(pa_allocator *a, const int64_t *seq_ids, int32_t n, int64_t *pairs,
                           int32_t capacity, int32_t *num_pairs);

/* Bring a group of swapped-out sequences back: the mirror of
 * pa_seqs_swap_out, pairs = (swap block, device block).  Generation resumes
 * from the same tokens, in new device blocks. */
pa_status pa_seqs_swap_in(pa_allocator *a, const int64_t *seq_ids, int32_t n, int64_t *pairs,
                          int32_t capacity, int32_t *num_pairs);

/* Pack the tables and lengths of n sequences for upload: out_tables is a
 * host int32 [n][max_blocks] filled with each table, padded with pad;
 * out_lens a host int32 [n].  PA_ERR_INVALID_ARG if a table is longer than
 * max_blocks or a length exceeds INT32_MAX. */
pa_status pa_build_block_tables(const pa_allocator *a, const int64_t *seq_ids, int32_t n,
                                int32_t max_blocks, int32_t pad, int32_t *out_tables,
                                int32_t *out_lens);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
