// Host block allocator: free list, reference counts, copy-on-write.
//
// Follows the memory-management half of the method: fixed-size blocks and a
// per-sequence logical -> physical block table (dmarx note-023 "Method";
// crackai.dev "How It Works"), blocks allocated on demand and freed when a
// sequence finishes (note-023 "Method"), and physical blocks shared by
// reference with a copy only when a sharer writes (note-023 "Concepts",
// copy-on-write; inferensys glossary "Paged Attention", second paragraph).
//
// The free list is a LIFO stack held in a vector whose back is the next
// block handed out.  A finished sequence pushes its blocks from the last
// logical block to the first, so its first block is reused first -- in the
// skillsintelligence glossary's worked example a finished request's blocks
// go straight to a newly arriving request in the following step.
//
// Every operation checks everything it needs before mutating anything, so a
// failing call leaves the allocator exactly as it was.
#include <limits.h>

#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_allocator {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t pop() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

}  // namespace

extern "C" {

pa_allocator *pa_allocator_create(int64_t num_blocks, int32_t block_size,
                                  const int32_t *initial_free_order) {
  pa_clear_error();
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) {
    pa_fail(PA_ERR_INVALID_ARG, "pa_allocator_create: num_blocks must be in [1, 2^31) and "
            "block_size positive (got %lld, %d)", (long long)num_blocks, block_size);
    return nullptr;
  }
  auto *a = new pa_allocator;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcount.assign((size_t)num_blocks, 0);
  a->free_stack.resize((size_t)num_blocks);
  if (initial_free_order) {
    std::vector<char> seen((size_t)num_blocks, 0);
    for (int64_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
        delete a;
        pa_fail(PA_ERR_INVALID_ARG, "pa_allocator_create: initial_free_order is not a "
                "permutation of 0..%lld (entry %lld = %d)", (long long)(num_blocks - 1),
                (long long)i, b);
        return nullptr;
      }
      seen[(size_t)b] = 1;
    }
    // order[0] is handed out first, so it sits at the back of the stack.
    for (int64_t i = 0; i < num_blocks; ++i)
      a->free_stack[(size_t)i] = initial_free_order[num_blocks - 1 - i];
  } else {
    for (int64_t i = 0; i < num_blocks; ++i)
      a->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
  }
  return a;
}

void pa_allocator_destroy(pa_allocator *a) { delete a; }

int64_t pa_allocator_num_free(const pa_allocator *a) {
  return a ? (int64_t)a->free_stack.size() : -1;
}

int32_t pa_allocator_block_size(const pa_allocator *a) { return a ? a->block_size : -1; }

pa_status pa_seq_create(pa_allocator *a, int64_t seq_id, int64_t num_tokens) {
  pa_clear_error();
  if (!a) return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_create: null allocator");
  if (num_tokens < 0)
    return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_create: negative length %lld",
                   (long long)num_tokens);
  if (a->seqs.count(seq_id))
    return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_create: sequence %lld exists", (long long)seq_id);
  const int64_t need = blocks_for(num_tokens, a->block_size);
  if (need > (int64_t)a->free_stack.size())
    return pa_fail(PA_ERR_OUT_OF_BLOCKS, "pa_seq_create: %lld blocks needed, %zu free",
                   (long long)need, a->free_stack.size());
  pa_allocator::Seq s;
  s.blocks.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(a->pop());
  s.len = num_tokens;
  a->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status pa_seq_fork(pa_allocator *a, int64_t parent_id, int64_t child_id) {
  pa_clear_error();
  if (!a) return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_fork: null allocator");
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end())
    return pa_fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_fork: unknown parent %lld", (long long)parent_id);
  if (a->seqs.count(child_id))
    return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_fork: child %lld exists", (long long)child_id);
  pa_allocator::Seq child = it->second;  // copy before emplace may rehash
  for (int32_t b : child.blocks) a->refcount[(size_t)b] += 1;
  a->seqs.emplace(child_id, std::move(child));
  return PA_OK;
}

pa_status pa_seq_append_slot(pa_allocator *a, int64_t seq_id, int64_t *slot, int64_t *cow_src,
                             int64_t *cow_dst) {
  pa_clear_error();
  if (!a || !slot || !cow_src || !cow_dst)
    return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_append_slot: null argument");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa_fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_append_slot: unknown sequence %lld",
                   (long long)seq_id);
  pa_allocator::Seq &s = it->second;
  const int64_t pos = s.len;
  const int32_t off = (int32_t)(pos % a->block_size);
  int64_t src = -1, dst = -1;
  if (off == 0) {
    if (a->free_stack.empty())
      return pa_fail(PA_ERR_OUT_OF_BLOCKS, "pa_seq_append_slot: pool exhausted");
    s.blocks.push_back(a->pop());
  } else {
    const int32_t last = s.blocks.back();
    if (a->refcount[(size_t)last] > 1) {
      if (a->free_stack.empty())
        return pa_fail(PA_ERR_OUT_OF_BLOCKS, "pa_seq_append_slot: pool exhausted (copy)");
      const int32_t fresh = a->pop();
      a->refcount[(size_t)last] -= 1;
      s.blocks.back() = fresh;
      src = last;
      dst = fresh;
    }
  }
  s.len = pos + 1;
  *slot = (int64_t)s.blocks.back() * a->block_size + off;
  *cow_src = src;
  *cow_dst = dst;
  return PA_OK;
}

pa_status pa_seq_free(pa_allocator *a, int64_t seq_id) {
  pa_clear_error();
  if (!a) return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_free: null allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa_fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_free: unknown sequence %lld", (long long)seq_id);
  const std::vector<int32_t> &blocks = it->second.blocks;
  for (size_t i = blocks.size(); i-- > 0;) {
    const int32_t b = blocks[i];
    if (--a->refcount[(size_t)b] == 0) a->free_stack.push_back(b);
  }
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_seq_block_table(const pa_allocator *a, int64_t seq_id, int32_t *out,
                             int32_t capacity, int32_t *n_out) {
  pa_clear_error();
  if (!a || !n_out) return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_block_table: null argument");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa_fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_block_table: unknown sequence %lld",
                   (long long)seq_id);
  const std::vector<int32_t> &blocks = it->second.blocks;
  if ((int64_t)blocks.size() > capacity || (!out && !blocks.empty()))
    return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_block_table: capacity %d < %zu blocks", capacity,
                   blocks.size());
  for (size_t i = 0; i < blocks.size(); ++i) out[i] = blocks[i];
  *n_out = (int32_t)blocks.size();
  return PA_OK;
}

int64_t pa_seq_len(const pa_allocator *a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : it->second.len;
}

int32_t pa_block_refcount(const pa_allocator *a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refcount[(size_t)block];
}

pa_status pa_build_block_tables(const pa_allocator *a, const int64_t *seq_ids, int32_t n,
                                int32_t max_blocks, int32_t pad, int32_t *out_tables,
                                int32_t *out_lens) {
  pa_clear_error();
  if (!a || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !out_tables || !out_lens)))
    return pa_fail(PA_ERR_INVALID_ARG, "pa_build_block_tables: bad arguments");
  // Check everything first so a failure writes nothing.
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return pa_fail(PA_ERR_UNKNOWN_SEQ, "pa_build_block_tables: unknown sequence %lld",
                     (long long)seq_ids[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks || it->second.len > INT32_MAX)
      return pa_fail(PA_ERR_INVALID_ARG, "pa_build_block_tables: sequence %lld has %zu blocks "
                     "> max_blocks %d", (long long)seq_ids[i], it->second.blocks.size(),
                     max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const pa_allocator::Seq &s = a->seqs.find(seq_ids[i])->second;
    int32_t *row = out_tables + (int64_t)i * max_blocks;
    size_t j = 0;
    for (; j < s.blocks.size(); ++j) row[j] = s.blocks[j];
    for (; j < (size_t)max_blocks; ++j) row[j] = pad;
    out_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

}  // extern "C"
