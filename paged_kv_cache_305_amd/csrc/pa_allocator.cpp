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
// Swapping (inferensys glossary "Paged Attention", third and fifth
// paragraphs; crackai.dev "How It Works", preemption and swapping): under
// memory pressure a group of sequences is preempted by moving its blocks to
// a swap space in host memory, and later brought back, generation resuming
// where it stopped.  The swap space is a second pool of block ids with its
// own LIFO free list.  A group's distinct blocks, in order of first
// appearance (sequences in the given order, each table in logical order),
// each get one block in the other pool; the call returns the (from, to)
// pairs for pa_swap_blocks and releases the blocks the group no longer
// needs, pushing them in reverse order of first appearance.  Blocks shared
// inside the group stay shared; blocks shared with sequences outside it are
// copied, and the others keep the original.
//
// Every operation checks everything it needs before mutating anything, so a
// failing call leaves the allocator exactly as it was.
#include <limits.h>

#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

struct pa_allocator {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  struct Seq {
    std::vector<int32_t> blocks;   // device block ids, or host ones while swapped
    int64_t len = 0;
    bool swapped = false;
  };
  std::unordered_map<int64_t, Seq> seqs;
  // Swap space in host memory (empty until pa_allocator_set_swap_space).
  std::vector<int32_t> host_free;  // back() is handed out next
  std::vector<int32_t> host_ref;

  int32_t pop() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

// One direction of a group swap: sequences `ids` move from the pool
// (from_ref, from_free) to the pool (to_ref, to_free).
pa_status swap_group(pa_allocator *a, const char *fn, const int64_t *ids, int32_t n,
                     bool to_host, int64_t *pairs, int32_t capacity, int32_t *num_pairs) {
  if (!a || n < 0 || (n > 0 && !ids) || !num_pairs || capacity < 0 || (capacity > 0 && !pairs))
    return pa_fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
  std::vector<int32_t> &from_ref = to_host ? a->refcount : a->host_ref;
  std::vector<int32_t> &from_free = to_host ? a->free_stack : a->host_free;
  std::vector<int32_t> &to_ref = to_host ? a->host_ref : a->refcount;
  std::vector<int32_t> &to_free = to_host ? a->host_free : a->free_stack;
  // Check everything first.
  std::unordered_set<int64_t> seen;
  std::unordered_map<int32_t, int32_t> uses;   // block -> references from the group
  std::vector<int32_t> order;                  // distinct blocks, first appearance
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(ids[i]);
    if (it == a->seqs.end())
      return pa_fail(PA_ERR_UNKNOWN_SEQ, "%s: unknown sequence %lld", fn, (long long)ids[i]);
    if (it->second.swapped == to_host)
      return pa_fail(PA_ERR_INVALID_ARG, "%s: sequence %lld is already %s", fn,
                     (long long)ids[i], to_host ? "swapped out" : "resident");
    if (!seen.insert(ids[i]).second)
      return pa_fail(PA_ERR_INVALID_ARG, "%s: sequence %lld given twice", fn, (long long)ids[i]);
    for (int32_t b : it->second.blocks)
      if (uses[b]++ == 0) order.push_back(b);
  }
  if (order.size() > to_free.size())
    return pa_fail(PA_ERR_OUT_OF_BLOCKS, "%s: %zu blocks needed, %zu free in the %s pool", fn,
                   order.size(), to_free.size(), to_host ? "swap" : "device");
  if ((int64_t)order.size() > capacity)
    return pa_fail(PA_ERR_INVALID_ARG, "%s: %zu pairs, capacity %d", fn, order.size(), capacity);
  // Move.
  std::unordered_map<int32_t, int32_t> moved;
  for (size_t k = 0; k < order.size(); ++k) {
    const int32_t b = order[k];
    const int32_t t = to_free.back();
    to_free.pop_back();
    to_ref[(size_t)t] = uses[b];
    moved[b] = t;
    pairs[2 * k] = b;
    pairs[2 * k + 1] = t;
  }
  for (size_t k = order.size(); k-- > 0;) {
    const int32_t b = order[k];
    from_ref[(size_t)b] -= uses[b];
    if (from_ref[(size_t)b] == 0) from_free.push_back(b);
  }
  for (int32_t i = 0; i < n; ++i) {
    pa_allocator::Seq &s = a->seqs.find(ids[i])->second;
    for (int32_t &b : s.blocks) b = moved[b];
    s.swapped = to_host;
  }
  *num_pairs = (int32_t)order.size();
  return PA_OK;
}

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
  if (it->second.swapped)
    return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_fork: parent %lld is swapped out",
                   (long long)parent_id);
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
  if (s.swapped)
    return pa_fail(PA_ERR_INVALID_ARG, "pa_seq_append_slot: sequence %lld is swapped out",
                   (long long)seq_id);
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
  std::vector<int32_t> &ref = it->second.swapped ? a->host_ref : a->refcount;
  std::vector<int32_t> &fr = it->second.swapped ? a->host_free : a->free_stack;
  for (size_t i = blocks.size(); i-- > 0;) {
    const int32_t b = blocks[i];
    if (--ref[(size_t)b] == 0) fr.push_back(b);
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

pa_status pa_allocator_set_swap_space(pa_allocator *a, int64_t num_host_blocks) {
  pa_clear_error();
  if (!a || num_host_blocks < 0 || num_host_blocks > INT32_MAX)
    return pa_fail(PA_ERR_INVALID_ARG, "pa_allocator_set_swap_space: bad arguments");
  for (const auto &kv : a->seqs)
    if (kv.second.swapped)
      return pa_fail(PA_ERR_INVALID_ARG, "pa_allocator_set_swap_space: sequence %lld is "
                     "swapped out", (long long)kv.first);
  a->host_ref.assign((size_t)num_host_blocks, 0);
  a->host_free.resize((size_t)num_host_blocks);
  for (int64_t i = 0; i < num_host_blocks; ++i)
    a->host_free[(size_t)i] = (int32_t)(num_host_blocks - 1 - i);
  return PA_OK;
}

int64_t pa_allocator_num_free_host(const pa_allocator *a) {
  return a ? (int64_t)a->host_free.size() : -1;
}

int32_t pa_host_block_refcount(const pa_allocator *a, int32_t block) {
  if (!a || block < 0 || (size_t)block >= a->host_ref.size()) return -1;
  return a->host_ref[(size_t)block];
}

int32_t pa_seq_is_swapped(const pa_allocator *a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

pa_status pa_seqs_swap_out(pa_allocator *a, const int64_t *seq_ids, int32_t n, int64_t *pairs,
                           int32_t capacity, int32_t *num_pairs) {
  pa_clear_error();
  return swap_group(a, "pa_seqs_swap_out", seq_ids, n, true, pairs, capacity, num_pairs);
}

pa_status pa_seqs_swap_in(pa_allocator *a, const int64_t *seq_ids, int32_t n, int64_t *pairs,
                          int32_t capacity, int32_t *num_pairs) {
  pa_clear_error();
  return swap_group(a, "pa_seqs_swap_in", seq_ids, n, false, pairs, capacity, num_pairs);
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
    if (it->second.swapped)
      return pa_fail(PA_ERR_INVALID_ARG, "pa_build_block_tables: sequence %lld is swapped out",
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
