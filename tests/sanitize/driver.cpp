// Host sanitizer driver -- TEST INFRASTRUCTURE ONLY.
//
// Built by tests/test_sanitizers.py with -fsanitize=address,undefined
// together with the library's host allocator sources and the CPU oracle
// (each from its own sources; they share nothing), then run.  It drives
// the allocator through seeded random traces, pool exhaustion and invalid
// ids, and the oracle's three operations on exactly sized heap buffers, so
// any out-of-bounds access, leak or undefined behaviour aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "pagedattn.h"

extern "C" {
int oracle_paged_attention(double *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, int64_t num_blocks, double scale, int dtype,
                           int nthreads);
int oracle_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                             int dtype);
int oracle_copy_blocks(void *key_cache, void *value_cache, const int64_t *block_mapping,
                       int num_pairs, int num_kv_heads, int head_dim, int block_size,
                       int64_t num_blocks, int dtype);
}

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      exit(1);                                                     \
    }                                                              \
  } while (0)

static void allocator_traces(uint32_t seed) {
  std::mt19937 rng(seed);
  const int64_t nblocks = 1 + rng() % 64;
  const int32_t bs = 1 + (int32_t)(rng() % 16);
  std::vector<int32_t> order((size_t)nblocks);
  for (int64_t i = 0; i < nblocks; ++i) order[(size_t)i] = (int32_t)i;
  std::shuffle(order.begin(), order.end(), rng);
  pa_allocator *a = pa_allocator_create(nblocks, bs, (rng() & 1) ? order.data() : nullptr);
  CHECK(a != nullptr);
  std::vector<int64_t> live;
  int64_t next_id = 0;
  for (int step = 0; step < 400; ++step) {
    const int op = (int)(rng() % 6);
    if (op == 0 || live.empty()) {
      const int64_t id = next_id++;
      if (pa_seq_create(a, id, (int64_t)(rng() % (3 * bs + 1))) == PA_OK) live.push_back(id);
    } else if (op == 1) {
      const int64_t child = next_id++;
      if (pa_seq_fork(a, live[rng() % live.size()], child) == PA_OK) live.push_back(child);
    } else if (op == 2 || op == 3) {
      int64_t slot, src, dst;
      const pa_status s = pa_seq_append_slot(a, live[rng() % live.size()], &slot, &src, &dst);
      CHECK(s == PA_OK || s == PA_ERR_OUT_OF_BLOCKS);
      if (s == PA_OK) CHECK(slot >= 0 && slot < nblocks * bs);
    } else if (op == 4) {
      const size_t k = rng() % live.size();
      CHECK(pa_seq_free(a, live[k]) == PA_OK);
      live.erase(live.begin() + (long)k);
    } else {
      const int32_t maxb = 8;
      std::vector<int32_t> tabs(live.size() * maxb), lens(live.size());
      const pa_status s = pa_build_block_tables(a, live.data(), (int32_t)live.size(), maxb, -1,
                                                tabs.data(), lens.data());
      CHECK(s == PA_OK || s == PA_ERR_INVALID_ARG);
      std::vector<int32_t> one(4);
      int32_t n = 0;
      const pa_status t = pa_seq_block_table(a, live[0], one.data(), 4, &n);
      CHECK(t == PA_OK || t == PA_ERR_INVALID_ARG);
    }
    // Invalid ids and arguments never change anything.
    int64_t slot, src, dst;
    CHECK(pa_seq_append_slot(a, -5, &slot, &src, &dst) == PA_ERR_UNKNOWN_SEQ);
    CHECK(pa_seq_free(a, -5) == PA_ERR_UNKNOWN_SEQ);
    CHECK(pa_block_refcount(a, (int32_t)nblocks) == -1);
    int64_t referenced = 0;
    for (int32_t b = 0; b < nblocks; ++b) referenced += pa_block_refcount(a, b) > 0;
    CHECK(referenced + pa_allocator_num_free(a) == nblocks);
  }
  pa_allocator_destroy(a);   // with sequences still live
}

static void fill(std::vector<uint8_t> &v, std::mt19937 &rng, int dtype) {
  if (dtype == PA_FP32) {
    std::normal_distribution<float> nd;
    float *f = reinterpret_cast<float *>(v.data());
    for (size_t i = 0; i < v.size() / 4; ++i) f[i] = nd(rng);
  } else {
    std::normal_distribution<float> nd;
    uint16_t *h = reinterpret_cast<uint16_t *>(v.data());
    for (size_t i = 0; i < v.size() / 2; ++i) {
      float x = nd(rng);
      uint32_t u;
      memcpy(&u, &x, 4);
      h[i] = (uint16_t)(u >> 16);
    }
  }
}

static void oracle_cases(uint32_t seed) {
  std::mt19937 rng(seed);
  const int dtype = (rng() & 1) ? PA_FP32 : PA_BF16;
  const int esz = dtype == PA_FP32 ? 4 : 2;
  const int hkv = 1 + (int)(rng() % 3), g = 1 + (int)(rng() % 3), hq = hkv * g;
  const int d = (dtype == PA_FP32 ? 4 : 8) * (1 + (int)(rng() % 3));
  const int bs = 1 + (int)(rng() % 8), B = (int)(rng() % 4), maxb = 1 + (int)(rng() % 5);
  const int64_t N = maxb * (B + 1);
  std::vector<uint8_t> q((size_t)B * hq * d * esz), kc((size_t)N * hkv * bs * d * esz),
      vc(kc.size());
  fill(q, rng, dtype);
  fill(kc, rng, dtype);
  fill(vc, rng, dtype);
  std::vector<int32_t> tabs((size_t)B * maxb), lens((size_t)B);
  for (int i = 0; i < B; ++i) {
    lens[(size_t)i] = (int32_t)(rng() % (maxb * bs + 1));
    for (int j = 0; j < maxb; ++j) tabs[(size_t)i * maxb + j] = (int32_t)(rng() % N);
  }
  std::vector<double> out((size_t)B * hq * d);
  CHECK(oracle_paged_attention(out.data(), q.data(), kc.data(), vc.data(), tabs.data(),
                               lens.data(), B, hq, hkv, d, bs, maxb, N, 0.3, dtype,
                               1 + (int)(rng() % 3)) == 0);
  const int T = 1 + (int)(rng() % 5);
  std::vector<uint8_t> nk((size_t)T * hkv * d * esz), nv(nk.size());
  fill(nk, rng, dtype);
  fill(nv, rng, dtype);
  std::vector<int64_t> slots((size_t)T);
  for (int i = 0; i < T; ++i) slots[(size_t)i] = (int64_t)(rng() % (N * bs + 2)) - 1;
  slots[0] = N * bs - 1;
  for (int i = 0; i < T; ++i)
    if (slots[(size_t)i] >= N * bs) slots[(size_t)i] = -1;
  CHECK(oracle_reshape_and_cache(nk.data(), nv.data(), kc.data(), vc.data(), slots.data(), T,
                                 hkv, d, bs, N, dtype) == 0);
  slots[0] = N * bs;   // out of range: rejected
  CHECK(oracle_reshape_and_cache(nk.data(), nv.data(), kc.data(), vc.data(), slots.data(), T,
                                 hkv, d, bs, N, dtype) != 0);
  std::vector<int64_t> pairs = {0, N - 1, 0, N - 2 >= 0 ? N - 2 : 0};
  CHECK(oracle_copy_blocks(kc.data(), vc.data(), pairs.data(), 2, hkv, d, bs, N, dtype) == 0);
  pairs[1] = N;
  CHECK(oracle_copy_blocks(kc.data(), vc.data(), pairs.data(), 2, hkv, d, bs, N, dtype) != 0);
}

int main() {
  for (uint32_t s = 0; s < 40; ++s) allocator_traces(s);
  CHECK(pa_allocator_create(0, 16, nullptr) == nullptr);
  int32_t bad[3] = {0, 0, 1};
  CHECK(pa_allocator_create(3, 16, bad) == nullptr);
  for (uint32_t s = 0; s < 60; ++s) oracle_cases(1000 + s);
  printf("sanitizer driver: ok\n");
  return 0;
}
