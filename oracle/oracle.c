/*
 * CPU oracle for the paged decode path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code with the HIP path: it is plain C,
 * built by gcc, with every index formula written out here from the layout
 * definition below.
 *
 * What it computes (all from the method as the pages state it):
 *
 *  - paged attention (dmarx note-023, Method; Concepts "PagedAttention"):
 *    the kernel reads each sequence's
 *    K/V through a per-sequence block table that maps logical block index to
 *    physical block, and the result is plain softmax attention, the gain
 *    coming from memory management alone and not from changing the attention
 *    computation (inferensys glossary "Paged Attention", fourth paragraph).
 *    So the oracle gathers each sequence's blocks into one contiguous fp64
 *    buffer and runs naive fp64 softmax(scale * q.K^T) V over all L cached
 *    positions.  Grouped-query attention (same glossary, GQA paragraph):
 *    query head h reads KV head h / (Hq / Hkv).
 *
 *  - reshape_and_cache: the new token's K/V are written into the slot the
 *    block table gives it -- a block is taken only when a sequence's
 *    growth needs one (note-023 Method; crackai.dev "How It Works", KV cache
 *    pages).  A slot is block * Bs + offset; a negative slot is skipped.
 *    Bit copy.
 *
 *  - copy_blocks: under copy-on-write a sequence that writes to a shared
 *    block is given a private duplicate of it (note-023 Concepts
 *    "Copy-on-write"; inferensys, second paragraph).  The whole block is copied, K and V, every head and slot.
 *    All sources are read before any destination is written.
 *
 * Pool layout (the library's, stated here so the oracle can address it):
 *   x = 16 / element size (4 for fp32, 8 for bf16)
 *   key   pool [num_blocks][Hkv][d / x][Bs][x]
 *   T = 16 when Bs is a multiple of 16, else T = Bs (values kept in
 *       groups of T tokens)
 *   value pool [num_blocks][Hkv][Bs/T][d][T]
 *   token o of block b, KV head g, feature e is
 *     key   (((b*Hkv + g)*(d/x) + e/x)*Bs + o)*x + e%x
 *     value (((b*Hkv + g)*(Bs/T) + o/T)*d + e)*T + o%T
 *
 * bf16 values are passed as raw uint16 bits and widened exactly
 * (bits << 16 is the fp32 value; fp32 -> fp64 is exact).
 *
 * Threads over (sequence, KV head) units are for timing only: each unit's
 * arithmetic runs sequentially in token order, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_FP32 0
#define OR_BF16 1

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_NOMEM (-2)

static double widen(const void *base, int64_t idx, int dtype) {
  if (dtype == OR_FP32) return (double)((const float *)base)[idx];
  uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int elem_size(int dtype) { return dtype == OR_FP32 ? 4 : 2; }

static int64_t key_index(int64_t b, int64_t g, int64_t o, int64_t e, int64_t hkv,
                         int64_t d, int64_t bs, int64_t x) {
  return (((b * hkv + g) * (d / x) + e / x) * bs + o) * x + e % x;
}

static int64_t value_index(int64_t b, int64_t g, int64_t o, int64_t e, int64_t hkv,
                           int64_t d, int64_t bs) {
  const int64_t t = bs % 16 == 0 ? 16 : bs;
  return (((b * hkv + g) * (bs / t) + o / t) * d + e) * t + o % t;
}

typedef struct {
  double *out;
  const void *q, *kc, *vc;
  const int32_t *tables, *lens;
  int64_t num_blocks;
  int B, hq, hkv, d, bs, maxb, dtype;
  double scale;
  int nthreads, tid;
  int status;
} attn_job;

/* One (sequence i, KV head g) unit: gather, then every query head of the group. */
static int attend_unit(const attn_job *j, int i, int g) {
  const int G = j->hq / j->hkv, d = j->d, bs = j->bs;
  const int x = 16 / elem_size(j->dtype);
  const int64_t L = j->lens[i];
  if (L < 0 || L > (int64_t)j->maxb * bs) return OR_ERR_ARG;
  if (L == 0) {
    for (int h = g * G; h < (g + 1) * G; ++h)
      memset(j->out + ((int64_t)i * j->hq + h) * d, 0, sizeof(double) * d);
    return OR_OK;
  }
  double *Kc = malloc(sizeof(double) * L * d);
  double *Vc = malloc(sizeof(double) * L * d);
  double *z = malloc(sizeof(double) * L);
  double *qv = malloc(sizeof(double) * d);
  if (!Kc || !Vc || !z || !qv) {
    free(Kc); free(Vc); free(z); free(qv);
    return OR_ERR_NOMEM;
  }
  /* Step 1: gather the sequence's blocks into contiguous per-token rows. */
  for (int64_t t = 0; t < L; ++t) {
    int64_t b = j->tables[(int64_t)i * j->maxb + t / bs];
    int64_t o = t % bs;
    if (b < 0 || b >= j->num_blocks) {
      free(Kc); free(Vc); free(z); free(qv);
      return OR_ERR_ARG;
    }
    for (int e = 0; e < d; ++e) {
      Kc[t * d + e] = widen(j->kc, key_index(b, g, o, e, j->hkv, d, bs, x), j->dtype);
      Vc[t * d + e] = widen(j->vc, value_index(b, g, o, e, j->hkv, d, bs), j->dtype);
    }
  }
  for (int h = g * G; h < (g + 1) * G; ++h) {
    const int64_t row = (int64_t)i * j->hq + h;
    for (int e = 0; e < d; ++e) qv[e] = widen(j->q, row * d + e, j->dtype);
    /* Step 2: logits z_t = scale * <q, k_t>. */
    double m = -INFINITY;
    for (int64_t t = 0; t < L; ++t) {
      double s = 0.0;
      for (int e = 0; e < d; ++e) s += qv[e] * Kc[t * d + e];
      z[t] = j->scale * s;
      if (z[t] > m) m = z[t];
    }
    /* Step 3: softmax weights w_t = exp(z_t - max z), normaliser l. */
    double l = 0.0;
    for (int64_t t = 0; t < L; ++t) {
      z[t] = exp(z[t] - m);
      l += z[t];
    }
    /* Step 4: out = sum_t w_t v_t / l. */
    double *o = j->out + row * d;
    for (int e = 0; e < d; ++e) {
      double acc = 0.0;
      for (int64_t t = 0; t < L; ++t) acc += z[t] * Vc[t * d + e];
      o[e] = acc / l;
    }
  }
  free(Kc); free(Vc); free(z); free(qv);
  return OR_OK;
}

static void *attn_worker(void *arg) {
  attn_job *j = (attn_job *)arg;
  const int64_t units = (int64_t)j->B * j->hkv;
  for (int64_t u = j->tid; u < units; u += j->nthreads) {
    int rc = attend_unit(j, (int)(u / j->hkv), (int)(u % j->hkv));
    if (rc != OR_OK) { j->status = rc; break; }
  }
  return NULL;
}

int oracle_paged_attention(double *out, const void *query, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, int64_t num_blocks, double scale,
                           int dtype, int nthreads) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0 ||
      (dtype != OR_FP32 && dtype != OR_BF16) || head_dim % (16 / elem_size(dtype)) != 0)
    return OR_ERR_ARG;
  if (num_seqs == 0) return OR_OK;
  if (nthreads < 1) nthreads = 1;
  attn_job *jobs = calloc((size_t)nthreads, sizeof *jobs);
  pthread_t *th = calloc((size_t)nthreads, sizeof *th);
  if (!jobs || !th) { free(jobs); free(th); return OR_ERR_NOMEM; }
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (attn_job){out, query, key_cache, value_cache, block_tables, context_lens,
                         num_blocks, num_seqs, num_q_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, dtype, scale, nthreads, t, OR_OK};
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t, ++started)
    if (pthread_create(&th[t], NULL, attn_worker, &jobs[t]) != 0) break;
  attn_worker(&jobs[0]);
  /* Threads that failed to start: run their share here. */
  for (int t = started + 1; t < nthreads; ++t) attn_worker(&jobs[t]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  int rc = OR_OK;
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status != OR_OK) rc = jobs[t].status;
  free(jobs);
  free(th);
  return rc;
}

int oracle_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int block_size,
                             int64_t num_blocks, int dtype) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      (dtype != OR_FP32 && dtype != OR_BF16) || head_dim % (16 / elem_size(dtype)) != 0)
    return OR_ERR_ARG;
  const int esz = elem_size(dtype), x = 16 / esz;
  for (int i = 0; i < num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;
    if (s >= num_blocks * block_size) return OR_ERR_ARG;
    const int64_t b = s / block_size, o = s % block_size;
    for (int g = 0; g < num_kv_heads; ++g) {
      for (int e = 0; e < head_dim; ++e) {
        const int64_t src = ((int64_t)i * num_kv_heads + g) * head_dim + e;
        memcpy((char *)key_cache + key_index(b, g, o, e, num_kv_heads, head_dim, block_size, x) * esz,
               (const char *)key + src * esz, (size_t)esz);
        memcpy((char *)value_cache + value_index(b, g, o, e, num_kv_heads, head_dim, block_size) * esz,
               (const char *)value + src * esz, (size_t)esz);
      }
    }
  }
  return OR_OK;
}

int oracle_copy_blocks(void *key_cache, void *value_cache, const int64_t *block_mapping,
                       int num_pairs, int num_kv_heads, int head_dim, int block_size,
                       int64_t num_blocks, int dtype) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      (dtype != OR_FP32 && dtype != OR_BF16))
    return OR_ERR_ARG;
  if (num_pairs == 0) return OR_OK;
  const size_t block_bytes = (size_t)num_kv_heads * head_dim * block_size * elem_size(dtype);
  for (int p = 0; p < num_pairs; ++p) {
    const int64_t s = block_mapping[2 * p], t = block_mapping[2 * p + 1];
    if (s < 0 || s >= num_blocks || t < 0 || t >= num_blocks) return OR_ERR_ARG;
  }
  /* Snapshot every source block first, then write the destinations. */
  char *snap = malloc(2 * block_bytes * (size_t)num_pairs);
  if (!snap) return OR_ERR_NOMEM;
  for (int p = 0; p < num_pairs; ++p) {
    const int64_t s = block_mapping[2 * p];
    memcpy(snap + (2 * (size_t)p) * block_bytes, (char *)key_cache + s * block_bytes, block_bytes);
    memcpy(snap + (2 * (size_t)p + 1) * block_bytes, (char *)value_cache + s * block_bytes, block_bytes);
  }
  for (int p = 0; p < num_pairs; ++p) {
    const int64_t t = block_mapping[2 * p + 1];
    memcpy((char *)key_cache + t * block_bytes, snap + (2 * (size_t)p) * block_bytes, block_bytes);
    memcpy((char *)value_cache + t * block_bytes, snap + (2 * (size_t)p + 1) * block_bytes, block_bytes);
  }
  free(snap);
  return OR_OK;
}

/* swap_blocks: the copy of swapping a preempted sequence's blocks to host
 * memory and back (inferensys glossary "Paged Attention", third and fifth
 * paragraphs).  For each pair (s, t), block t of the destination pools
 * becomes a copy of block s of the source pools: K and V, every head and
 * slot.  The pools are distinct, so the order of the pairs does not matter. */
int oracle_swap_blocks(void *dst_key, void *dst_value, const void *src_key,
                       const void *src_value, const int64_t *block_mapping, int num_pairs,
                       int num_kv_heads, int head_dim, int block_size, int64_t src_num_blocks,
                       int64_t dst_num_blocks, int dtype) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      (dtype != OR_FP32 && dtype != OR_BF16))
    return OR_ERR_ARG;
  const size_t block_bytes = (size_t)num_kv_heads * head_dim * block_size * elem_size(dtype);
  for (int p = 0; p < num_pairs; ++p) {
    const int64_t s = block_mapping[2 * p], t = block_mapping[2 * p + 1];
    if (s < 0 || s >= src_num_blocks || t < 0 || t >= dst_num_blocks) return OR_ERR_ARG;
  }
  for (int p = 0; p < num_pairs; ++p) {
    const int64_t s = block_mapping[2 * p], t = block_mapping[2 * p + 1];
    memcpy((char *)dst_key + t * block_bytes, (const char *)src_key + s * block_bytes, block_bytes);
    memcpy((char *)dst_value + t * block_bytes, (const char *)src_value + s * block_bytes,
           block_bytes);
  }
  return OR_OK;
}
