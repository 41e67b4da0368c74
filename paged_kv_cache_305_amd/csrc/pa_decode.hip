// Paged decode attention for gfx950 (CDNA4).
//
// One query token per sequence attends to the sequence's L cached tokens,
// whose K/V live in fixed-size physical blocks named by a per-sequence block
// table (dmarx note-023, "Method" and "Concepts"; crackai.dev, "How It
// Works").  The arithmetic is plain softmax attention: paging only changes
// where the bytes come from (inferensys glossary "Paged Attention", fourth
// paragraph).  Query head h reads KV head h / G, G = Hq / Hkv (same
// glossary, GQA paragraph).
//
// Work unit: one wave64 workgroup per (sequence, head unit, context
// partition).  A partition is `partition_size` tokens (or the whole context
// when it is 0); partitions of a sequence are merged exactly by a
// log-sum-exp reduce (decode_reduce) when there is more than one.
//
// Two main kernels, chosen per call:
//  * decode_valu -- head unit = one query head.  Vector-ALU dot products;
//    used for MHA (G = 1) and for fp32 KV.
//  * decode_mfma -- head unit = one KV head and up to 16 of its query heads.
//    bf16 KV with G >= 2: Q.K^T and P.V run on v_mfma_f32_16x16x32_bf16 and
//    v_mfma_f32_16x16x16_bf16 with the group's query heads on the N side of
//    both products, so each KV byte is read once for the whole group.
//
// Both kernels walk the partition in 16-token tiles (a block of 32 tokens is
// two tiles), keep PF tiles of K/V loads in flight in registers, keep the
// running max / sum / output in registers, and fix every reduction order
// by logical token position, so results are deterministic and independent
// of where the blocks sit physically.
//
// Softmax runs in base 2: logits are multiplied by scale * log2(e) and
// exponentiated with v_exp_f32; the stored partition maxima are base-2.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 mfma_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short mfma_i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float mfma_f32x4;

constexpr float kLog2e = 1.4426950408889634f;
#ifndef PA_PREFETCH
#define PA_PREFETCH 2
#endif
constexpr int kPrefetch = PA_PREFETCH;   // tiles of K/V loads kept in flight per wave

struct bf16_t {
  uint16_t bits;
};

// ---- element access -------------------------------------------------------

// Element e of a 16-byte chunk holding fp32 or bf16 values, widened to fp32
// (bf16 -> fp32 is exact: the bits are the top half of the fp32 pattern).
template <typename KV>
__device__ __forceinline__ float elem(const u32x4 &c, int e);
template <>
__device__ __forceinline__ float elem<float>(const u32x4 &c, int e) {
  return __uint_as_float(c[e]);
}
template <>
__device__ __forceinline__ float elem<bf16_t>(const u32x4 &c, int e) {
  const unsigned w = c[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

template <typename KV>
__device__ __forceinline__ u32x4 zero_elem(u32x4 c, int e);
template <>
__device__ __forceinline__ u32x4 zero_elem<float>(u32x4 c, int e) {
  c[e] = 0u;
  return c;
}
template <>
__device__ __forceinline__ u32x4 zero_elem<bf16_t>(u32x4 c, int e) {
  c[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  return c;
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN.
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(unsigned, b);
}

template <typename OUT>
__device__ __forceinline__ void store_out(OUT *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t *p, float v) {
  p->bits = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
}

// Four consecutive outputs (16 B fp32 or 8 B bf16, naturally aligned).
template <typename OUT>
__device__ __forceinline__ void store_out4(OUT *p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store_out4<float>(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}
template <>
__device__ __forceinline__ void store_out4<bf16_t>(bf16_t *p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// ---- cross-lane ------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within 16

// Lane l gets the value of lane l ^ 16 (within each half-wave).
__device__ __forceinline__ float xor16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
// Lane l gets the value of lane l ^ 32.
__device__ __forceinline__ float xor32(float v) {
  const int src = (int)(threadIdx.x ^ 32u) << 2;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
}

// Max / sum over the 16 lanes of each row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  v = fmaxf(v, dpp<kRowMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- work decomposition ----------------------------------------------------

struct Params {
  void *out;
  const void *query;
  const char *key_cache;
  const char *value_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float *ws_max, *ws_sum, *ws_acc;
  int64_t num_blocks;
  int num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, max_context_len;
  int partition_size, num_partitions, units, group, head_tiles;
  float scale_log2e;
};

// Linear workgroup id -> (unit, sequence, partition).  The head unit varies
// fastest: consecutive workgroups go round-robin to the 8 XCDs, so when the
// unit count is a multiple of 8 every workgroup of one head unit lands on
// the same XCD and shares its L2 (what the shared-prefix workload reuses).
struct Work {
  int unit, seq, part;
  int t0, t1;     // token range [t0, t1) of this partition
  int nparts;     // partitions of this sequence
  bool active;    // false: nothing to do (partition past the end)
};

__device__ __forceinline__ Work decode_work(const Params &p) {
  Work w;
  int id = (int)blockIdx.x;
  w.unit = id % p.units;
  id /= p.units;
  w.seq = id % p.num_seqs;
  w.part = id / p.num_seqs;
  int L = p.context_lens[w.seq];
  L = L < 0 ? 0 : (L > p.max_context_len ? p.max_context_len : L);
  if (p.partition_size > 0) {
    w.nparts = (L + p.partition_size - 1) / p.partition_size;
    w.t0 = w.part * p.partition_size;
    w.t1 = min(L, w.t0 + p.partition_size);
  } else {
    w.nparts = L > 0 ? 1 : 0;
    w.t0 = 0;
    w.t1 = L;
  }
  // Partition 0 of an empty sequence still runs, to write the zero row.
  w.active = w.part < (w.nparts > 0 ? w.nparts : 1);
  return w;
}

// Block-table reader: 64 entries per VGPR chunk, read back with readlane.
// Entries outside [0, num_blocks) are replaced by block 0, so a corrupt
// table can give a wrong row but never an out-of-bounds access.
struct TableReader {
  const int32_t *row;
  int first, count;   // blocks [first, first + count) of the row
  int chunk = -1;
  int vals = 0;
  int64_t num_blocks;

  __device__ __forceinline__ int phys(int blk) {  // blk: absolute logical block
    const int rel = blk - first;
    const int c = rel >> 6;
    if (c != chunk) {
      chunk = c;
      const int idx = (c << 6) + (int)threadIdx.x;
      vals = idx < count ? row[first + idx] : 0;
    }
    int b = __builtin_amdgcn_readlane(vals, rel & 63);
    return (unsigned)b < (unsigned long long)num_blocks ? b : 0;
  }
};

// ---- VALU kernel (MHA, or fp32 KV) ----------------------------------------
//
// Lane l = 16*g + t.  Keys: for each tile, lane l loads the 16-byte key
// chunks c = 4j + g (j < KJ) of token t; dot products are summed over the
// lane's chunks, then across g with two cross-row exchanges, leaving token
// t's logit in lanes t, t+16, t+32, t+48.  Values ([d][Bs] rows): lane l
// loads 16-byte row segments (rows j*RPI + l/LPR, tokens X*(l%LPR)..+X) and
// reads those tokens' probabilities from LDS.

#ifdef PA_WAVES_PER_EU
#define PA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(PA_WAVES_PER_EU)))
#else
#define PA_OCCUPANCY
#endif

template <typename KV, int D, int BS, typename OUT>
__global__ __launch_bounds__(64) PA_OCCUPANCY void decode_valu(Params p) {
  constexpr int X = 16 / (int)sizeof(KV);   // elements per 16-byte chunk
  constexpr int KJ = D / X / 4;             // key chunks per lane per tile
  constexpr int LPR = (int)sizeof(KV);      // lanes per 16-token value row
  constexpr int RPI = 64 / LPR;             // value rows per load
  constexpr int VJ = D / RPI;               // value loads per lane per tile
  constexpr int TPB = BS / 16;              // tiles per block
  static_assert(KJ >= 1 && VJ >= 1, "unsupported shape");

  const Work w = decode_work(p);
  if (!w.active) return;
  const int lane = (int)threadIdx.x;
  const int t = lane & 15, g = lane >> 4;
  const int qh = w.unit;
  const int kvh = qh / p.group;
  OUT *out = static_cast<OUT *>(p.out) + ((int64_t)w.seq * p.num_q_heads + qh) * D;

  if (w.t1 <= w.t0) {  // empty sequence: zero row
    for (int d = lane; d < D; d += 64) store_out<OUT>(out + d, 0.f);
    return;
  }

  // Query chunks of this lane, pre-scaled into the base-2 logit domain.
  float q[KJ][X];
  {
    const KV *qp = static_cast<const KV *>(p.query) + ((int64_t)w.seq * p.num_q_heads + qh) * D;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const u32x4 c = *reinterpret_cast<const u32x4 *>(qp + (4 * j + g) * X);
#pragma unroll
      for (int e = 0; e < X; ++e) q[j][e] = elem<KV>(c, e) * p.scale_log2e;
    }
  }

  const int64_t chunk_elems = (int64_t)D * BS;
  const int64_t head_off = (int64_t)kvh * chunk_elems;
  const int64_t block_stride = (int64_t)p.num_kv_heads * chunk_elems;
  // Per-lane element offsets inside a (block, head) chunk, tile 0.
  int koff[KJ], voff[VJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) koff[j] = ((4 * j + g) * BS + t) * X;
  const int vrow = lane / LPR, vpiece = lane % LPR;
#pragma unroll
  for (int j = 0; j < VJ; ++j) voff[j] = (j * RPI + vrow) * BS + vpiece * X;

  TableReader tab{p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq, w.t0 / BS,
                  (w.t1 + BS - 1) / BS - w.t0 / BS};
  tab.num_blocks = p.num_blocks;

  struct Tile {
    u32x4 k[KJ];
    u32x4 v[VJ];
  };
  auto load = [&](Tile &tl, int kt) {
    const int blk = kt / TPB, sub = kt % TPB;
    const int64_t base = (int64_t)tab.phys(blk) * block_stride + head_off;
    // Tile `sub` of a block: keys start 16 tokens * X further into each
    // [Bs][X] slab, values 16 tokens further into each [Bs] row.
    const KV *kb = reinterpret_cast<const KV *>(p.key_cache) + base + sub * 16 * X;
    const KV *vb = reinterpret_cast<const KV *>(p.value_cache) + base + sub * 16;
#pragma unroll
    for (int j = 0; j < KJ; ++j) tl.k[j] = *reinterpret_cast<const u32x4 *>(kb + koff[j]);
#pragma unroll
    for (int j = 0; j < VJ; ++j) tl.v[j] = *reinterpret_cast<const u32x4 *>(vb + voff[j]);
  };

  __shared__ float p_lds[2][16];
  float m = -INFINITY, lsum = 0.f;
  float o[VJ];
#pragma unroll
  for (int j = 0; j < VJ; ++j) o[j] = 0.f;

  auto compute = [&](Tile &tl, int kt) {
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < KJ; ++j)
#pragma unroll
      for (int e = 0; e < X; ++e) dot = fmaf(q[j][e], elem<KV>(tl.k[j], e), dot);
    dot += xor16(dot);
    dot += xor32(dot);
    const int pos = kt * 16 + t;
    const float s = pos < w.t1 ? dot : -INFINITY;
    const float mnew = fmaxf(m, row16_max(s));
    const float alpha = fast_exp2(m - mnew);
    const float pr = fast_exp2(s - mnew);
    lsum = lsum * alpha + pr;
    if (mnew > m) {  // uniform: every row holds the same 16 logits
#pragma unroll
      for (int j = 0; j < VJ; ++j) o[j] *= alpha;
    }
    m = mnew;
    const int buf = kt & 1;
    if (lane < 16) p_lds[buf][t] = pr;
    __syncthreads();
    if (kt * 16 + 16 > w.t1) {  // ragged last tile: unwritten slots may hold NaN
#pragma unroll
      for (int j = 0; j < VJ; ++j)
#pragma unroll
        for (int e = 0; e < X; ++e)
          if (kt * 16 + vpiece * X + e >= w.t1) tl.v[j] = zero_elem<KV>(tl.v[j], e);
    }
    float pv[X];
#pragma unroll
    for (int e = 0; e < X; ++e) pv[e] = p_lds[buf][vpiece * X + e];
#pragma unroll
    for (int j = 0; j < VJ; ++j)
#pragma unroll
      for (int e = 0; e < X; ++e) o[j] = fmaf(pv[e], elem<KV>(tl.v[j], e), o[j]);
  };

  const int k0 = w.t0 / 16, k1 = (w.t1 + 15) / 16;
  Tile buf[kPrefetch];
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s)
    if (k0 + s < k1) load(buf[s], k0 + s);
  for (int kt = k0; kt < k1; kt += kPrefetch) {
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      if (kt + s < k1) {
        compute(buf[s], kt + s);
        if (kt + s + kPrefetch < k1) load(buf[s], kt + s + kPrefetch);
      }
    }
  }

  // Combine: the sum over the 16 token lanes, the rows over their LPR lanes.
  const float ltot = row16_sum(lsum);
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    o[j] += dpp<kQuadXor1>(o[j]);
    if (LPR == 4) o[j] += dpp<kQuadXor2>(o[j]);
  }
  if (vpiece != 0) return;
  if (w.nparts <= 1) {
    const float inv = 1.f / ltot;
#pragma unroll
    for (int j = 0; j < VJ; ++j) store_out<OUT>(out + j * RPI + vrow, o[j] * inv);
  } else {
    const int64_t slot = ((int64_t)w.seq * p.num_q_heads + qh) * p.num_partitions + w.part;
#pragma unroll
    for (int j = 0; j < VJ; ++j) p.ws_acc[slot * D + j * RPI + vrow] = o[j];
    if (lane == 0) {
      p.ws_max[slot] = m;
      p.ws_sum[slot] = ltot;
    }
  }
}

// ---- MFMA kernel (bf16 KV, G >= 2) -----------------------------------------
//
// Lane l = 16*g + c.  Q.K^T as S^T[t][h] = sum_d K[t][d] Q[h][d] with
// v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 features (lane: token c,
// features of key chunk 4j + g), B = 32 features x 16 heads (lane: head c,
// same features).  The result gives lane l the logits of tokens 4g..4g+3
// for head c.  P.V as O^T[d][h] = sum_t V^T[d][t] P^T[t][h] with
// v_mfma_f32_16x16x16_bf16: A = 16 features x 16 tokens straight from the
// [d][Bs] value rows (lane: feature c, tokens 4g..4g+3), B = the
// probabilities exactly as the first product left them.  Every per-head
// quantity (max, sum, rescale) therefore lives in lane%16 = head, and the
// accumulators are rescaled by each lane's own factor.

template <int D, int BS, typename OUT>
__global__ __launch_bounds__(64) PA_OCCUPANCY void decode_mfma(Params p) {
  constexpr int QJ = D / 32;   // 16x16x32 steps over the features
  constexpr int VT = D / 16;   // 16-feature output tiles
  constexpr int TPB = BS / 16;

  const Work w = decode_work(p);
  if (!w.active) return;
  const int lane = (int)threadIdx.x;
  const int c = lane & 15, g = lane >> 4;
  const int kvh = w.unit / p.head_tiles;
  const int h = (w.unit % p.head_tiles) * 16 + c;   // head within the group
  const bool live_head = h < p.group;
  const int qh = kvh * p.group + h;
  OUT *out = static_cast<OUT *>(p.out) + ((int64_t)w.seq * p.num_q_heads + qh) * D;

  if (w.t1 <= w.t0) {  // empty sequence: zero rows
    if (live_head)
#pragma unroll
      for (int i = 0; i < VT; ++i) store_out4<OUT>(out + 16 * i + 4 * g, 0.f, 0.f, 0.f, 0.f);
    return;
  }

  u32x4 qreg[QJ];
  {
    const bf16_t *qp = static_cast<const bf16_t *>(p.query) +
                       ((int64_t)w.seq * p.num_q_heads + (live_head ? qh : 0)) * D;
#pragma unroll
    for (int j = 0; j < QJ; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(qp + (4 * j + g) * 8);
      qreg[j] = live_head ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int64_t chunk_elems = (int64_t)D * BS;
  const int64_t head_off = (int64_t)kvh * chunk_elems;
  const int64_t block_stride = (int64_t)p.num_kv_heads * chunk_elems;
  int koff[QJ], voff[VT];
#pragma unroll
  for (int j = 0; j < QJ; ++j) koff[j] = ((4 * j + g) * BS + c) * 8;
#pragma unroll
  for (int i = 0; i < VT; ++i) voff[i] = (16 * i + c) * BS + 4 * g;

  TableReader tab{p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq, w.t0 / BS,
                  (w.t1 + BS - 1) / BS - w.t0 / BS};
  tab.num_blocks = p.num_blocks;

  struct Tile {
    u32x4 k[QJ];
    u32x2 v[VT];
  };
  auto load = [&](Tile &tl, int kt) {
    const int blk = kt / TPB, sub = kt % TPB;
    const int64_t base = (int64_t)tab.phys(blk) * block_stride + head_off;
    const bf16_t *kb = reinterpret_cast<const bf16_t *>(p.key_cache) + base + sub * 16 * 8;
    const bf16_t *vb = reinterpret_cast<const bf16_t *>(p.value_cache) + base + sub * 16;
#pragma unroll
    for (int j = 0; j < QJ; ++j) tl.k[j] = *reinterpret_cast<const u32x4 *>(kb + koff[j]);
#pragma unroll
    for (int i = 0; i < VT; ++i) tl.v[i] = *reinterpret_cast<const u32x2 *>(vb + voff[i]);
  };

  float m = -INFINITY, lsum = 0.f;
  mfma_f32x4 acc[VT];
#pragma unroll
  for (int i = 0; i < VT; ++i) acc[i] = mfma_f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](Tile &tl, int kt) {
    mfma_f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < QJ; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfma_bf16x8, tl.k[j]),
                                                  __builtin_bit_cast(mfma_bf16x8, qreg[j]), s,
                                                  0, 0, 0);
    const int pos0 = kt * 16 + 4 * g;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = pos0 + r < w.t1 ? s[r] * p.scale_log2e : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const float mnew = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    const unsigned p01 = pack_bf16x2(fast_exp2(sc[0] - mnew), fast_exp2(sc[1] - mnew));
    const unsigned p23 = pack_bf16x2(fast_exp2(sc[2] - mnew), fast_exp2(sc[3] - mnew));
    // The normaliser sums the same rounded probabilities the product uses.
    lsum = lsum * alpha + ((__uint_as_float(p01 << 16) + __uint_as_float(p01 & 0xffff0000u)) +
                           (__uint_as_float(p23 << 16) + __uint_as_float(p23 & 0xffff0000u)));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // some head's max moved
#pragma unroll
      for (int i = 0; i < VT; ++i) acc[i] *= alpha;
    }
    if (kt * 16 + 16 > w.t1) {  // ragged last tile: unwritten slots may hold NaN
#pragma unroll
      for (int i = 0; i < VT; ++i) {
        if (pos0 + 0 >= w.t1) tl.v[i][0] &= 0xffff0000u;
        if (pos0 + 1 >= w.t1) tl.v[i][0] &= 0x0000ffffu;
        if (pos0 + 2 >= w.t1) tl.v[i][1] &= 0xffff0000u;
        if (pos0 + 3 >= w.t1) tl.v[i][1] &= 0x0000ffffu;
      }
    }
    const mfma_i16x4 pb = __builtin_bit_cast(mfma_i16x4, u32x2{p01, p23});
#pragma unroll
    for (int i = 0; i < VT; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mfma_i16x4, tl.v[i]),
                                                         pb, acc[i], 0, 0, 0);
  };

  const int k0 = w.t0 / 16, k1 = (w.t1 + 15) / 16;
  Tile buf[kPrefetch];
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s)
    if (k0 + s < k1) load(buf[s], k0 + s);
  for (int kt = k0; kt < k1; kt += kPrefetch) {
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      if (kt + s < k1) {
        compute(buf[s], kt + s);
        if (kt + s + kPrefetch < k1) load(buf[s], kt + s + kPrefetch);
      }
    }
  }

  float ltot = lsum + xor16(lsum);
  ltot += xor32(ltot);
  if (!live_head) return;
  if (w.nparts <= 1) {
    const float inv = 1.f / ltot;
#pragma unroll
    for (int i = 0; i < VT; ++i)
      store_out4<OUT>(out + 16 * i + 4 * g, acc[i][0] * inv, acc[i][1] * inv, acc[i][2] * inv,
                      acc[i][3] * inv);
  } else {
    const int64_t slot = ((int64_t)w.seq * p.num_q_heads + qh) * p.num_partitions + w.part;
#pragma unroll
    for (int i = 0; i < VT; ++i)
      *reinterpret_cast<f32x4 *>(p.ws_acc + slot * D + 16 * i + 4 * g) =
          f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    if (g == 0) {
      p.ws_max[slot] = m;
      p.ws_sum[slot] = ltot;
    }
  }
}

// ---- log-sum-exp merge of partitions ----------------------------------------
//
// Per (sequence, query head) with n > 1 partitions holding base-2 maxima
// m_p, sums l_p and unnormalised outputs o_p:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// accumulated in partition order.

template <int D, typename OUT>
__global__ __launch_bounds__(64) void decode_reduce(Params p) {
  const int qh = (int)blockIdx.x % p.num_q_heads;
  const int seq = (int)blockIdx.x / p.num_q_heads;
  int L = p.context_lens[seq];
  L = L < 0 ? 0 : (L > p.max_context_len ? p.max_context_len : L);
  const int n = (L + p.partition_size - 1) / p.partition_size;
  if (n <= 1) return;
  const int64_t base = ((int64_t)seq * p.num_q_heads + qh) * p.num_partitions;
  const int lane = (int)threadIdx.x;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, p.ws_max[base + i]);
  constexpr int R = D / 64;
  float num[R];
#pragma unroll
  for (int r = 0; r < R; ++r) num[r] = 0.f;
  float den = 0.f;
  for (int i = 0; i < n; ++i) {
    const float wgt = fast_exp2(p.ws_max[base + i] - M);
    den = fmaf(wgt, p.ws_sum[base + i], den);
    const float *acc = p.ws_acc + (base + i) * D;
#pragma unroll
    for (int r = 0; r < R; ++r) num[r] = fmaf(wgt, acc[r * 64 + lane], num[r]);
  }
  OUT *out = static_cast<OUT *>(p.out) + ((int64_t)seq * p.num_q_heads + qh) * D;
  const float inv = 1.f / den;
#pragma unroll
  for (int r = 0; r < R; ++r) store_out<OUT>(out + r * 64 + lane, num[r] * inv);
}

// ---- dispatch ---------------------------------------------------------------

template <typename KV, int D, int BS, typename OUT>
hipError_t launch_valu(const Params &p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_valu<KV, D, BS, OUT>), dim3(grid), dim3(64), 0, st, p);
  return hipGetLastError();
}

template <int D, int BS, typename OUT>
hipError_t launch_mfma(const Params &p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_mfma<D, BS, OUT>), dim3(grid), dim3(64), 0, st, p);
  return hipGetLastError();
}

template <typename OUT>
hipError_t dispatch_out(const DecodeArgs &a, const Params &p, bool use_mfma, int grid,
                        hipStream_t st) {
  const bool bf = a.kv_dtype == PA_BF16;
  const int D = a.head_dim, BS = a.block_size;
#define PA_CASE(d, bs)                                                              \
  if (D == d && BS == bs) {                                                         \
    if (use_mfma) return launch_mfma<d, bs, OUT>(p, grid, st);                      \
    return bf ? launch_valu<bf16_t, d, bs, OUT>(p, grid, st)                        \
              : launch_valu<float, d, bs, OUT>(p, grid, st);                        \
  }
  PA_CASE(64, 16)
  PA_CASE(64, 32)
  PA_CASE(128, 16)
  PA_CASE(128, 32)
#undef PA_CASE
  return hipErrorInvalidValue;
}

template <typename OUT>
hipError_t launch_reduce(const DecodeArgs &a, const Params &p, hipStream_t st) {
  const int grid = a.num_seqs * a.num_q_heads;
  if (a.head_dim == 64)
    hipLaunchKernelGGL((decode_reduce<64, OUT>), dim3(grid), dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL((decode_reduce<128, OUT>), dim3(grid), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int launch_decode(const DecodeArgs &a, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = a.num_q_heads / a.num_kv_heads;
  const bool use_mfma = a.kv_dtype == PA_BF16 && G >= 2;
  Params p;
  p.out = a.out;
  p.query = a.query;
  p.key_cache = static_cast<const char *>(a.key_cache);
  p.value_cache = static_cast<const char *>(a.value_cache);
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.ws_max = a.ws_max;
  p.ws_sum = a.ws_sum;
  p.ws_acc = a.ws_acc;
  p.num_blocks = a.num_blocks;
  p.num_seqs = a.num_seqs;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.max_context_len = a.max_context_len;
  p.partition_size = a.partition_size;
  p.num_partitions = a.num_partitions;
  p.group = G;
  p.head_tiles = use_mfma ? (G + 15) / 16 : 1;
  p.units = use_mfma ? a.num_kv_heads * p.head_tiles : a.num_q_heads;
  p.scale_log2e = a.scale * kLog2e;
  const int64_t grid64 = (int64_t)p.units * a.num_seqs * a.num_partitions;
  if (grid64 <= 0) return (int)hipSuccess;   // unreachable: num_seqs > 0 is checked
  if (grid64 > INT32_MAX) return (int)hipErrorInvalidConfiguration;
  const int grid = (int)grid64;
  hipError_t e;
  if (a.ev_before_main) {
    e = hipEventRecord(static_cast<hipEvent_t>(a.ev_before_main), st);
    if (e != hipSuccess) return (int)e;
  }
  e = a.out_dtype == PA_BF16 ? dispatch_out<bf16_t>(a, p, use_mfma, grid, st)
                             : dispatch_out<float>(a, p, use_mfma, grid, st);
  if (e != hipSuccess) return (int)e;
  if (a.ev_after_main) {
    e = hipEventRecord(static_cast<hipEvent_t>(a.ev_after_main), st);
    if (e != hipSuccess) return (int)e;
  }
  if (a.num_partitions <= 1) return (int)e;
  e = a.out_dtype == PA_BF16 ? launch_reduce<bf16_t>(a, p, st) : launch_reduce<float>(a, p, st);
  return (int)e;
}

}  // namespace pa
