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
// The work is cut into segments, one per (sequence, head unit), each a run
// of 16-token tiles (a 32-token block is two tiles).  A wave64 processes a
// piece -- a contiguous tile range of one segment -- keeping the running
// max / sum / output in registers and the next tile's K/V loads in flight.  A
// piece covering its whole segment writes the output row; any other piece
// writes a partial (max, sum, unnormalised output) that decode_merge
// combines exactly by log-sum-exp.
//
// Head units, chosen per call:
//  * VALU body -- one query head.  Vector-ALU dot products; used for MHA
//    (G = 1) and for fp32 KV.
//  * MFMA body -- one KV head and up to 16 of its query heads.  bf16 KV with
//    G >= 2: Q.K^T and P.V run on v_mfma_f32_16x16x32_bf16 and
//    v_mfma_f32_16x16x16_bf16 with the group's query heads on the N side of
//    both products, so each KV byte is read once for the whole group.
//
// How segments become pieces:
//  * fixed partitions (partition_size > 0, or 0 = whole segment): one
//    workgroup per (unit, sequence, partition);
//  * balanced (partition_size < 0): exactly as many waves as the GPU holds
//    at once; the tiles of all segments, laid end to end, are cut into one
//    contiguous range per wave.  No wave waits on a long segment while
//    others idle, and a segment is split only where a range ends.  Ranges
//    are weighted per XCD (workgroups are dealt round-robin to the 8 XCDs):
//    on MI355X the even-numbered XCDs stream about 10% faster than the odd
//    ones, so by default they get 10% more tiles (pa_set_balance_weights).
//    When the caller says blocks are reused across sequences
//    (PA_DECODE_KV_REUSED) and the unit count is a multiple of 8, the split
//    is instead done per XCD: 8 sub-problems, units u = x (mod 8) on waves
//    w = x (mod 8), so each KV head's blocks stay in one XCD's L2.
//
// Appending calls (the step's new tokens given): the wave that loads the
// tile holding a sequence's last position puts the new token into its
// registers, and every wave stores a share of the new tokens into their
// slots after its pieces.  Shared-prefix calls: prefix waves read the common
// blocks once per KV head for all query rows, tail waves run the balanced
// split over each sequence's own tiles, both kinds in one launch.
//
// Every reduction order is fixed by logical token position, so results are
// deterministic and independent of where the blocks sit physically.
//
// Softmax runs in base 2: logits are multiplied by scale * log2(e) and
// exponentiated with v_exp_f32; the stored partition maxima are base-2.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "pa_internal.h"
#include "pa_launch_map.h"

// Scratch of pa_paged_attention_decode_noalloc, for callers that cannot
// allocate device memory: the call's partial rows, merge counters and
// per-wave records live here instead of in a caller's workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never uses this name as an address (on the host it is only a stand-in
// for the symbol): noalloc_scratch() looks the device address up.  Calls on
// one GPU share the array, so calls that overlap on one GPU race.
static __device__ __align__(256) unsigned char scratch[pa::kNoAllocScratchBytes];

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

// Element e of a 16-byte chunk replaced by v (bit copy).  Written as
// selects over constant indices: a runtime index into a vector register
// would move the vector to scratch memory.
template <typename KV>
__device__ __forceinline__ u32x4 set_elem(u32x4 c, int e, KV v);
template <>
__device__ __forceinline__ u32x4 set_elem<float>(u32x4 c, int e, float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = k == e ? __float_as_uint(v) : c[k];
  return c;
}
template <>
__device__ __forceinline__ u32x4 set_elem<bf16_t>(u32x4 c, int e, bf16_t v) {
  const unsigned lo = v.bits, hi = (unsigned)v.bits << 16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    c[k] = 2 * k == e ? ((c[k] & 0xffff0000u) | lo) : c[k];
    c[k] = 2 * k + 1 == e ? ((c[k] & 0x0000ffffu) | hi) : c[k];
  }
  return c;
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

// Lane within the wave.  Every routine below works on one wave; workgroups
// of several waves (the merge, the shared-prefix launch) are built from them.
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// Orders this wave's LDS writes before its following LDS reads of other
// lanes' values: an exchange within one wave needs no workgroup barrier (a
// wave's LDS operations complete in order), only that the compiler keep the
// order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within 16

// Max or sum of the values of lanes l and l ^ 16 (l ^ 32), in every lane:
// v_permlane16_swap / v_permlane32_swap hand each lane both values of its
// pair (lower lane first) without a trip through LDS.  Both orders of a
// pair give the same bits (max and + are commutative).
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// K/V loads.  Streaming (NT): each block is read once in the call, so the
// loads carry the non-temporal hint and do not displace other lines; on
// MI355X this raises random 4 KiB gathers from ~6.0 to ~6.7 TB/s.  Reused
// (!NT): blocks shared by several sequences are re-read, so they are loaded
// normally and can hit in L2.
template <typename V, bool NT>
__device__ __forceinline__ V load_kv(const void *ptr) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const V *>(ptr));
  else
    return *reinterpret_cast<const V *>(ptr);
}

// ---- work decomposition ----------------------------------------------------

struct Params {
  void *out;
  const void *query;
  char *key_cache;          // written only by the appending variant
  char *value_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  // Appending variant (all null otherwise): the token at position L - 1 of
  // sequence i is new_key/new_value[i], stored into slot slots[i] (< 0: no
  // new token, position L - 1 is read from the cache like the others).
  const void *new_key;
  const void *new_value;
  const int64_t *slots;
  // Copy-on-write inside the launch (null: none): cow_src[i] >= 0 is the
  // block whose contents sequence i's last block (the new token's block,
  // slots[i] / block_size) takes.  The attention reads cow_src[i] in its
  // place, and the launch copies it over before storing the new token.
  const int64_t *cow_src;
  float *ws_max, *ws_sum, *ws_acc;   // partial rows: [piece * gu + head in unit]
  int32_t *seg_units;                // balanced: per segment, first and last owning wave
  int32_t *seg_cnt;                  // balanced: per segment, chunks merged so far (merge)
  int32_t *wave_segs;                // balanced: per wave, the segment its range starts in
  int64_t num_blocks;
  int num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, max_context_len;
  int partition_size;   // > 0 fixed partitions, 0 whole segments, < 0 balanced
  int num_partitions;   // fixed mode: partitions of the longest sequence
  int units;            // head units per sequence
  int group;            // G = Hq / Hkv
  int head_tiles;       // MFMA: 16-head tiles per KV head (1 for VALU)
  int gu;               // partial rows per piece: heads a unit can hold
  int waves;            // balanced mode: number of waves in the grid
  int xsplit;           // balanced mode: sub-problems (1, or 8 = one per XCD)
  int64_t id_stride;    // balanced mode: piece ids per sub-problem
  int xcd_prefix[9];    // balanced mode: prefix sums of the 8 per-XCD weights
  float scale_log2e;
  // Shared prefix (0 tiles when unused): every sequence's first
  // prefix_tiles * 16 tokens are the same physical blocks, those of
  // sequence 0.  The prefix waves (run_prefix) cover them for all query
  // rows at once and the balanced split only the tiles after them.
  int prefix_tiles;
  int pf_chunks, pf_chunk_tiles;   // prefix split into chunks of tiles
  int pf_rows;                     // query rows per KV head: num_seqs * group
  int pf_waves;                    // prefix waves of the launch
  float *pf_max, *pf_sum, *pf_acc; // partials [chunk][KV head][row]
};

__device__ __forceinline__ int seq_len(const Params &p, int i) {
  const int L = p.context_lens[i];
  return L < 0 ? 0 : (L > p.max_context_len ? p.max_context_len : L);
}

__device__ __forceinline__ int tiles_of(int L) { return (L + 15) >> 4; }

// Tiles of a sequence the per-sequence pieces cover: those after the
// shared prefix.
__device__ __forceinline__ int own_tiles(const Params &p, int L) {
  const int n = tiles_of(L) - p.prefix_tiles;
  return n > 0 ? n : 0;
}

// One contiguous tile range [t0/16, ceil(t1/16)) of segment (seq, unit).
struct Piece {
  int seq, unit;
  int t0, t1;       // tokens [t0, t1), t0 a multiple of 16
  bool whole;       // covers the whole segment: write the output row
  bool last;        // ends where the segment ends (t1 = L)
  int64_t id;       // partial rows id * gu + h when !whole
  // Set by the driver: the new token's slot when this piece ends with an
  // appended token at t1 - 1, else -1.
  int64_t slot;
};

// Slot of the token appended at the end of piece pc, or -1.  Out-of-range
// slots count as none, so they are neither written nor substituted.
template <int BS>
__device__ __forceinline__ int64_t append_slot(const Params &p, const Piece &pc) {
  if (p.slots == nullptr || !pc.last) return -1;
  const int64_t s = p.slots[pc.seq];
  return (s >= 0 && s < p.num_blocks * BS) ? s : -1;
}

// True when tile kt of piece pc holds the piece's appended token.
__device__ __forceinline__ bool appends_in(const Piece &pc, int kt) {
  return pc.slot >= 0 && kt == (pc.t1 - 1) >> 4;
}

// Block-table reader over blocks [first, first + count) of one table row:
// 64 entries per VGPR chunk, read back with readlane.  Blocks are read in
// order, so the chunk after the current one is requested as soon as the
// current one is entered.  Entries outside [0, num_blocks) are replaced by
// block 0, so a corrupt table can give a wrong row but never an
// out-of-bounds access.  With copy-on-write inside the launch, a
// sequence's last block is read from its copy source instead (sub_blk,
// sub_phys), by whichever piece reads it: a block of more than 16 tokens
// can be split between two pieces.
struct TableReader {
  const int32_t *row;
  int first, count;
  int chunk, vals, vals_next;
  int sub_blk;
  int64_t sub_phys;

  __device__ __forceinline__ int fetch(int c) const {
    const int idx = (c << 6) + lane_id();
    return idx < count ? row[first + idx] : 0;
  }

  // Request the first two chunks (no wait: the values are used later).
  // cow: apply the copy sources (the per-sequence pieces, not the shared
  // prefix's, which never holds a new token's block).
  __device__ __forceinline__ void start(const Params &p, const Piece &pc, int bs,
                                        bool cow = true) {
    row = p.block_tables + (int64_t)pc.seq * p.max_blocks_per_seq;
    first = pc.t0 / bs;
    count = (pc.t1 + bs - 1) / bs - first;
    chunk = 0;
    vals = fetch(0);
    vals_next = count > 64 ? fetch(1) : 0;
    sub_blk = -1;
    sub_phys = 0;
    if (cow && p.cow_src != nullptr) {
      sub_phys = p.cow_src[pc.seq];
      const int last = (seq_len(p, pc.seq) - 1) / bs;   // the sequence's last block
      if (sub_phys >= 0 && sub_phys < p.num_blocks && last >= first && last < first + count)
        sub_blk = last;
    }
  }

  __device__ __forceinline__ int64_t phys(int blk, int64_t num_blocks) {  // absolute logical block
    if (blk == sub_blk) return sub_phys;
    const int rel = blk - first;
    const int c = rel >> 6;
    if (c != chunk) {
      vals = c == chunk + 1 ? vals_next : fetch(c);
      chunk = c;
      vals_next = ((c + 1) << 6) < count ? fetch(c + 1) : 0;
    }
    const int b = __builtin_amdgcn_readlane(vals, rel & 63);
    return (unsigned)b < (unsigned long long)num_blocks ? b : 0;
  }
};

// Context lengths of sequences [base, base + 64) in one VGPR, read back with
// readlane; clamped like seq_len().
struct LenWindow {
  int base, vals;
  __device__ __forceinline__ void load(const Params &p, int b) {
    base = b;
    const int i = b + lane_id();
    vals = i < p.num_seqs ? seq_len(p, i) : 0;
  }
  __device__ __forceinline__ int get(const Params &p, int seq) {
    if (seq - base >= 64 || seq < base) load(p, seq);
    return __builtin_amdgcn_readlane(vals, seq - base);
  }
};

// ---- the streaming driver ----------------------------------------------------
//
// A wave walks its pieces as one continuous stream of tiles, two tile
// buffers deep: while one tile is computed the next one is in flight.  The
// loader steps into the next piece as soon as the current one is fully
// requested, so the first tiles of a piece are in flight while the last
// tile of the previous one is computed.  One piece further on (the peeked
// piece) has its first table chunk requested early, so stepping in never
// waits on a table read.  With two buffers the loader is never more than one
// piece ahead of the compute side: it holds that piece's query registers
// until the compute side reaches it.
//
// Body provides Tile, QRaw (query registers as loaded), QReady (as used),
// Acc (running max / sum / output) and: kBlockSize, head_offset, load_q,
// ready_q, load_tile, init, compute, finish.

template <class Body, class Gen>
__device__ __forceinline__ void stream_pieces(const Params &p, Gen &gen, float (&p_lds)[2][16]) {
  using Tile = typename Body::Tile;
  using QRaw = typename Body::QRaw;
  using QReady = typename Body::QReady;
  using Acc = typename Body::Acc;
  constexpr int BS = Body::kBlockSize;

  Piece cp;                       // piece being computed
  if (!gen.next(cp)) return;
  cp.slot = append_slot<BS>(p, cp);
  Piece lp = cp;                  // piece being loaded
  Piece pk;                       // peeked piece after lp (valid if has_pk)
  bool has_pk = gen.next(pk);
  TableReader tab, tab_pk;
  tab.start(p, lp, BS);
  if (has_pk) tab_pk.start(p, pk, BS);
  QRaw qraw, qraw_next;
  Body::load_q(p, cp, qraw);
  QReady q;
  int64_t head_off = Body::head_offset(p, lp.unit);
  int lk = lp.t0 >> 4, lk1 = (lp.t1 + 15) >> 4;   // loader tile cursor
  int ck = cp.t0 >> 4, ck1 = (cp.t1 + 15) >> 4;   // compute tile cursor
  bool ahead = false;             // lp is the piece after cp
  Acc acc;
  Body::init(acc);

  // Request the next tile of the stream into tl; false when none is left.
  auto load_next = [&](Tile &tl) -> bool {
    if (lk >= lk1) {
      if (!has_pk) return false;
      // Step into the peeked piece (its first table chunk is already
      // requested) and request its query.
      lp = pk;
      lp.slot = append_slot<BS>(p, lp);
      tab = tab_pk;
      head_off = Body::head_offset(p, lp.unit);
      lk = lp.t0 >> 4;
      lk1 = (lp.t1 + 15) >> 4;
      Body::load_q(p, lp, qraw_next);
      ahead = true;
      has_pk = gen.next(pk);
      if (has_pk) tab_pk.start(p, pk, BS);
    }
    Body::load_tile(p, tab, head_off, lk, tl);
    ++lk;
    return true;
  };

  // Compute one tile; at the end of a piece write its result and move to
  // the next.  False when the last piece is done.  When cp ends, the loader
  // has already tried to step past it (every tile of cp was requested at
  // least one load earlier), so `ahead` tells whether a next piece exists.
  auto consume = [&](Tile &tl) -> bool {
    Body::compute(p, cp, q, acc, tl, ck, p_lds);
    if (++ck < ck1) return true;
    Body::finish(p, cp, acc);
    if (!ahead) return false;
    cp = lp;
    Body::ready_q(p, cp, qraw_next, q);
    ahead = false;
    ck = cp.t0 >> 4;
    ck1 = (cp.t1 + 15) >> 4;
    Body::init(acc);
    return true;
  };

  Tile b0, b1;
  bool h0 = load_next(b0);
  bool h1 = load_next(b1);
  Body::ready_q(p, cp, qraw, q);   // after the first tiles are requested
  // A wave that has just computed a tile issues the next tile's loads at a
  // raised priority, ahead of the other wave's arithmetic on the SIMD
  // (70B-shaped main kernel about 1 us faster over 7 same-box A/B rounds).
  while (h0) {
    if (!consume(b0)) return;
    __builtin_amdgcn_s_setprio(2);
    h0 = load_next(b0);
    __builtin_amdgcn_s_setprio(0);
    if (!h1) return;
    if (!consume(b1)) return;
    __builtin_amdgcn_s_setprio(2);
    h1 = load_next(b1);
    __builtin_amdgcn_s_setprio(0);
  }
}

// ---- VALU body (MHA, or fp32 KV) --------------------------------------------
//
// Lane l = 16*g + t.  Keys: for each tile, lane l loads the 16-byte key
// chunks c = 4j + g (j < KJ) of token t; dot products are summed over the
// lane's chunks, then across g with two cross-row exchanges, leaving token
// t's logit in lanes t, t+16, t+32, t+48.  Values ([d][16] rows): lane l
// loads 16-byte row segments (rows j*RPI + l/LPR, tokens X*(l%LPR)..+X) and
// reads those tokens' probabilities from LDS.

template <typename KV, int D, int BS, typename OUT, bool NT>
struct ValuBody {
  using KVT = KV;
  static constexpr int kBlockSize = BS, kHeadDim = D;
  static constexpr bool kStreams = NT;
  static constexpr int kWavesPerEU = sizeof(KV) == 4 && D == 128 ? 1 : 2;
  static constexpr int X = 16 / (int)sizeof(KV);   // elements per 16-byte chunk
  static constexpr int KJ = D / X / 4;             // key chunks per lane per tile
  static constexpr int LPR = (int)sizeof(KV);      // lanes per 16-token value row
  static constexpr int RPI = 64 / LPR;             // value rows per load
  static constexpr int VJ = D / RPI;               // value loads per lane per tile
  static constexpr int TPB = BS / 16;              // tiles per block
  static_assert(KJ >= 1 && VJ >= 1, "unsupported shape");

  struct Tile {
    u32x4 k[KJ];
    u32x4 v[VJ];
  };
  struct QRaw {
    u32x4 c[KJ];
  };
  struct QReady {
    float v[KJ][X];
  };
  struct Acc {
    float m, lsum;
    float o[VJ];
  };

  __device__ static void zero_rows(const Params &p, int seq, int unit) {
    OUT *out = static_cast<OUT *>(p.out) + ((int64_t)seq * p.num_q_heads + unit) * D;
    for (int d = lane_id(); d < D; d += 64) store_out<OUT>(out + d, 0.f);
  }

  __device__ static int64_t head_offset(const Params &p, int unit) {
    return (int64_t)(unit / p.group) * D * BS;
  }

  // The lane's key chunks c = 4j + g of query head `unit`.
  __device__ static void load_q(const Params &p, const Piece &pc, QRaw &q) {
    const int g = lane_id() >> 4;
    const KV *qp =
        static_cast<const KV *>(p.query) + ((int64_t)pc.seq * p.num_q_heads + pc.unit) * D;
#pragma unroll
    for (int j = 0; j < KJ; ++j) q.c[j] = *reinterpret_cast<const u32x4 *>(qp + (4 * j + g) * X);
  }

  // Widen and pre-scale into the base-2 logit domain.
  __device__ static void ready_q(const Params &p, const Piece &, const QRaw &raw, QReady &q) {
#pragma unroll
    for (int j = 0; j < KJ; ++j)
#pragma unroll
      for (int e = 0; e < X; ++e) q.v[j][e] = elem<KV>(raw.c[j], e) * p.scale_log2e;
  }

  __device__ static void load_tile(const Params &p, TableReader &tab, int64_t head_off, int kt,
                                   Tile &tl) {
    const int lane = lane_id();
    const int t = lane & 15, g = lane >> 4;
    const int blk = kt / TPB, sub = kt % TPB;
    const int64_t base = (int64_t)tab.phys(blk, p.num_blocks) * p.num_kv_heads * D * BS + head_off;
    // Tile `sub` of a block: keys start 16 tokens * X further into each
    // [Bs][X] slab; values are the sub-th [D][16] group.
    const KV *kb = reinterpret_cast<const KV *>(p.key_cache) + base + sub * 16 * X;
    const KV *vb = reinterpret_cast<const KV *>(p.value_cache) + base + sub * D * 16;
#pragma unroll
    for (int j = 0; j < KJ; ++j) tl.k[j] = load_kv<u32x4, NT>(kb + ((4 * j + g) * BS + t) * X);
#pragma unroll
    for (int j = 0; j < VJ; ++j)
      tl.v[j] = load_kv<u32x4, NT>(vb + (j * RPI + lane / LPR) * 16 + (lane % LPR) * X);
  }

  __device__ static void init(Acc &a) {
    a.m = -INFINITY;
    a.lsum = 0.f;
#pragma unroll
    for (int j = 0; j < VJ; ++j) a.o[j] = 0.f;
  }

  __device__ static void compute(const Params &p, const Piece &pc, const QReady &q, Acc &a,
                                 Tile &tl, int kt, float (&p_lds)[2][16]) {
    if (appends_in(pc, kt)) patch_tile(p, pc, tl, kt);
    const int lane = lane_id();
    const int t = lane & 15, vpiece = lane % LPR;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < KJ; ++j)
#pragma unroll
      for (int e = 0; e < X; ++e) dot = fmaf(q.v[j][e], elem<KV>(tl.k[j], e), dot);
    dot = pair32_sum(pair16_sum(dot));
    const float sc = kt * 16 + t < pc.t1 ? dot : -INFINITY;
    const float mnew = fmaxf(a.m, row16_max(sc));
    const float alpha = fast_exp2(a.m - mnew);
    const float pr = fast_exp2(sc - mnew);
    a.lsum = a.lsum * alpha + pr;
    if (mnew > a.m) {  // uniform: every row holds the same 16 logits
#pragma unroll
      for (int j = 0; j < VJ; ++j) a.o[j] *= alpha;
    }
    a.m = mnew;
    const int buf = kt & 1;
    if (lane < 16) p_lds[buf][t] = pr;
    wave_lds_sync();
    if (kt * 16 + 16 > pc.t1) {  // ragged last tile: unwritten slots may hold NaN
#pragma unroll
      for (int j = 0; j < VJ; ++j)
#pragma unroll
        for (int e = 0; e < X; ++e)
          if (kt * 16 + vpiece * X + e >= pc.t1) tl.v[j] = zero_elem<KV>(tl.v[j], e);
    }
    float pv[X];
#pragma unroll
    for (int e = 0; e < X; ++e) pv[e] = p_lds[buf][vpiece * X + e];
#pragma unroll
    for (int j = 0; j < VJ; ++j)
#pragma unroll
      for (int e = 0; e < X; ++e) a.o[j] = fmaf(pv[e], elem<KV>(tl.v[j], e), a.o[j]);
  }

  // Put the appended token (position t1 - 1, lane row r0 of tile kt) into
  // the loaded tile, as if it had been read from its slot.  The slot itself
  // is written at the end of the launch (store_new_tokens).
  __device__ static void patch_tile(const Params &p, const Piece &pc, Tile &tl, int) {
    const int lane = lane_id();
    const int t = lane & 15, g = lane >> 4, vpiece = lane % LPR;
    const int r0 = (pc.t1 - 1) & 15;
    const int kvh = pc.unit / p.group;
    const int64_t src = ((int64_t)pc.seq * p.num_kv_heads + kvh) * D;
    const KV *nk = static_cast<const KV *>(p.new_key) + src;
    const KV *nv = static_cast<const KV *>(p.new_value) + src;
    // Every lane loads and selects: no divergent branch around the loads.
    u32x4 kn[KJ];
    KV vn[VJ];
#pragma unroll
    for (int j = 0; j < KJ; ++j) kn[j] = *reinterpret_cast<const u32x4 *>(nk + (4 * j + g) * X);
#pragma unroll
    for (int j = 0; j < VJ; ++j) vn[j] = nv[j * RPI + lane / LPR];
    const bool krow = t == r0, vrow = r0 / X == vpiece;
#pragma unroll
    for (int j = 0; j < KJ; ++j) tl.k[j] = krow ? kn[j] : tl.k[j];
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      const u32x4 w = set_elem<KV>(tl.v[j], r0 % X, vn[j]);
      tl.v[j] = vrow ? w : tl.v[j];
    }
  }

  // Combine the sum over the 16 token lanes and each row over its LPR lanes,
  // then write the output row or the partial.
  __device__ static void finish(const Params &p, const Piece &pc, Acc &a) {
    const int lane = lane_id();
    const int vrow = lane / LPR;
    const float ltot = row16_sum(a.lsum);
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      a.o[j] += dpp<kQuadXor1>(a.o[j]);
      if (LPR == 4) a.o[j] += dpp<kQuadXor2>(a.o[j]);
    }
    if (lane % LPR == 0) {
      if (pc.whole) {
        OUT *out = static_cast<OUT *>(p.out) + ((int64_t)pc.seq * p.num_q_heads + pc.unit) * D;
        const float inv = 1.f / ltot;
#pragma unroll
        for (int j = 0; j < VJ; ++j) store_out<OUT>(out + j * RPI + vrow, a.o[j] * inv);
      } else {
        const int64_t row = pc.id * p.gu;
#pragma unroll
        for (int j = 0; j < VJ; ++j) p.ws_acc[row * D + j * RPI + vrow] = a.o[j];
        if (lane == 0) {
          p.ws_max[row] = a.m;
          p.ws_sum[row] = ltot;
        }
      }
    }
  }
};

// ---- MFMA body (bf16 KV, G >= 2) ---------------------------------------------
//
// Lane l = 16*g + c.  Q.K^T as S^T[t][h] = sum_d K[t][d] Q[h][d] with
// v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 features (lane: token c,
// features of key chunk 4j + g), B = 32 features x 16 heads (lane: head c,
// same features).  The result gives lane l the logits of tokens 4g..4g+3
// for head c.  P.V as O^T[d][h] = sum_t V^T[d][t] P^T[t][h] with
// v_mfma_f32_16x16x16_bf16: A = 16 features x 16 tokens straight from the
// [d][16] value rows (lane: feature c, tokens 4g..4g+3), B = the
// probabilities exactly as the first product left them.  Every per-head
// quantity (max, sum, rescale) therefore lives in lane%16 = head, and the
// accumulators are rescaled by each lane's own factor.

template <int D, int BS, typename OUT, bool NT>
struct MfmaBody {
  using KVT = bf16_t;
  static constexpr int kBlockSize = BS, kHeadDim = D;
  static constexpr bool kStreams = NT;
  static constexpr int kWavesPerEU = 2;
  static constexpr int QJ = D / 32;   // 16x16x32 steps over the features
  static constexpr int VT = D / 16;   // 16-feature output tiles
  static constexpr int TPB = BS / 16;

  struct Tile {
    u32x4 k[QJ];
    u32x2 v[VT];
  };
  struct QRaw {
    u32x4 c[QJ];
  };
  using QReady = QRaw;
  struct Acc {
    float m, lsum;
    mfma_f32x4 o[VT];
  };

  // Head of the group this lane's column holds, and whether it exists.
  __device__ static int group_head(const Params &p, int unit) {
    return (unit % p.head_tiles) * 16 + (lane_id() & 15);
  }

  __device__ static void zero_rows(const Params &p, int seq, int unit) {
    const int g = lane_id() >> 4;
    const int h = group_head(p, unit);
    if (h >= p.group) return;
    OUT *out = static_cast<OUT *>(p.out) +
               ((int64_t)seq * p.num_q_heads + (unit / p.head_tiles) * p.group + h) * D;
#pragma unroll
    for (int i = 0; i < VT; ++i) store_out4<OUT>(out + 16 * i + 4 * g, 0.f, 0.f, 0.f, 0.f);
  }

  __device__ static int64_t head_offset(const Params &p, int unit) {
    return (int64_t)(unit / p.head_tiles) * D * BS;
  }

  __device__ static void load_q(const Params &p, const Piece &pc, QRaw &q) {
    const int g = lane_id() >> 4;
    const int h = group_head(p, pc.unit);
    const int qh = (pc.unit / p.head_tiles) * p.group + (h < p.group ? h : 0);
    const bf16_t *qp = static_cast<const bf16_t *>(p.query) +
                       ((int64_t)pc.seq * p.num_q_heads + qh) * D;
#pragma unroll
    for (int j = 0; j < QJ; ++j) q.c[j] = *reinterpret_cast<const u32x4 *>(qp + (4 * j + g) * 8);
  }

  // Columns past the group's last head (a group of G < 16, or the last tile
  // of G > 16) hold a copy of a real head's query: every column runs through
  // both products on its own, so they cost nothing but unused outputs,
  // which finish() never stores.
  __device__ static void ready_q(const Params &, const Piece &, const QRaw &raw, QReady &q) {
    q = raw;
  }

  __device__ static void load_tile(const Params &p, TableReader &tab, int64_t head_off, int kt,
                                   Tile &tl) {
    const int lane = lane_id();
    const int c = lane & 15, g = lane >> 4;
    const int blk = kt / TPB, sub = kt % TPB;
    const int64_t base = (int64_t)tab.phys(blk, p.num_blocks) * p.num_kv_heads * D * BS + head_off;
    const bf16_t *kb = reinterpret_cast<const bf16_t *>(p.key_cache) + base + sub * 16 * 8;
    const bf16_t *vb = reinterpret_cast<const bf16_t *>(p.value_cache) + base + sub * D * 16;
#pragma unroll
    for (int j = 0; j < QJ; ++j) tl.k[j] = load_kv<u32x4, NT>(kb + ((4 * j + g) * BS + c) * 8);
#pragma unroll
    for (int i = 0; i < VT; ++i) tl.v[i] = load_kv<u32x2, NT>(vb + (16 * i + c) * 16 + 4 * g);
  }

  __device__ static void init(Acc &a) {
    a.m = -INFINITY;
    a.lsum = 0.f;
#pragma unroll
    for (int i = 0; i < VT; ++i) a.o[i] = mfma_f32x4{0.f, 0.f, 0.f, 0.f};
  }

  __device__ static void compute(const Params &p, const Piece &pc, const QReady &q, Acc &a,
                                 Tile &tl, int kt, float (&)[2][16]) {
    if (appends_in(pc, kt)) patch_tile(p, pc, tl, kt);
    const int g = lane_id() >> 4;
    mfma_f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < QJ; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfma_bf16x8, tl.k[j]),
                                                  __builtin_bit_cast(mfma_bf16x8, q.c[j]), s, 0,
                                                  0, 0);
    const int pos0 = kt * 16 + 4 * g;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = pos0 + r < pc.t1 ? s[r] * p.scale_log2e : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = pair32_max(pair16_max(mx));
    const float mnew = fmaxf(a.m, mx);
    const float alpha = fast_exp2(a.m - mnew);
    a.m = mnew;
    const unsigned p01 = pack_bf16x2(fast_exp2(sc[0] - mnew), fast_exp2(sc[1] - mnew));
    const unsigned p23 = pack_bf16x2(fast_exp2(sc[2] - mnew), fast_exp2(sc[3] - mnew));
    // The normaliser sums the same rounded probabilities the product uses.
    a.lsum = a.lsum * alpha + ((__uint_as_float(p01 << 16) + __uint_as_float(p01 & 0xffff0000u)) +
                               (__uint_as_float(p23 << 16) + __uint_as_float(p23 & 0xffff0000u)));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // some head's max moved
#pragma unroll
      for (int i = 0; i < VT; ++i) a.o[i] *= alpha;
    }
    if (kt * 16 + 16 > pc.t1) {  // ragged last tile: unwritten slots may hold NaN
#pragma unroll
      for (int i = 0; i < VT; ++i) {
        if (pos0 + 0 >= pc.t1) tl.v[i][0] &= 0xffff0000u;
        if (pos0 + 1 >= pc.t1) tl.v[i][0] &= 0x0000ffffu;
        if (pos0 + 2 >= pc.t1) tl.v[i][1] &= 0xffff0000u;
        if (pos0 + 3 >= pc.t1) tl.v[i][1] &= 0x0000ffffu;
      }
    }
    const mfma_i16x4 pb = __builtin_bit_cast(mfma_i16x4, u32x2{p01, p23});
#pragma unroll
    for (int i = 0; i < VT; ++i)
      a.o[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mfma_i16x4, tl.v[i]),
                                                         pb, a.o[i], 0, 0, 0);
  }

  // Put the appended token (position t1 - 1, row r0 of tile kt) into the
  // loaded tile, as if it had been read from its slot.  The slot itself is
  // written at the end of the launch (store_new_tokens).
  __device__ static void patch_tile(const Params &p, const Piece &pc, Tile &tl, int) {
    const int lane = lane_id();
    const int c = lane & 15, g = lane >> 4;
    const int r0 = (pc.t1 - 1) & 15;
    const int kvh = pc.unit / p.head_tiles;
    const int64_t src = ((int64_t)pc.seq * p.num_kv_heads + kvh) * D;
    const bf16_t *nk = static_cast<const bf16_t *>(p.new_key) + src;
    const bf16_t *nv = static_cast<const bf16_t *>(p.new_value) + src;
    // Every lane loads and selects (no divergent branches): see ValuBody.
    u32x4 kn[QJ];
    bf16_t vn[VT];
#pragma unroll
    for (int j = 0; j < QJ; ++j) kn[j] = *reinterpret_cast<const u32x4 *>(nk + (4 * j + g) * 8);
#pragma unroll
    for (int i = 0; i < VT; ++i) vn[i] = nv[16 * i + c];
    const bool krow = c == r0, vrow = g == (r0 >> 2);
    const int e = r0 & 3;
#pragma unroll
    for (int j = 0; j < QJ; ++j) tl.k[j] = krow ? kn[j] : tl.k[j];
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      const u32x4 w = set_elem<bf16_t>(u32x4{tl.v[i][0], tl.v[i][1], 0u, 0u}, e, vn[i]);
      tl.v[i] = vrow ? u32x2{w[0], w[1]} : tl.v[i];
    }
  }

  __device__ static void finish(const Params &p, const Piece &pc, Acc &a) {
    const int g = lane_id() >> 4, hh = lane_id() & 15;
    const float ltot = pair32_sum(pair16_sum(a.lsum));
    const int h = group_head(p, pc.unit);
    if (h >= p.group) return;
    const int qh = (pc.unit / p.head_tiles) * p.group + h;
    if (pc.whole) {
      OUT *out = static_cast<OUT *>(p.out) + ((int64_t)pc.seq * p.num_q_heads + qh) * D;
      const float inv = 1.f / ltot;
#pragma unroll
      for (int i = 0; i < VT; ++i)
        store_out4<OUT>(out + 16 * i + 4 * g, a.o[i][0] * inv, a.o[i][1] * inv, a.o[i][2] * inv,
                        a.o[i][3] * inv);
    } else {
      const int64_t row = pc.id * p.gu + hh;
#pragma unroll
      for (int i = 0; i < VT; ++i)
        *reinterpret_cast<f32x4 *>(p.ws_acc + row * D + 16 * i + 4 * g) =
            f32x4{a.o[i][0], a.o[i][1], a.o[i][2], a.o[i][3]};
      if (g == 0) {
        p.ws_max[row] = a.m;
        p.ws_sum[row] = ltot;
      }
    }
  }
};

// ---- grid strategies ---------------------------------------------------------

// Waves per SIMD the body is compiled for (Body::kWavesPerEU): two, so that
// enough bytes are in flight; one for fp32 K/V at d = 128, whose two 16 KiB
// tile buffers and query registers do not fit in half the register file
// (at two it spilled ~300 bytes per lane to scratch) and which keeps the
// same bytes in flight per CU with one.
#define PA_OCCUPANCY(Body) __attribute__((amdgpu_waves_per_eu(Body::kWavesPerEU)))

// Fixed partitions: workgroup id -> (unit, sequence, partition), the unit
// varying fastest.  Consecutive workgroups go round-robin to the 8 XCDs, so
// when the unit count is a multiple of 8 every workgroup of one head unit
// lands on the same XCD and shares its L2 (what shared prefixes reuse).
struct OnePiece {
  Piece pc;
  bool given;
  __device__ bool next(Piece &out) {
    if (given) return false;
    given = true;
    out = pc;
    return true;
  }
};

// The appending variant's cache write: each new token's K and V go into its
// slot, for every sequence with a slot in the pool, as reshape_and_cache
// writes them.  With copy-on-write inside the launch, the (sequence, KV
// head)'s part of the copy source block is first copied over the slot's
// block, as copy_blocks copies it (the source is never written here, and
// the slot's block is read by no wave: its reader reads the source).  No
// wave of the launch reads these bytes from memory (the tile holding a new
// token is patched in registers), so the stores wait
// until the wave has finished its pieces: stores issued between the reads
// slow the reads of every wave.  Wave w of n stores the (sequence, KV head)
// pairs j = n - 1 - w, j + n, ...: the last waves to start take the first
// pairs, so a grid larger than the GPU stores from its last waves.
//
// The first of those pairs can be staged (TokenStash): its slot, copy source
// and token are requested at the start of the wave and parked in LDS, so
// the end of the wave waits on no global read before its stores.
template <class Body>
struct TokenStash {
  using KV = typename Body::KVT;
  static constexpr int X = 16 / (int)sizeof(KV);
  static constexpr int C = Body::kHeadDim / X;   // 16-byte chunks of one K (or V) row
  static_assert(2 * C <= 64, "one wave holds the token's K and V chunks");
  static constexpr int kLdsChunks = 2 * C + 1;   // K chunks, V chunks, (slot, source)

  // The pair wave w of n stores first, or -1.
  __device__ static int64_t first_pair(const Params &p, int64_t w, int64_t n) {
    const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads, j = n - 1 - w;
    return p.slots != nullptr && j >= 0 && j < pairs ? j : -1;
  }

  int64_t j, slot, src;
  u32x4 chunk;   // lane c < C: K chunk c; C <= lane < 2C: V chunk lane - C

  __device__ __forceinline__ void request(const Params &p, int64_t w, int64_t n) {
    j = first_pair(p, w, n);
    if (j < 0) return;
    const int seq = (int)(j / p.num_kv_heads), lane = lane_id();
    slot = p.slots[seq];
    src = p.cow_src != nullptr ? p.cow_src[seq] : -1;
    const KV *row = static_cast<const KV *>(lane < C ? p.new_key : p.new_value) + j * Body::kHeadDim;
    if (lane < 2 * C) chunk = *reinterpret_cast<const u32x4 *>(row + (lane % C) * X);
  }
  // Once the loads have arrived (after the set-up lengths, requested later).
  __device__ __forceinline__ void park(u32x4 *lds) const {
    if (j < 0) return;
    const int lane = lane_id();
    if (lane < 2 * C) lds[lane] = chunk;
    if (lane == 0) {
      union {
        int64_t s[2];
        u32x4 v;
      } u;
      u.s[0] = slot;
      u.s[1] = src;
      lds[2 * C] = u.v;
    }
  }
};

// Store pair j's token: K chunks and V elements from kp / vp (global input
// or the stash in LDS), after copying the copy source's part of the block
// when there is one.
template <class Body>
__device__ __forceinline__ void store_token_pair(const Params &p, int64_t j, int64_t slot,
                                                 int64_t src, const typename Body::KVT *kp,
                                                 const typename Body::KVT *vp) {
  using KV = typename Body::KVT;
  constexpr int D = Body::kHeadDim, BS = Body::kBlockSize;
  constexpr int X = 16 / (int)sizeof(KV);
  const int lane = lane_id();
  if (slot < 0 || slot >= p.num_blocks * BS) return;
  const int o = (int)(slot % BS);
  const int64_t base = (slot / BS * p.num_kv_heads + j % p.num_kv_heads) * (int64_t)D * BS;
  if (src >= 0 && src < p.num_blocks && src != slot / BS) {
    const int64_t sbase = (src * p.num_kv_heads + j % p.num_kv_heads) * (int64_t)D * BS;
    const u32x4 *ks = reinterpret_cast<const u32x4 *>(reinterpret_cast<const KV *>(p.key_cache) + sbase);
    const u32x4 *vs = reinterpret_cast<const u32x4 *>(reinterpret_cast<const KV *>(p.value_cache) + sbase);
    u32x4 *kd = reinterpret_cast<u32x4 *>(reinterpret_cast<KV *>(p.key_cache) + base);
    u32x4 *vd = reinterpret_cast<u32x4 *>(reinterpret_cast<KV *>(p.value_cache) + base);
    for (int i = lane; i < D * BS / X; i += 64) {
      const u32x4 a = ks[i], b = vs[i];
      kd[i] = a;
      vd[i] = b;
    }
    // The token's stores below overwrite part of these: let these land first.
    __builtin_amdgcn_s_waitcnt(0);
  }
  KV *kc = reinterpret_cast<KV *>(p.key_cache) + base + o * X;
  KV *vc = reinterpret_cast<KV *>(p.value_cache) + base + (o / 16) * D * 16 + o % 16;
  for (int c = lane; c < D / X; c += 64)   // key chunk c: x features of the token
    *reinterpret_cast<u32x4 *>(kc + c * BS * X) = *reinterpret_cast<const u32x4 *>(kp + c * X);
  for (int e = lane; e < D; e += 64) vc[e * 16] = vp[e];   // value row e of its group
}

// Wave w of n: its pairs j = n - 1 - w, + n, ...; with `stash`, the first
// one from the TokenStash parked there.
template <class Body>
__device__ __forceinline__ void store_new_tokens(const Params &p, int64_t w, int64_t n,
                                                 const u32x4 *stash = nullptr) {
  using KV = typename Body::KVT;
  constexpr int D = Body::kHeadDim;
  if (p.slots == nullptr) return;
  const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
  int64_t j = n - 1 - w;
  if (stash != nullptr && TokenStash<Body>::first_pair(p, w, n) >= 0) {
    constexpr int C = TokenStash<Body>::C;
    union {
      int64_t s[2];
      u32x4 v;
    } u;
    u.v = stash[2 * C];
    const KV *kp = reinterpret_cast<const KV *>(stash), *vp = reinterpret_cast<const KV *>(stash + C);
    store_token_pair<Body>(p, j, u.s[0], u.s[1], kp, vp);
    j += n;
  }
  for (; j < pairs; j += n) {
    const int seq = (int)(j / p.num_kv_heads);
    const int64_t src = p.cow_src != nullptr ? p.cow_src[seq] : -1;
    store_token_pair<Body>(p, j, p.slots[seq], src, static_cast<const KV *>(p.new_key) + j * D,
                           static_cast<const KV *>(p.new_value) + j * D);
  }
}

template <class Body>
__device__ __forceinline__ void run_fixed(const Params &p, float (&p_lds)[2][16]) {
  int id = (int)blockIdx.x;
  const int unit = id % p.units;
  id /= p.units;
  const int seq = id % p.num_seqs;
  const int part = id / p.num_seqs;
  const int L = seq_len(p, seq);
  int nparts, t0, t1;
  if (p.partition_size > 0) {
    nparts = (L + p.partition_size - 1) / p.partition_size;
    t0 = part * p.partition_size;
    t1 = min(L, t0 + p.partition_size);
  } else {
    nparts = L > 0 ? 1 : 0;
    t0 = 0;
    t1 = L;
  }
  if (L == 0) {   // the zero row, written once
    if (part == 0) Body::zero_rows(p, seq, unit);
    return;
  }
  if (part >= nparts) return;
  OnePiece gen{Piece{seq, unit, t0, t1, nparts == 1, part == nparts - 1,
                     ((int64_t)seq * p.units + unit) * p.num_partitions + part, -1},
               false};
  stream_pieces<Body>(p, gen, p_lds);
}

template <class Body>
__global__ __launch_bounds__(64) PA_OCCUPANCY(Body) void decode_fixed(Params p) {
  __shared__ float p_lds[2][16];
  run_fixed<Body>(p, p_lds);
  store_new_tokens<Body>(p, blockIdx.x, gridDim.x);
}

// Sum over the wave (all lanes get it): within each row of 16 lanes by DPP,
// then over the row pairs by lane-pair swaps; no LDS round trip.
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_mov_dpp(v, kQuadXor1, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, kQuadXor2, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, kRowHalfMirror, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, kRowMirror, 0xF, 0xF, false);
  const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = (int)(r16[0] + r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return (int)(r32[0] + r32[1]);
}

// Inclusive prefix sum over the wave's lanes: within each row of 16 lanes by
// DPP row shifts (a lane shifted in from outside the row adds 0), then each
// row adds the totals of the rows before it.
__device__ __forceinline__ int wave_incl_scan(int v) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr8, 0xF, 0xF, false);
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane_id() >> 4;
  return v + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Extra tiles each nonempty segment counts for in the balanced split, placed
// after its real tiles on the tile line: a range that touches more segments
// (more pieces: query loads, table starts, partial rows) gets fewer tiles.
// No range ever holds a virtual tile between two real tiles of a segment,
// so a segment's owning waves stay consecutive.
#ifndef PA_SEGMENT_COST
#define PA_SEGMENT_COST 4
#endif
constexpr int kSegmentCost = PA_SEGMENT_COST;

// Extent of a segment of n real tiles on the balanced split's tile line.
__device__ __forceinline__ int seg_extent(int n) { return n > 0 ? n + kSegmentCost : 0; }

// The clamped context lengths a wave needs at set-up: the split's total and
// its search both run over every sequence.  Up to 64 * kLenRegs sequences
// are requested in one round of loads and kept in registers (lane l of
// register r: sequence 64 r + l), so set-up waits on memory once instead of
// once per 64 sequences for the total and again for the search.  Larger
// batches read each 64-sequence chunk from memory when it is needed.
constexpr int kLenRegs = 8;
struct SetupLens {
  int v[kLenRegs];
  bool held;
  __device__ __forceinline__ void load(const Params &p) {
    held = p.num_seqs <= 64 * kLenRegs;
    if (!held) return;
#pragma unroll
    for (int r = 0; r < kLenRegs; ++r) {
      const int i = 64 * r + lane_id();
      v[r] = i < p.num_seqs ? seq_len(p, i) : 0;
    }
  }
  // Length of sequence c + lane (0 past the last), c a multiple of 64.
  __device__ __forceinline__ int chunk(const Params &p, int c) const {
    if (held) {
      const int r = c >> 6;
      int x = 0;
#pragma unroll
      for (int k = 0; k < kLenRegs; ++k) x = r == k ? v[k] : x;
      return x;
    }
    const int i = c + lane_id();
    return i < p.num_seqs ? seq_len(p, i) : 0;
  }
};

// Tiles of one unit summed over all sequences: sum_i ceil(L_i / 16).
__device__ __forceinline__ int64_t tiles_per_unit(const Params &p, const SetupLens &sl) {
  int64_t tot = 0;
  for (int c = 0; c < p.num_seqs; c += 64) tot += wave_sum(seg_extent(own_tiles(p, sl.chunk(p, c))));
  return tot;
}


// Balanced split.  Sub-problem x (of xsplit) holds the head units
// u = x + xsplit*k, k < Ux = units / xsplit, of every sequence, and the waves
// w = x + xsplit*j, j < Wx = waves / xsplit.  Its segments (seq, k), laid end
// to end in that order, hold T = Ux * sum_i tiles_i tiles, cut into one
// contiguous range per wave.  Ranges are weighted: workgroups are dealt
// round-robin to the 8 XCDs, so wave j of a single sub-problem runs on XCD
// j mod 8, and XCDs that stream faster get proportionally more tiles
// (weights: one per XCD, prefix sums in Params::xcd_prefix).  Every range
// is nonempty, so along the tile line the wave index j and the local
// segment index s = seq * Ux + k both only grow: the piece of segment s in
// wave j's range gets id x * id_stride + s + j, ids of distinct pieces
// differ, and a segment's pieces have consecutive ids.  The wave producing
// a segment's first (last) piece records j in seg_units[2*g] ([2*g+1]),
// g = seq * units + u, for the merge.
struct Split {
  int64_t T, W;
  bool weighted;
  const Params *p;
  __device__ Split(const Params &pp, int64_t unit_tiles) : p(&pp) {
    const int64_t wx = pp.waves / pp.xsplit;
    T = unit_tiles * (pp.units / pp.xsplit);
    // A weighted range holds at least floor(T * weight / sum of weights)
    // tiles: all are nonempty when T * min weight >= that sum.  Otherwise
    // plain equal ranges over at most T waves.
    int wmin = pp.xcd_prefix[1] - pp.xcd_prefix[0];
    for (int i = 1; i < 8; ++i) wmin = min(wmin, pp.xcd_prefix[i + 1] - pp.xcd_prefix[i]);
    weighted = pp.xsplit == 1 && T * wmin >= cum(wx);
    W = weighted ? wx : (T < wx ? T : wx);
  }
  // Weighted waves before wave j: sum over v < j of weight[v mod 8].  The
  // prefix is picked with selects over constant indices: a runtime index
  // would copy the array to scratch memory.
  __device__ int64_t cum(int64_t j) const {
    const int r = (int)(j & 7);
    int pre = 0;
#pragma unroll
    for (int i = 1; i < 8; ++i) pre = r == i ? p->xcd_prefix[i] : pre;
    return (j >> 3) * p->xcd_prefix[8] + pre;
  }
  __device__ int64_t begin(int64_t j) const {
    return weighted ? T * cum(j) / cum(W) : T * j / W;
  }
};

struct RangePieces {
  const Params *p;
  int x, ux, seq, k, a, L, n_seq;
  int64_t unit, t, te, id_base;
  int64_t first_g;           // segment holding the range's first tile (-1: none)
  LenWindow lens;
  // A range that starts inside a segment and goes on past it processes that
  // first piece last: its partial row is then written at the end of the
  // wave's stream, with the last piece's, instead of in the middle of it
  // (mid-stream partial writes slow the reads of every wave).
  Piece deferred;
  bool has_deferred;

  __device__ void defer_first() {
    has_deferred = false;
    if (a > 0 && a < n_seq && te - t > seg_extent(n_seq) - a) {
      next(deferred);
      has_deferred = true;
    }
  }

  // The next piece: the real tiles of the next segment the range covers
  // (positions a.. of its extent; a range may cover only a segment's
  // virtual tiles, which give no piece).
  __device__ bool next(Piece &out) {
    while (t < te) {
      const int ext = seg_extent(n_seq);
      const int len = (int)min((int64_t)(ext - a), te - t);
      const int ra = min(a, n_seq), rb = min(a + len, n_seq);   // real tiles [ra, rb)
      const int u = x + p->xsplit * k;
      const int64_t g = (int64_t)seq * p->units + u;
      const bool has = ra < rb;
      if (has) {
        if (lane_id() == 0) {
          if (ra == 0) {
            p->seg_units[2 * g] = (int32_t)unit;
            if (p->seg_cnt) p->seg_cnt[g] = 0;   // the merge counts this segment's chunks
          }
          if (rb == n_seq) p->seg_units[2 * g + 1] = (int32_t)unit;
        }
        const int pt = p->prefix_tiles;
        out = Piece{seq, u, (ra + pt) * 16, min((rb + pt) * 16, L),
                    pt == 0 && ra == 0 && rb == n_seq, rb == n_seq,
                    id_base + (int64_t)seq * ux + k + unit, -1};
      }
      t += len;
      a = 0;
      if (t < te && ++k == ux) {
        k = 0;
        do {
          if (++seq >= p->num_seqs) {   // unreachable while t < te
            t = te;
            break;
          }
          L = lens.get(*p, seq);
          n_seq = own_tiles(*p, L);
        } while (n_seq == 0);
      }
      if (has) return true;
    }
    if (!has_deferred) return false;
    has_deferred = false;
    out = deferred;
    return true;
  }
};

// vb: the wave's index in the split (its workgroup id, or its place among
// the tail waves of a shared-prefix launch; vb and the workgroup id agree
// mod 8, so the wave runs on XCD vb mod 8).  tok_lds: where the wave's
// first new token is staged for store_new_tokens(p, vb, n_store, tok_lds).
template <class Body>
__device__ __forceinline__ void run_balanced(const Params &p, float (&p_lds)[2][16], int vb,
                                             u32x4 *tok_lds, int64_t n_store) {
  const int lane = lane_id();
  RangePieces gen;
  gen.p = &p;
  gen.x = vb % p.xsplit;
  gen.unit = (int64_t)vb / p.xsplit;
  gen.ux = p.units / p.xsplit;
  gen.first_g = -1;
  // The wave's record for the merge: the segment its range starts in.
  auto record = [&]() {
    if (p.wave_segs != nullptr && lane == 0) p.wave_segs[vb] = (int32_t)gen.first_g;
  };
  // The token is requested before the lengths: once the split has waited
  // for those, it has arrived too (loads return in order).
  TokenStash<Body> ts;
  ts.request(p, vb, n_store);
  SetupLens sl;
  sl.load(p);
  const Split sp(p, tiles_per_unit(p, sl));
  ts.park(tok_lds);
  if (gen.unit >= sp.W) {
    record();
    return;
  }
  gen.t = sp.begin(gen.unit);
  gen.te = sp.begin(gen.unit + 1);
  gen.id_base = (int64_t)gen.x * p.id_stride;
  // Find the sequence holding tile t: the first whose cumulative tiles pass t.
  gen.seq = -1;
  int64_t seq_first = 0, base = 0;
  for (int c = 0; c < p.num_seqs && gen.seq < 0; c += 64) {
    const int n = own_tiles(p, sl.chunk(p, c));
    const int incl = wave_incl_scan(seg_extent(n));
    const uint64_t hit = __builtin_amdgcn_ballot_w64((base + incl) * gen.ux > gen.t);
    if (hit) {
      const int l0 = (int)__builtin_ctzll(hit);
      gen.seq = c + l0;
      gen.n_seq = __builtin_amdgcn_readlane(n, l0);
      seq_first = (base + __builtin_amdgcn_readlane(incl, l0) - seg_extent(gen.n_seq)) * gen.ux;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (gen.seq < 0) {   // unreachable while t < T
    record();
    return;
  }
  gen.lens.base = gen.seq & ~63;
  gen.lens.vals = sl.chunk(p, gen.lens.base);
  gen.L = gen.lens.get(p, gen.seq);
  gen.k = (int)((gen.t - seq_first) / seg_extent(gen.n_seq));
  gen.a = (int)((gen.t - seq_first) % seg_extent(gen.n_seq));
  gen.first_g = (int64_t)gen.seq * p.units + gen.x + p.xsplit * gen.k;
  gen.has_deferred = false;
  gen.defer_first();
  record();
  stream_pieces<Body>(p, gen, p_lds);
}

template <class Body>
__global__ __launch_bounds__(64) PA_OCCUPANCY(Body) void decode_balanced(Params p) {
  __shared__ float p_lds[2][16];
  __shared__ u32x4 tok_lds[TokenStash<Body>::kLdsChunks];
  run_balanced<Body>(p, p_lds, (int)blockIdx.x, tok_lds, gridDim.x);
  store_new_tokens<Body>(p, blockIdx.x, gridDim.x, tok_lds);
}

// ---- shared prefix -------------------------------------------------------------
//
// When every sequence starts with the same physical blocks (a prompt shared
// by parallel samples: inferensys glossary "Paged Attention", second
// paragraph; skillsintelligence glossary, worked example), those blocks are
// read once per KV head for all the query rows that use them: the rows
// r = seq * G + h' of KV head h (query head h * G + h') take the N side of
// the MFMA body's products, 16 rows per tile, exactly as a group's heads do
// in decode.  Wave (row block, chunk, KV head) covers RT row tiles against
// one chunk of the prefix's tiles and writes one partial per row; the merge
// adds them to the sequence's own pieces.  Wave ids put all row blocks of
// one (chunk, KV head) on the same XCD, so a tile read by several row
// blocks is served by that XCD's L2.

// vb: the wave's index among the launch's prefix waves.
template <int D, int BS>
__device__ __forceinline__ void run_prefix(const Params &p, float (&p_lds)[2][16], int vb) {
  using Body = MfmaBody<D, BS, float, false>;   // cached loads: rows blocks re-read tiles
  using Tile = typename Body::Tile;
  constexpr int RT = kPrefixRowTiles;
  const int lane = lane_id();
  const int c = lane & 15, g = lane >> 4;
  const int pairs = p.num_kv_heads * p.pf_chunks;
  const int pair = vb % pairs, rb = vb / pairs;
  const int h = pair % p.num_kv_heads, chunk = pair / p.num_kv_heads;
  const int t_lo = chunk * p.pf_chunk_tiles;
  const int t_hi = min(t_lo + p.pf_chunk_tiles, p.prefix_tiles);
  if (t_lo >= t_hi) return;
  const int R = p.pf_rows;

  typename Body::QRaw q[RT];
  typename Body::Acc acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = min(rb * 16 * RT + t * 16 + c, R - 1);   // rows past R: unused copies
    const int seq = row / p.group, hq = h * p.group + row % p.group;
    const bf16_t *qp = static_cast<const bf16_t *>(p.query) + ((int64_t)seq * p.num_q_heads + hq) * D;
#pragma unroll
    for (int j = 0; j < Body::QJ; ++j)
      q[t].c[j] = *reinterpret_cast<const u32x4 *>(qp + (4 * j + g) * 8);
    Body::init(acc[t]);
  }
  const Piece pc{0, 0, t_lo * 16, t_hi * 16, false, false, 0, -1};
  TableReader tab;
  tab.start(p, pc, BS, false);
  const int64_t head_off = (int64_t)h * D * BS;
  int lk = t_lo, ck = t_lo;
  auto load = [&](Tile &tl) -> bool {
    if (lk >= t_hi) return false;
    Body::load_tile(p, tab, head_off, lk++, tl);
    return true;
  };
  // One tile against every row tile, as straight-line code: prefix tiles
  // are always full (no masking) and the rescale is unconditional, so the
  // RT independent chains (QK^T, softmax, PV) interleave.
  auto compute = [&](Tile &tl) {
    mfma_f32x4 sv[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) sv[t] = mfma_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < Body::QJ; ++j)
#pragma unroll
      for (int t = 0; t < RT; ++t)
        sv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(mfma_bf16x8, tl.k[j]), __builtin_bit_cast(mfma_bf16x8, q[t].c[j]),
            sv[t], 0, 0, 0);
    mfma_i16x4 pb[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = sv[t][r] * p.scale_log2e;
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = pair32_max(pair16_max(mx));
      const float mnew = fmaxf(acc[t].m, mx);
      const float alpha = fast_exp2(acc[t].m - mnew);
      acc[t].m = mnew;
      const unsigned p01 = pack_bf16x2(fast_exp2(sc[0] - mnew), fast_exp2(sc[1] - mnew));
      const unsigned p23 = pack_bf16x2(fast_exp2(sc[2] - mnew), fast_exp2(sc[3] - mnew));
      acc[t].lsum = acc[t].lsum * alpha +
                    ((__uint_as_float(p01 << 16) + __uint_as_float(p01 & 0xffff0000u)) +
                     (__uint_as_float(p23 << 16) + __uint_as_float(p23 & 0xffff0000u)));
#pragma unroll
      for (int i = 0; i < Body::VT; ++i) acc[t].o[i] *= alpha;
      pb[t] = __builtin_bit_cast(mfma_i16x4, u32x2{p01, p23});
    }
#pragma unroll
    for (int i = 0; i < Body::VT; ++i)
#pragma unroll
      for (int t = 0; t < RT; ++t)
        acc[t].o[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(mfma_i16x4, tl.v[i]), pb[t], acc[t].o[i], 0, 0, 0);
    ++ck;
  };
  Tile b0, b1;
  bool h0 = load(b0);
  bool h1 = load(b1);
  while (h0) {
    compute(b0);
    h0 = load(b0);
    if (!h1) break;
    compute(b1);
    h1 = load(b1);
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const float ltot = pair32_sum(pair16_sum(acc[t].lsum));
    const int row = rb * 16 * RT + t * 16 + c;
    if (row >= R) continue;
    const int64_t pr = ((int64_t)chunk * p.num_kv_heads + h) * R + row;
#pragma unroll
    for (int i = 0; i < Body::VT; ++i)
      *reinterpret_cast<f32x4 *>(p.pf_acc + pr * D + 16 * i + 4 * g) =
          f32x4{acc[t].o[i][0], acc[t].o[i][1], acc[t].o[i][2], acc[t].o[i][3]};
    if (g == 0) {
      p.pf_max[pr] = acc[t].m;
      p.pf_sum[pr] = ltot;
    }
  }
}

// Shared prefix and per-sequence tails in one launch: prefix waves wait on
// cache-level reads of the few prefix blocks, tail waves stream the
// sequences' own blocks from HBM, so the two kinds overlap.  Workgroups are
// dealt in runs of 8, alternating tail / prefix while both kinds have a
// run left, then the remaining tail waves and the remaining prefix waves
// (mixed_wave): every wave of each kind runs exactly once.
template <class Body>
__global__ __launch_bounds__(64) PA_OCCUPANCY(Body) void decode_prefix_tails(Params p) {
  __shared__ float p_lds[2][16];
  __shared__ u32x4 tok_lds[TokenStash<Body>::kLdsChunks];
  const MixedWave mw = mixed_wave((int)blockIdx.x, p.waves, p.pf_waves);
  if (mw.tail) {
    if (mw.index >= p.waves) return;   // only if the grid were larger than both kinds
    run_balanced<Body>(p, p_lds, mw.index, tok_lds, p.waves);
    store_new_tokens<Body>(p, mw.index, p.waves, tok_lds);
  } else {
    if (mw.index >= p.pf_waves) return;
    run_prefix<Body::kHeadDim, Body::kBlockSize>(p, p_lds, mw.index);
  }
}

// ---- log-sum-exp merge -------------------------------------------------------
//
// One wave per output row (sequence, unit, head in unit).  A row split into
// pieces with base-2 maxima m_p, sums l_p and unnormalised outputs o_p gets
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Rows of one piece were written whole by the main kernel; in balanced mode
// this kernel also writes the zero rows of empty sequences.
//
// Lanes are (piece group, 4-float chunk of the row): with d = 128, lanes
// 0-31 take pieces 0, 2, 4, ... and lanes 32-63 pieces 1, 3, 5, ...  Each
// group folds its pieces in order with an online rescale, four pieces'
// maxima, sums and outputs requested together, and the groups are combined
// at the end: a fixed order.  A row of up to 4 * (64 / (d / 4)) pieces per
// wave costs two dependent memory round trips (its piece range, then the
// partials); rows with more pieces (long contexts) get a workgroup of NW
// waves, the groups spread over them and the waves combined through LDS.

template <int D, typename OUT, int NW>
__global__ __launch_bounds__(64 * NW) void decode_merge(Params p) {
  const int lane = (int)threadIdx.x & 63, w = (int)threadIdx.x >> 6;
  int r = (int)blockIdx.x;
  const int hh = r % p.gu;
  r /= p.gu;
  const int unit = r % p.units;
  const int seq = r / p.units;
  int qh;
  if (p.head_tiles == 1 && p.gu == 1) {
    qh = unit;
  } else {
    const int h = (unit % p.head_tiles) * 16 + hh;
    if (h >= p.group) return;
    qh = (unit / p.head_tiles) * p.group + h;
  }
  constexpr int CH = D / 4;      // 4-float chunks per row
  constexpr int PG = 64 / CH;    // piece groups per wave
  constexpr int GT = PG * NW;    // piece groups in the workgroup
  constexpr int KB = 4;          // pieces per group whose loads are issued together
  const int ch = lane % CH, pg = lane / CH;
  OUT *out = static_cast<OUT *>(p.out) + ((int64_t)seq * p.num_q_heads + qh) * D;
  const int L = seq_len(p, seq);
  const bool balanced = p.partition_size < 0;
  // Balanced split: the segment's owning waves, requested together with the
  // length (they are stale, and unused, when the sequence has no own tiles).
  const int64_t g = (int64_t)seq * p.units + unit;
  int u0 = 0, u1 = 0;
  if (balanced) {
    u0 = p.seg_units[2 * g];
    u1 = p.seg_units[2 * g + 1];
  }
  if (L == 0) {
    if (balanced && w == 0 && pg == 0) store_out4<OUT>(out + 4 * ch, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  int64_t id0 = 0;
  int n = 0;
  if (balanced) {
    if (own_tiles(p, L) > 0) {
      const int x = unit % p.xsplit, ux = p.units / p.xsplit;
      n = u1 - u0 + 1;
      id0 = (int64_t)x * p.id_stride + (int64_t)seq * ux + unit / p.xsplit + u0;
    }
  } else {
    n = p.partition_size > 0 ? (L + p.partition_size - 1) / p.partition_size : 1;
    id0 = ((int64_t)seq * p.units + unit) * p.num_partitions;
  }
  // The shared prefix's partials of this row: one per chunk, in chunk
  // order, before the sequence's own pieces.
  const int npf = p.prefix_tiles > 0 ? p.pf_chunks : 0;
  const int64_t pf0 = npf ? (int64_t)(qh / p.group) * p.pf_rows + seq * p.group + qh % p.group : 0;
  const int64_t pf_step = (int64_t)p.num_kv_heads * p.pf_rows;
  if (npf == 0 && n <= 1) return;
  const int total = npf + n;
  auto row_of = [&](int i, const float *&mx, const float *&sm, const float *&ac) {
    if (i < npf) {
      const int64_t r = pf0 + i * pf_step;
      mx = p.pf_max + r; sm = p.pf_sum + r; ac = p.pf_acc + r * D;
    } else {
      const int64_t r = (id0 + (i - npf)) * p.gu + hh;
      mx = p.ws_max + r; sm = p.ws_sum + r; ac = p.ws_acc + r * D;
    }
  };
  // Each lane group folds its pieces in order with an online rescale
  // (running max mg, sum sg, output ag), KB pieces' loads at a time.
  float mg = -INFINITY, sg = 0.f;
  f32x4 ag = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = w * PG + pg; i0 < total; i0 += GT * KB) {
    float pm[KB], ps[KB];
    f32x4 po[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int i = i0 + GT * j;
      pm[j] = -INFINITY;
      ps[j] = 0.f;
      po[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < total) {
        const float *mx, *sm, *ac;
        row_of(i, mx, sm, ac);
        pm[j] = *mx;
        ps[j] = *sm;
        po[j] = *reinterpret_cast<const f32x4 *>(ac + 4 * ch);
      }
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (i0 + GT * j < total) {
        const float mn = fmaxf(mg, pm[j]);
        const float a = fast_exp2(mg - mn), b = fast_exp2(pm[j] - mn);
        ag = ag * a + po[j] * b;
        sg = sg * a + ps[j] * b;
        mg = mn;
      }
    }
  }
  // Combine the wave's groups: M over its pieces, each group's share
  // rescaled to it; then the waves in order.
  float M = mg;
#pragma unroll
  for (int off = CH; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float f = mg == -INFINITY ? 0.f : fast_exp2(mg - M);
  f32x4 acc = ag * f;
  float den = sg * f;
#pragma unroll
  for (int off = CH; off < 64; off <<= 1) {
    acc[0] += __shfl_xor(acc[0], off);
    acc[1] += __shfl_xor(acc[1], off);
    acc[2] += __shfl_xor(acc[2], off);
    acc[3] += __shfl_xor(acc[3], off);
    den += __shfl_xor(den, off);
  }
  if constexpr (NW > 1) {
    __shared__ f32x4 s_acc[NW][CH];
    __shared__ float s_m[NW], s_den[NW];
    if (pg == 0) {
      s_acc[w][ch] = acc;
      if (ch == 0) {
        s_m[w] = M;
        s_den[w] = den;
      }
    }
    __syncthreads();
    if (w != 0) return;
    float Mt = s_m[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) Mt = fmaxf(Mt, s_m[k]);
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    den = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float fk = s_m[k] == -INFINITY ? 0.f : fast_exp2(s_m[k] - Mt);
      acc += s_acc[k][ch] * fk;
      den += s_den[k] * fk;
    }
  }
  const float inv = 1.f / den;
  if (pg == 0) store_out4<OUT>(out + 4 * ch, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
}

// ---- merge of the balanced split, many sequences -----------------------------
//
// Used when segments are expected to span few pieces (many sequences: each
// wave's range holds about one segment).  A segment split over the main
// kernel's waves u0..u1 (n = u1 - u0 + 1 pieces, consecutive piece ids) has
// its pieces grouped into chunks of C (merge_chunk); the leader of a chunk
// folds its pieces, for every row of the segment's unit, in position order.
//   * Chunk 0 is led by wave g of this kernel, g the segment's index.  With
//     one chunk (n small, the usual case) it writes the output rows: two
//     dependent memory round trips, the segment's owners then its partials.
//   * A segment far longer than the rest (one long context among short
//     ones) has several chunks, and chunk c >= 1 is led by this kernel's
//     wave u0 + c * C.  The main kernel's wave of that index has a range
//     starting inside the segment (its predecessor owns part of it too), and
//     it recorded that segment, so the leader finds it in one load.  Each
//     leader writes its chunk's max, sum and output over the
//     partial row of the chunk's first piece (no other wave reads that row),
//     then counts itself in on the segment's counter, reset to 0 by the main
//     kernel.  The leader that arrives last folds the chunks in chunk order
//     and writes the output rows, so the order depends on positions only.
//     The release and acquire around the counter write back and invalidate
//     an XCD's L2, which is why segments with many pieces as the rule (few,
//     long sequences) go to decode_merge instead.
// Wave g also writes the zero rows of segment g when its sequence is empty.
// Lanes are (four-float chunk ch, row group rg); row group rg owns rows
// hh = rg + RGN * r, r < RG, of the unit (one row with the VALU body).
// Grid: max(segments, main-kernel waves).

// Lambdas that hold references to register arrays must be inlined: an
// outlined call would put those arrays in scratch memory.
#define PA_INLINE_LAMBDA __attribute__((always_inline))

// Pieces per chunk of a segment of n pieces: one chunk up to four rounds of
// KB loads (no synchronisation), else max(4 KB, about sqrt(n)), so that the
// leaders' folds and the last fold over the chunks take about as many
// rounds.
template <int KB>
__device__ __forceinline__ int merge_chunk(int n) {
  if (n <= 4 * KB) return n;
  const int c = (int)ceilf(sqrtf((float)n));
  return c > 4 * KB ? c : 4 * KB;
}

template <int D, typename OUT, int RG>
__global__ __launch_bounds__(64) void decode_merge_segments(Params p) {
  constexpr int CH = D / 4;      // 4-float chunks per row
  constexpr int RGN = 64 / CH;   // row groups per wave
  constexpr int KB = RG <= 4 ? 4 : 2;   // pieces per row whose loads are issued together
  const int lane = lane_id();
  const int ch = lane % CH, rg = lane / CH;
  const int b = (int)blockIdx.x;
  const int64_t segs = (int64_t)p.num_seqs * p.units;
  const int ux = p.units / p.xsplit;

  float mg[RG], sg[RG];
  f32x4 ag[RG];
  // Fold `count` partial rows, ids first, first + step, ... (in that order),
  // for every row this lane group owns, into (mg, sg, ag).
  auto fold = [&](int64_t first, int count, int step, int nh) PA_INLINE_LAMBDA {
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      mg[r] = -INFINITY;
      sg[r] = 0.f;
      ag[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int i0 = 0; i0 < count; i0 += KB) {
      float pm[KB][RG], ps[KB][RG];
      f32x4 po[KB][RG];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const int hh = rg + RGN * r;
          pm[k][r] = -INFINITY;
          ps[k][r] = 0.f;
          po[k][r] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (i0 + k < count && hh < nh) {
            const int64_t row = (first + (int64_t)(i0 + k) * step) * p.gu + hh;
            pm[k][r] = p.ws_max[row];
            ps[k][r] = p.ws_sum[row];
            po[k][r] = *reinterpret_cast<const f32x4 *>(p.ws_acc + row * D + 4 * ch);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (i0 + k < count) {
#pragma unroll
          for (int r = 0; r < RG; ++r) {
            const float mn = fmaxf(mg[r], pm[k][r]);
            const float a = fast_exp2(mg[r] - mn), c = fast_exp2(pm[k][r] - mn);
            ag[r] = ag[r] * a + po[k][r] * c;
            sg[r] = sg[r] * a + ps[k][r] * c;
            mg[r] = mn;
          }
        }
      }
    }
  };
  // Segment g's first output row (query head), rows, output pointer.
  auto rows_of = [&](int64_t g, int &nh) PA_INLINE_LAMBDA -> OUT * {
    const int unit = (int)(g % p.units);
    int qh0;
    if (p.gu == 1) {   // VALU body: one query head per unit
      qh0 = unit;
      nh = 1;
    } else {
      const int h0 = (unit % p.head_tiles) * 16;
      qh0 = (unit / p.head_tiles) * p.group + h0;
      nh = min(p.gu, p.group - h0);
    }
    return static_cast<OUT *>(p.out) + ((g / p.units) * p.num_q_heads + qh0) * D + 4 * ch;
  };
  auto store_rows = [&](OUT *out, int nh, bool zero) PA_INLINE_LAMBDA {
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int hh = rg + RGN * r;
      if (hh < nh) {
        const float inv = zero ? 0.f : 1.f / sg[r];
        store_out4<OUT>(out + (int64_t)hh * D, ag[r][0] * inv, ag[r][1] * inv, ag[r][2] * inv,
                        ag[r][3] * inv);
      }
    }
  };
  // Lead chunk c of segment g (owners u0..u1).
  auto lead = [&](int64_t g, int u0, int u1, int c) PA_INLINE_LAMBDA {
    const int n = u1 - u0 + 1;
    const int C = merge_chunk<KB>(n), nc = (n + C - 1) / C;
    const int unit = (int)(g % p.units), seq = (int)(g / p.units);
    const int64_t id0 = (int64_t)(unit % p.xsplit) * p.id_stride + (int64_t)seq * ux +
                        unit / p.xsplit + u0;
    const int64_t first = id0 + (int64_t)c * C;
    int nh;
    OUT *out = rows_of(g, nh);
    fold(first, min(C, n - c * C), 1, nh);
    if (nc == 1) {
      store_rows(out, nh, false);
      return;
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int hh = rg + RGN * r;
      if (hh < nh) {
        const int64_t row = first * p.gu + hh;
        *reinterpret_cast<f32x4 *>(p.ws_acc + row * D + 4 * ch) = ag[r];
        if (ch == 0) {
          p.ws_max[row] = mg[r];
          p.ws_sum[row] = sg[r];
        }
      }
    }
    // Release this chunk's rows to the other XCDs, then count in; the last
    // leader acquires the others' rows before reading them.  (Release and
    // acquire apart: each costs an XCD-wide L2 write-back or invalidate.)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int before = 0;
    if (lane == 0) before = atomicAdd(p.seg_cnt + g, 1);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before != nc - 1) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    fold(id0, nc, C, nh);
    store_rows(out, nh, false);
  };

  // The segment the main kernel's wave b started in and its owners, for
  // the chunks c >= 1 below: requested first, so that these loads overlap
  // the chunk-0 work instead of following it.
  int gb = -1, gu0 = 0, gu1 = 0;
  if (b < p.waves) gb = p.wave_segs[b];
  if (gb >= 0) {
    gu0 = p.seg_units[2 * (int64_t)gb];
    gu1 = p.seg_units[2 * (int64_t)gb + 1];
  }
  // Chunk 0 of segment b, or its zero rows.
  if (b < segs) {
    // The owning waves are requested with the length (stale, and unused,
    // when the sequence is empty).
    const int L = seq_len(p, (int)(b / p.units));
    const int u0 = p.seg_units[2 * (int64_t)b], u1 = p.seg_units[2 * (int64_t)b + 1];
    if (L == 0) {
      int nh;
      OUT *out = rows_of(b, nh);
#pragma unroll
      for (int r = 0; r < RG; ++r) ag[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      store_rows(out, nh, true);
    } else if (u1 > u0) {   // one piece: the main kernel wrote the rows
      lead(b, u0, u1, 0);
    }
  }
  // A chunk c >= 1 this wave leads: in the segment the main kernel's wave b
  // started in.
  if (gb >= 0) {
    const int j = b / p.xsplit;
    const int n = gu1 - gu0 + 1;
    if (n > 4 * KB && j > gu0 && j <= gu1) {   // several chunks, not chunk 0
      const int C = merge_chunk<KB>(n);
      if ((j - gu0) % C == 0) lead(gb, gu0, gu1, (j - gu0) / C);
    }
  }
}

// ---- dispatch ----------------------------------------------------------------

// Launch `kernel`(p).  With a pair of timing events (pa_set_timing_events)
// the runtime stamps them with the kernel's own start and end, adding no
// work to the stream; otherwise a plain launch.
hipError_t launch(const void *kernel, dim3 grid, dim3 block, Params &p, hipStream_t st,
                  void *ev_start = nullptr, void *ev_end = nullptr) {
  void *args[] = {&p};
  if (ev_start != nullptr || ev_end != nullptr)
    return hipExtLaunchKernel(kernel, grid, block, args, 0, st, static_cast<hipEvent_t>(ev_start),
                              static_cast<hipEvent_t>(ev_end), 0);
  return hipLaunchKernel(kernel, grid, block, args, 0, st);
}

// Waves of `kernel` the device holds at once (64-thread workgroups).
int resident_waves(const void *kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

// The balanced split, alone or (shared prefix) with the prefix waves: the
// tails then get the resident waves the prefix waves leave.
template <class Body>
hipError_t launch_balanced(const DecodeArgs &a, Params &p, hipStream_t st) {
  const bool pf = p.prefix_tiles > 0;
  constexpr bool pf_ok = std::is_same<typename Body::KVT, bf16_t>::value && Body::kStreams;
  if (pf && !pf_ok) return hipErrorInvalidValue;   // prefix calls are bf16 and stream their tails
  const void *k = reinterpret_cast<const void *>(&decode_balanced<Body>);
  if constexpr (pf_ok) {
    if (pf) k = reinterpret_cast<const void *>(&decode_prefix_tails<Body>);
  }
  int resident = resident_waves(k);
  if (resident <= 0) return hipErrorInvalidDevice;
  if (pf) resident = resident - p.pf_waves > 64 ? resident - p.pf_waves : 64;
  const BalancedPlan plan = balanced_plan(a, p.units, resident);
  if (plan.waves <= 0) return hipErrorInvalidDevice;
  p.waves = plan.waves;
  p.xsplit = plan.xsplit;
  p.id_stride = plan.id_stride;
  p.xcd_prefix[0] = 0;
  for (int i = 0; i < 8; ++i) p.xcd_prefix[i + 1] = p.xcd_prefix[i] + a.xcd_weights[i];
  if constexpr (pf_ok) {
    if (pf) {
      const int64_t grid = (int64_t)plan.waves + p.pf_waves;
      if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
      return launch(k, dim3((unsigned)grid), dim3(64), p, st, a.ev_main_start, a.ev_main_end);
    }
  }
  return launch(k, dim3(plan.waves), dim3(64), p, st, a.ev_main_start, a.ev_main_end);
}

template <class Body, typename OUT>
hipError_t launch_body(const DecodeArgs &a, Params &p, hipStream_t st) {
  if (p.partition_size < 0) {
    return launch_balanced<Body>(a, p, st);
  } else {
    const int64_t grid = (int64_t)p.units * a.num_seqs * p.num_partitions;
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    return launch(reinterpret_cast<const void *>(&decode_fixed<Body>), dim3((unsigned)grid),
                  dim3(64), p, st, a.ev_main_start, a.ev_main_end);
  }
}

template <typename OUT, bool NT>
hipError_t dispatch_out(const DecodeArgs &a, Params &p, bool use_mfma, hipStream_t st) {
  const bool bf = a.kv_dtype == PA_BF16;
  const int D = a.head_dim, BS = a.block_size;
#define PA_CASE(d, bs)                                                              \
  if (D == d && BS == bs) {                                                         \
    if (use_mfma) return launch_body<MfmaBody<d, bs, OUT, NT>, OUT>(a, p, st);      \
    return bf ? launch_body<ValuBody<bf16_t, d, bs, OUT, NT>, OUT>(a, p, st)        \
              : launch_body<ValuBody<float, d, bs, OUT, NT>, OUT>(a, p, st);        \
  }
  PA_CASE(64, 16)
  PA_CASE(64, 32)
  PA_CASE(64, 64)
  PA_CASE(128, 16)
  PA_CASE(128, 32)
  PA_CASE(128, 64)
#undef PA_CASE
  return hipErrorInvalidValue;
}

// The shared prefix's plan: chunks of the prefix and the waves that cover
// them, launched with the tails by launch_balanced.
hipError_t plan_prefix(const DecodeArgs &a, Params &p) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const PrefixPlan pf =
      prefix_plan(a.num_seqs, a.num_q_heads, a.num_kv_heads, a.prefix_len, cus);
  p.pf_chunks = pf.chunks;
  p.pf_chunk_tiles = pf.chunk_tiles;
  p.pf_rows = pf.rows;
  const int64_t grid = (int64_t)pf.row_blocks * a.num_kv_heads * pf.chunks;
  if (grid <= 0 || grid > INT32_MAX / 2) return hipErrorInvalidConfiguration;
  p.pf_waves = (int)grid;
  return hipSuccess;
}

// Expected pieces per segment up to which a balanced split (no shared
// prefix) is merged one wave per segment (decode_merge_segments).  Beyond
// it most segments span many pieces, and decode_merge's multi-wave rows,
// combined through LDS, avoid the cross-XCD synchronisation that the
// segment merge needs for such segments.
constexpr int64_t kSegmentMergeMaxPieces = 4;

// Waves per output row for the merge: enough that each wave's piece groups
// get at most one batch of loads for the pieces a row is expected to have
// (balanced split: a segment spans about waves / segments ranges, plus one
// for the cuts; fixed partitions: the longest sequence's count).
template <int D>
int merge_waves(const DecodeArgs &a, const Params &p) {
  constexpr int per_wave = 4 * (64 / (D / 4));
  int64_t est;
  if (a.partition_size < 0) {
    const int64_t segs = (int64_t)a.num_seqs * (p.units / p.xsplit);
    est = segs > 0 ? (p.waves / p.xsplit + segs - 1) / segs + 1 : 1;
  } else {
    est = a.num_partitions;
  }
  if (a.prefix_len > 0) est += p.pf_chunks;
  return est > 2 * per_wave ? 4 : est > per_wave ? 2 : 1;
}

template <int D, typename OUT>
hipError_t launch_merge_d(const DecodeArgs &a, Params &p, int64_t rows, int nw, hipStream_t st) {
  const dim3 grid((unsigned)rows);
  void *e0 = a.ev_merge_start, *e1 = a.ev_merge_end;
  if (nw == 4)
    return launch(reinterpret_cast<const void *>(&decode_merge<D, OUT, 4>), grid, dim3(256), p,
                  st, e0, e1);
  if (nw == 2)
    return launch(reinterpret_cast<const void *>(&decode_merge<D, OUT, 2>), grid, dim3(128), p,
                  st, e0, e1);
  return launch(reinterpret_cast<const void *>(&decode_merge<D, OUT, 1>), grid, dim3(64), p, st,
                e0, e1);
}

template <int D, typename OUT>
hipError_t launch_merge_segments_d(const DecodeArgs &a, Params &p, int64_t segs,
                                   hipStream_t st) {
  constexpr int RGN = 64 / (D / 4);
  const int rg = (p.gu + RGN - 1) / RGN;
  const int64_t n = segs > p.waves ? segs : p.waves;
  if (n > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n);
  const void *k = rg <= 1   ? reinterpret_cast<const void *>(&decode_merge_segments<D, OUT, 1>)
                  : rg <= 2 ? reinterpret_cast<const void *>(&decode_merge_segments<D, OUT, 2>)
                  : rg <= 4 ? reinterpret_cast<const void *>(&decode_merge_segments<D, OUT, 4>)
                            : reinterpret_cast<const void *>(&decode_merge_segments<D, OUT, 8>);
  return launch(k, grid, dim3(64), p, st, a.ev_merge_start, a.ev_merge_end);
}

template <typename OUT>
hipError_t launch_merge(const DecodeArgs &a, Params &p, hipStream_t st) {
  const int64_t rows = (int64_t)a.num_seqs * p.units * p.gu;
  if (rows > INT32_MAX) return hipErrorInvalidConfiguration;
  // Balanced split without a shared prefix, segments expected to span few
  // pieces (many sequences): one wave per segment.
  if (a.partition_size < 0 && a.prefix_len == 0) {
    if (p.waves <= 0 || p.wave_segs == nullptr || p.seg_cnt == nullptr)
      return hipErrorInvalidValue;
    const int64_t segs = (int64_t)a.num_seqs * p.units;
    const int64_t sx = (int64_t)a.num_seqs * (p.units / p.xsplit);
    const int64_t est = sx > 0 ? (p.waves / p.xsplit + sx - 1) / sx + 1 : 1;
    if (est <= kSegmentMergeMaxPieces) {
      if (a.head_dim == 64) return launch_merge_segments_d<64, OUT>(a, p, segs, st);
      return launch_merge_segments_d<128, OUT>(a, p, segs, st);
    }
  }
  if (a.head_dim == 64) return launch_merge_d<64, OUT>(a, p, rows, merge_waves<64>(a, p), st);
  return launch_merge_d<128, OUT>(a, p, rows, merge_waves<128>(a, p), st);
}

}  // namespace

int noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex m;
  static void *per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(m);
  if (per_device[dev] == nullptr) {
    // Once per device, with that device current: its copy of the array.
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return (int)hipSuccess;
}

BalancedPlan balanced_plan(const DecodeArgs &a, int units, int resident) {
  // Reused blocks: split by XCD so that each KV head's blocks stay in one
  // L2.  Streaming: one weighted split over all XCDs.
  BalancedPlan pl;
  int w = resident < a.max_waves ? resident : a.max_waves;
  // No more waves than give each at least kMinTiles tiles of the largest
  // possible problem: small calls are not shattered into one-tile pieces.
  // At batch 1 (latency-bound) 4 beat 8 by 3 us per step and 2 lost the
  // gain again in the larger merge.
  constexpr int64_t kMinTiles = 4;
  const int64_t tiles_max = (a.max_context_len + 15) / 16;
  const int64_t t_upper = (int64_t)units * a.num_seqs * tiles_max;
  const int64_t cap = (t_upper + kMinTiles - 1) / kMinTiles;
  if (cap < w) w = cap > 0 ? (int)cap : 1;
  pl.xsplit = ((a.flags & PA_DECODE_KV_REUSED) && a.prefix_len == 0 && units % 8 == 0 && w >= 64)
                  ? 8 : 1;
  if (w >= 8) w -= w % 8;   // whole rounds of the 8 XCDs
  w -= w % pl.xsplit;
  pl.waves = w;
  pl.id_stride = (int64_t)a.num_seqs * (units / pl.xsplit) + w / pl.xsplit;
  pl.rows = (size_t)pl.xsplit * pl.id_stride;
  return pl;
}

HeadUnits head_units(int32_t num_q_heads, int32_t num_kv_heads, pa_dtype kv_dtype) {
  const int G = num_q_heads / num_kv_heads;
  HeadUnits u;
  u.mfma = kv_dtype == PA_BF16 && G >= 2;
  u.head_tiles = u.mfma ? (G + 15) / 16 : 1;
  u.units = u.mfma ? num_kv_heads * u.head_tiles : num_q_heads;
  u.gu = u.mfma ? (G < 16 ? G : 16) : 1;
  return u;
}

int launch_decode(const DecodeArgs &a, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const HeadUnits hu = head_units(a.num_q_heads, a.num_kv_heads, a.kv_dtype);
  Params p;
  p.out = a.out;
  p.query = a.query;
  // The pools are written only when new tokens are given.
  p.key_cache = static_cast<char *>(const_cast<void *>(a.key_cache));
  p.value_cache = static_cast<char *>(const_cast<void *>(a.value_cache));
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.new_key = a.new_key;
  p.new_value = a.new_value;
  p.slots = a.slots;
  p.cow_src = a.slots != nullptr ? a.cow_src : nullptr;
  p.ws_max = a.ws_max;
  p.ws_sum = a.ws_sum;
  p.ws_acc = a.ws_acc;
  p.seg_units = a.seg_units;
  // Records for the waves' merge (balanced split without a shared prefix).
  const bool wave_merge = a.partition_size < 0 && a.prefix_len == 0;
  p.seg_cnt = wave_merge ? a.seg_cnt : nullptr;
  p.wave_segs = wave_merge ? a.wave_segs : nullptr;
  p.num_blocks = a.num_blocks;
  p.num_seqs = a.num_seqs;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.max_context_len = a.max_context_len;
  p.partition_size = a.partition_size;
  p.num_partitions = a.num_partitions;
  p.units = hu.units;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.head_tiles = hu.head_tiles;
  p.gu = hu.gu;
  p.waves = 0;
  p.xsplit = 1;
  p.id_stride = 0;
  p.scale_log2e = a.scale * kLog2e;
  p.prefix_tiles = a.prefix_len / 16;
  p.pf_chunks = p.pf_chunk_tiles = p.pf_rows = p.pf_waves = 0;
  p.pf_max = a.pf_max;
  p.pf_sum = a.pf_sum;
  p.pf_acc = a.pf_acc;
  hipError_t e;
  if (a.prefix_len > 0) {
    e = plan_prefix(a, p);
    if (e != hipSuccess) return (int)e;
  }
  // With a shared prefix the reused blocks are the prefix's, read by the
  // prefix waves; the tails are streamed.
  const bool reused = (a.flags & PA_DECODE_KV_REUSED) != 0 && a.prefix_len == 0;
  if (a.out_dtype == PA_BF16)
    e = reused ? dispatch_out<bf16_t, false>(a, p, hu.mfma, st)
               : dispatch_out<bf16_t, true>(a, p, hu.mfma, st);
  else
    e = reused ? dispatch_out<float, false>(a, p, hu.mfma, st)
               : dispatch_out<float, true>(a, p, hu.mfma, st);
  if (e != hipSuccess) return (int)e;
  const bool merge = a.partition_size < 0 || a.num_partitions > 1;
  if (!merge) return (int)hipSuccess;
  e = a.out_dtype == PA_BF16 ? launch_merge<bf16_t>(a, p, st) : launch_merge<float>(a, p, st);
  return (int)e;
}

}  // namespace pa
