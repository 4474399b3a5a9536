// paged_decode_attn on gfx950: one decode step of attention for many agents
// over a deduplicated, paged KV pool.
//
// Two kernels per call, both on the caller's stream.  A consumer with shift != 0
// reads its agent's query moved by R(-shift), so that (R(-s) q) . k == q . (R(s) k)
// (INMS walkthrough sec. 3.2: the compensation depends on the position
// difference only); the tile pass rotates it as it loads it (cos and sin from
// the plan) and splits it into a bf16 hi + lo pair.  Unshifted consumers read
// the bf16 query as it is.
//   1. tile    -- one workgroup of 4 waves per (work item, kv head); the item's
//                 physical blocks are split into 4 runs of 16-token tiles, one
//                 per wave.  A wave streams its tiles from HBM once with 16-byte
//                 non-temporal loads straight into registers (the next tile's
//                 loads in flight while the current one is computed), and every
//                 query row the item carries -- all agents and GQA heads that
//                 read those blocks -- is scored against the same registers, so
//                 a shared block is fetched once for all of them.  Online softmax
//                 per row (MemDecay blog sec. 4.2: scaled dot product, float32
//                 softmax); a delta block is an ordinary block of its owner, and
//                 the owner is masked out of the master block (TokenDance
//                 write-up sec. 3, the correction fused into the load); Q4 blocks
//                 are dequantised in registers (Q4 KV paper summary sec. 2.2).
//                 The path depends on the item's rows: VALU dot products for
//                 1-4 bf16 rows; matrix cores otherwise, with two (5-7 bf16
//                 rows) or four (2-4 Q4 rows) tiles sharing one 16-column result
//                 tile so that few-row items do not compute padding rows; items
//                 of more than 16 rows (a segment read by many agents) stage
//                 each pair of blocks in LDS once for all 4 waves.  The 4 waves
//                 merge through LDS and write one partial (max, sum, acc) per
//                 row.
//   2. combine -- log-sum-exp merge of each (agent, q head)'s partials in a
//                 fixed order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <mutex>
#include <type_traits>

#include "../host/kvpool_internal.h"
#include "device_common.h"
#include "kvpool.h"

namespace {
using namespace kvp;

constexpr float kNegBig = -1e30f;  // finite "no score yet" (keeps exp2 arguments finite)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;  // waves per tile workgroup
// The online softmax keeps a per-row reference max that is raised lazily: a
// tile's weights are exp2(s - ref), allowed up to 2^kSlack, and the running sums
// are rescaled only when some row of the wave exceeds its reference by more
// than that (a wave-uniform branch, rare after the first tiles).
constexpr float kSlack = 8.f;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct TileArgs {
  const kvp_item* items;
  const int32_t* plan_blocks;
  const int32_t* cons;
  const int32_t* qcons;
  const uint32_t* mask;
  const int32_t* phys_ntok;
  const int32_t* plan_ntok;  // [n_plan_blocks] valid tokens of each plan block
  const int32_t* cons_row;   // [n_cons] query row of each consumer (its agent, or its row of rope_cs)
  const uint16_t* q;       // [n_agents][Hq][D] bf16
  const float* rope_cs;    // [n_qcons_shifted][D/2][2] (cos, sin) of R(-shift)
  int n_unshifted;         // qcons ids below this have shift 0
  const uint8_t* kpool;
  const uint8_t* vpool;
  const uint8_t* kpar;  // Q4: fp16 (scale, zero) pairs
  const uint8_t* vpar;
  int64_t layer_blocks;  // layer * n_phys
  int Hq, Hkv, B;
  float sl2e;    // softmax scale * log2(e)
  float* pacc;   // [Hkv][P][D]
  float2* pml;   // [Hkv][P] (max in log2 units, sum)
  int P;
  int n_items;
  int xcd_span;  // units per XCD per dispatch window
  // extents of the plan's arrays (read by the checked build's bounds checks)
  int n_agents, n_phys, n_plan_blocks, n_cons, n_qcons, n_mask_words;
};

// Error word of the checked build, one per device: bits 1 (item ranges), 2 (block
// ids or token counts), 4 (consumers), 8 (combine lists).
__device__ uint32_t g_dev_err;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ld_nt16(const uint8_t* p) { return __builtin_nontemporal_load((const u32x4*)p); }
__device__ __forceinline__ u32x2 ld_nt8(const uint8_t* p) { return __builtin_nontemporal_load((const u32x2*)p); }
__device__ __forceinline__ uint32_t ld_nt4(const uint8_t* p) { return __builtin_nontemporal_load((const uint32_t*)p); }

// Cache policy of the wide path's loads into LDS: ordinary (allocating) loads.
// A shared segment block is read by several wide items (its consumers split
// into groups of at most 128 rows), which run side by side on one XCD; ordinary
// loads let the later groups find the block in that XCD's L2, so HBM delivers it
// about once (non-temporal loads measured 1.14x the unique bytes on the
// TokenDance round, ordinary ones 1.01x).
constexpr int kWideLoadPolicy = 0;

// ---------------------------------------------------------------------------
// 1. tile pass

// XCD-aware unit mapping.  A unit is one (item, kv head) pair; workgroups are
// dealt round-robin over the 8 XCDs (workgroup b runs on XCD b % 8).
//  * n_kv_heads a multiple of 8: XCD x owns kv heads [x*H/8, (x+1)*H/8) for the
//    whole launch and walks the items in plan order for them.  Every XCD gets the
//    same work, sees the plan's order (heavy items first, the short split items
//    last, which fill the end of the launch), and its reads stay within its own
//    kv heads.
//  * otherwise: units are numbered item-major and the grid is cut into windows of
//    8*S workgroups; inside a window XCD x takes S consecutive units (S = the
//    plan's unit_span, covering the items that read the same blocks).
// Returns false for padding workgroups.
__device__ __forceinline__ bool unit_of(int n_items, int Hkv, int span, int& item, int& g) {
  const int b = (int)blockIdx.x;
  if ((Hkv & 7) == 0) {
    const int hpx = Hkv >> 3, slot = b >> 3;
    item = slot / hpx;
    g = (b & 7) * hpx + slot % hpx;
    return item < n_items;
  }
  const int win = 8 * span;
  const int unit = (b / win) * win + (b % 8) * span + (b % win) / 8;
  item = unit / Hkv;
  g = unit % Hkv;
  return unit < n_items * Hkv;
}

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)lo, (__bf16)hi});
}

// The query of shifted consumer qc (its row of rope_cs: row), q head hq, rotated
// by R(-shift) for rotate-half pairs [i0, i0 + 8): the first-half elements
// (y1 = x1 c - x2 s, dims i0 + [0, 8)) and the second-half ones (y2 = x2 c + x1 s,
// dims D/2 + i0 + [0, 8)), in float32 with rope_apply's fused multiply-adds and
// the plan's cos and sin, each split into bf16 hi + lo (both rounded to nearest
// even) so that hi + lo carries the rotated value to about 16 bits.
template <int D>
__device__ __forceinline__ void rotate_q16(const TileArgs& a, int qc, int row, int hq, int i0, uint4& hi1, uint4& lo1,
                                           uint4& hi2, uint4& lo2) {
  constexpr int H = D / 2;
  const uint16_t* src = a.q + ((int64_t)a.qcons[2 * qc] * a.Hq + hq) * D;
  const uint4 x1 = *(const uint4*)(src + i0), x2 = *(const uint4*)(src + i0 + H);
  const f32x4_t* cs = (const f32x4_t*)(a.rope_cs + ((int64_t)row * H + i0) * 2);
  const uint32_t w1[4] = {x1.x, x1.y, x1.z, x1.w}, w2[4] = {x2.x, x2.y, x2.z, x2.w};
  uint32_t h1[4], l1[4], h2[4], l2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4_t t = cs[k];  // (cos, sin) of pairs i0 + 2k and i0 + 2k + 1
    float y1[2], y2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
      rope_apply(e ? bf16_hi(w1[k]) : bf16_lo(w1[k]), e ? bf16_hi(w2[k]) : bf16_lo(w2[k]), t[2 * e], t[2 * e + 1],
                 &y1[e], &y2[e]);
    h1[k] = pack_bf16(y1[0], y1[1]);
    l1[k] = pack_bf16(y1[0] - bf16_lo(h1[k]), y1[1] - bf16_hi(h1[k]));
    h2[k] = pack_bf16(y2[0], y2[1]);
    l2[k] = pack_bf16(y2[0] - bf16_lo(h2[k]), y2[1] - bf16_hi(h2[k]));
  }
  hi1 = make_uint4(h1[0], h1[1], h1[2], h1[3]);
  lo1 = make_uint4(l1[0], l1[1], l1[2], l1[3]);
  hi2 = make_uint4(h2[0], h2[1], h2[2], h2[3]);
  lo2 = make_uint4(l2[0], l2[1], l2[2], l2[3]);
}

// Query elements [i0, i0 + 8) and [D/2 + i0, D/2 + i0 + 8) of consumer entry c,
// q head hq (i0 a multiple of 8 below D/2), as bf16 hi/lo words as load_q8 gives
// them: the two halves of the same rotate-half pairs from one set of loads.
template <int D>
__device__ __forceinline__ void load_q16(const TileArgs& a, int c, int hq, int i0, uint4& hi1, uint4& lo1, uint4& hi2,
                                         uint4& lo2) {
  const int qc = a.cons[c], row = a.cons_row[c];
  if (qc < a.n_unshifted) {
    const uint16_t* src = a.q + ((int64_t)row * a.Hq + hq) * D + i0;
    hi1 = *(const uint4*)src;
    hi2 = *(const uint4*)(src + D / 2);
    lo1 = lo2 = make_uint4(0, 0, 0, 0);
    return;
  }
  rotate_q16<D>(a, qc, row, hq, i0, hi1, lo1, hi2, lo2);
}

// Query elements [d0, d0 + 8) of consumer entry c (an index into cons), q head
// hq, as bf16 hi/lo words (d0 a multiple of 8): an unshifted consumer's bf16
// query as it is (lo = 0), a shifted one's rotated (rotate_q16).
template <int D>
__device__ __forceinline__ void load_q8(const TileArgs& a, int c, int hq, int d0, uint4& hi, uint4& lo) {
  const int qc = a.cons[c], row = a.cons_row[c];
  if (qc < a.n_unshifted) {
    hi = *(const uint4*)(a.q + ((int64_t)row * a.Hq + hq) * D + d0);
    lo = make_uint4(0, 0, 0, 0);
    return;
  }
  constexpr int H = D / 2;
  uint4 h1, l1, h2, l2;
  rotate_q16<D>(a, qc, row, hq, d0 & (H - 1), h1, l1, h2, l2);
  hi = d0 < H ? h1 : h2;
  lo = d0 < H ? l1 : l2;
}

// The tiles of an item: every block has ceil(ntok/16) 16-token tiles.  Wave w of
// the workgroup takes tiles [T*w/4, T*(w+1)/4).
//
// The block metadata a wave walks through (physical id, valid tokens, consumer
// mask words) is held one block per lane, 64 blocks at a time, and read in the
// tile loop with v_readlane.  A memory load there would be a vector load whose
// wait also covers every K/V tile already in flight, which stalls the prefetch
// at each block boundary.
struct BlockMeta {
  int base;     // item block index held by lane 0
  int p, nt;    // this lane's block: physical id, valid tokens
  uint32_t m0, m1;  // its consumer mask words (all ones without a mask)
};

__device__ __forceinline__ void meta_fill(const TileArgs& a, const kvp_item& it, int base, BlockMeta& m) {
  const int bi = base + (int)(threadIdx.x & 63);
  m.base = base;
  m.p = 0;
  m.nt = 0;
  m.m0 = 0xffffffffu;
  m.m1 = 0xffffffffu;
  if (bi < it.blk_end) {
    m.p = a.plan_blocks[bi];
    m.nt = a.plan_ntok[bi];
    if (it.mask_base >= 0) {
      const uint32_t* mw = a.mask + it.mask_base + (int64_t)(bi - it.blk_begin) * it.mask_stride;
      m.m0 = mw[0];
      if (it.mask_stride > 1) m.m1 = mw[1];
    }
  }
  // complete the loads here (s_waitcnt vmcnt(0)): a fill inside the tile loop is
  // conditional, and without this the compiler waits for them -- and for every
  // tile in flight -- after the branch on every iteration
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

struct Cursor {
  int bi, s, p, nt;
  uint32_t m0, m1;
};

// cursor fields of block bi from the wave's metadata (refilled past its window)
__device__ __forceinline__ void meta_get(const TileArgs& a, const kvp_item& it, BlockMeta& m, Cursor& c) {
  if (c.bi - m.base >= 64) meta_fill(a, it, c.bi, m);
  const int l = c.bi - m.base;
  c.p = __builtin_amdgcn_readlane(m.p, l);
  c.nt = __builtin_amdgcn_readlane(m.nt, l);
  c.m0 = (uint32_t)__builtin_amdgcn_readlane((int)m.m0, l);
  c.m1 = (uint32_t)__builtin_amdgcn_readlane((int)m.m1, l);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// total tiles of the item (every wave computes the same value)
__device__ __forceinline__ int item_tiles(const TileArgs& a, const kvp_item& it, BlockMeta& m) {
  if (a.B == 16) return it.blk_end - it.blk_begin;
  int T = 0;
  for (int base = it.blk_begin; base < it.blk_end; base += 64) {
    meta_fill(a, it, base, m);
    T += wave_sum((m.nt + 15) >> 4);
  }
  return T;
}

// cursor at tile t of the item
__device__ __forceinline__ Cursor seek(const TileArgs& a, const kvp_item& it, int t, BlockMeta& m) {
  Cursor c;
  c.s = 0;
  if (a.B == 16) {
    c.bi = it.blk_begin + t;
    meta_fill(a, it, c.bi, m);
  } else {
    c.bi = it.blk_begin;
    if (m.base != c.bi) meta_fill(a, it, c.bi, m);
    while (true) {
      meta_get(a, it, m, c);
      const int n = (c.nt + 15) >> 4;
      if (t < n) break;
      t -= n;
      ++c.bi;
    }
    c.s = t;
  }
  meta_get(a, it, m, c);
  return c;
}

__device__ __forceinline__ void wave_range(const TileArgs& a, const kvp_item& it, int w, int& cnt, Cursor& c,
                                           BlockMeta& m) {
  m.base = -1;
  // (wave-uniform values, kept in scalar registers: the tile loops and the
  // cursor bookkeeping then branch on scalars, never under an exec mask)
  const int T = __builtin_amdgcn_readfirstlane(item_tiles(a, it, m));
  const int t0 = T * w / kWaves;
  cnt = __builtin_amdgcn_readfirstlane(T * (w + 1) / kWaves - t0);
  c = Cursor{it.blk_begin, 0, 0, 0, 0u, 0u};
  if (cnt <= 0) return;
  c = seek(a, it, t0, m);
}

// the cursor's fields are wave-uniform: in scalar registers, the cursor
// arithmetic and the addresses derived from it run on the scalar unit
__device__ __forceinline__ Cursor uniform(Cursor c) {
  c.bi = __builtin_amdgcn_readfirstlane(c.bi);
  c.s = __builtin_amdgcn_readfirstlane(c.s);
  c.p = __builtin_amdgcn_readfirstlane(c.p);
  c.nt = __builtin_amdgcn_readfirstlane(c.nt);
  c.m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.m0);
  c.m1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.m1);
  return c;
}

// wave_range for a BlockMeta already filled for the item's first 64 blocks
// (meta.base == it.blk_begin; the fill's loads need not be complete).
__device__ __forceinline__ void wave_range_filled(const TileArgs& a, const kvp_item& it, int w, int& cnt, Cursor& c,
                                                  BlockMeta& m) {
  const int nblk = it.blk_end - it.blk_begin;
  int T;
  if (a.B == 16) {
    T = nblk;
  } else if (nblk <= 64) {
    T = wave_sum((m.nt + 15) >> 4);
  } else {
    T = 0;
    for (int base = it.blk_begin; base < it.blk_end; base += 64) {
      if (m.base != base) meta_fill(a, it, base, m);
      T += wave_sum((m.nt + 15) >> 4);
    }
  }
  T = __builtin_amdgcn_readfirstlane(T);
  const int t0 = T * w / kWaves;
  cnt = __builtin_amdgcn_readfirstlane(T * (w + 1) / kWaves - t0);
  c = Cursor{it.blk_begin, 0, 0, 0, 0u, 0u};
  if (cnt <= 0) return;
  if (a.B == 16) {
    c.bi = it.blk_begin + t0;
    if (c.bi - m.base >= 64) meta_fill(a, it, c.bi, m);
  } else {
    if (m.base != it.blk_begin) meta_fill(a, it, it.blk_begin, m);
    int t = t0;
    c.bi = it.blk_begin;
    while (true) {
      meta_get(a, it, m, c);
      const int n = (c.nt + 15) >> 4;
      if (t < n) break;
      t -= n;
      ++c.bi;
    }
    c.s = t;
  }
  meta_get(a, it, m, c);
}

__device__ __forceinline__ Cursor advance(const TileArgs& a, const kvp_item& it, BlockMeta& m, Cursor c) {
  if ((c.s + 1) * 16 < c.nt) {
    ++c.s;
  } else {
    ++c.bi;
    c.s = 0;
    meta_get(a, it, m, c);
  }
  return c;
}

// Runs tile(S) over a wave's cnt tiles with three register sets S = 0, 1, 2 and
// every tile's loads issued (issue(S)) two tiles before it is computed.  In the
// steady-state loop every step issues exactly one tile, so the number of loads
// in flight is the same on every path into each computation and the compiler's
// waits keep two tiles in flight; the last two to four tiles (and ranges under
// five tiles) go through a conditional epilogue.
template <class Issue, class Tile>
__device__ __forceinline__ void ring3(const int cnt, Issue&& issue, Tile&& tile) {
  int i = 0;
  if (cnt >= 5) {
    issue(0);
    issue(1);
    do {
      issue(2);
      tile(0);
      issue(0);
      tile(1);
      issue(1);
      tile(2);
      i += 3;
    } while (i + 5 <= cnt);
  } else {
    if (cnt > 0) issue(0);
    if (cnt > 1) issue(1);
  }
  // sets 0 and 1 hold tiles i and i + 1 (where they exist); at most 4 are left
  const int r = cnt - i;
  if (r > 2) issue(2);
  if (r > 0) tile(0);
  if (r > 3) issue(0);
  if (r > 1) tile(1);
  if (r > 2) tile(2);
  if (r > 3) tile(0);
}

// The same with two register sets (one tile ahead), for paths whose row state
// leaves no room for a third.
template <class Issue, class Tile>
__device__ __forceinline__ void ring2(const int cnt, Issue&& issue, Tile&& tile) {
  int i = 0;
  if (cnt >= 3) {
    issue(0);
    do {
      issue(1);
      tile(0);
      issue(0);
      tile(1);
      i += 2;
    } while (i + 3 <= cnt);
  } else if (cnt > 0) {
    issue(0);
  }
  // set 0 holds tile i (where it exists); at most 2 are left
  const int r = cnt - i;
  if (r > 1) issue(1);
  if (r > 0) tile(0);
  if (r > 1) tile(1);
}

// Cross-wave merge through LDS, 4 rows at a time; EPL elements per lane, lanes
// [0, D/EPL) cover a row.  Wave 0 writes the partials.
template <int D>
struct MergeLds {
  float acc[kWaves][4][D];
  float ml[kWaves][4][2];
};

template <int D, int EPL, int R>
__device__ __forceinline__ void merge_store(const TileArgs& a, const kvp_item& it, int g, int rows, float (&M)[R],
                                            float (&L)[R], float (&O)[R][EPL], MergeLds<D>& sh) {
  auto& s_acc = sh.acc;
  auto& s_ml = sh.ml;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int LANES = D / EPL;
#pragma unroll
  for (int rc = 0; rc < R; rc += 4) {
    if (rc >= rows) break;
#pragma unroll
    for (int k = 0; k < 4 && rc + k < R; ++k) {
      const int r = rc + k;
      if (r < rows) {
        if (lane < LANES) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) s_acc[w][k][lane * EPL + i] = O[r][i];
        }
        if (lane == 0) {
          s_ml[w][k][0] = M[r];
          s_ml[w][k][1] = L[r];
        }
      }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int k = 0; k < 4 && rc + k < R; ++k) {
        const int r = rc + k;
        if (r < rows) {
          float mx = s_ml[0][k][0];
#pragma unroll
          for (int v = 1; v < kWaves; ++v) mx = fmaxf(mx, s_ml[v][k][0]);
          float sc[kWaves], lt = 0.f;
#pragma unroll
          for (int v = 0; v < kWaves; ++v) {
            sc[v] = ex2(s_ml[v][k][0] - mx);
            lt += sc[v] * s_ml[v][k][1];
          }
          const int64_t row = (int64_t)g * a.P + it.part_base + r;
          if (lane < LANES) {
            float o[EPL];
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
              o[i] = 0.f;
#pragma unroll
              for (int v = 0; v < kWaves; ++v) o[i] += sc[v] * s_acc[v][k][lane * EPL + i];
            }
            float4* dst = (float4*)(a.pacc + row * D + lane * EPL);
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
          }
          if (lane == 0) a.pml[row] = make_float2(mx, lt);
        }
      }
    }
    __syncthreads();
  }
}

template <int D, int R>
__device__ __forceinline__ void run_bf16(const TileArgs& a, const kvp_item& it, const int g, MergeLds<D>& sh) {
  constexpr int LPT = D / 8;     // lanes per token row (8 bf16 = 16 bytes each)
  constexpr int TPL = 64 / LPT;  // tokens per wave-wide load
  constexpr int NL = 16 / TPL;   // loads per lane per 16-token tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int dsl = (lane % LPT) * 8;
  const int tg = lane / LPT;
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;

  bool any_lo = false;
  for (int c = it.cons_begin; c < it.cons_end; ++c) any_lo |= a.cons[c] >= a.n_unshifted;

  uint4 qh[R], ql[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    qh[r] = make_uint4(0, 0, 0, 0);
    ql[r] = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      const int c = r / group;
      load_q8<D>(a, it.cons_begin + c, g * group + (r - c * group), dsl, qh[r], ql[r]);
    }
  }
  float m[R], l[R], acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegBig;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[r][i] = 0.f;
  }

  constexpr int64_t kTileBytes = 16 * D * 2;
  const int64_t head_bytes = (int64_t)a.B * D * 2;
  const int64_t lane_off = (int64_t)tg * D * 2 + dsl * 2;
  auto load = [&](u32x4* kk, u32x4* vv, const Cursor& c) {
    const int64_t off = ((a.layer_blocks + c.p) * a.Hkv + g) * head_bytes + c.s * kTileBytes + lane_off;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      kk[k] = ld_nt16(a.kpool + off + (int64_t)k * TPL * D * 2);
      vv[k] = ld_nt16(a.vpool + off + (int64_t)k * TPL * D * 2);
    }
  };

  int cnt;
  Cursor first;
  BlockMeta meta;
  wave_range(a, it, w, cnt, first, meta);
  auto tile = [&](const u32x4* kc, const u32x4* vc, const Cursor& cur) {
    const uint32_t rmask = cur.m0;
    const int valid = min(16, cur.nt - cur.s * 16);
    const bool partial = valid < 16;
    float vf[NL][8];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[k][2 * e] = bf16_lo(vc[k][e]);
        vf[k][2 * e + 1] = bf16_hi(vc[k][e]);
      }
      if (partial && k * TPL + tg >= valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[k][e] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rows && ((rmask >> (r / group)) & 1u)) {
        float sc[NL];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          float d = 0.f;
          d = dot2_bf16(qh[r].x, kc[k][0], d);
          d = dot2_bf16(qh[r].y, kc[k][1], d);
          d = dot2_bf16(qh[r].z, kc[k][2], d);
          d = dot2_bf16(qh[r].w, kc[k][3], d);
          if (any_lo) {
            d = dot2_bf16(ql[r].x, kc[k][0], d);
            d = dot2_bf16(ql[r].y, kc[k][1], d);
            d = dot2_bf16(ql[r].z, kc[k][2], d);
            d = dot2_bf16(ql[r].w, kc[k][3], d);
          }
          d = group_sum<LPT>(d);
          sc[k] = (partial && k * TPL + tg >= valid) ? -INFINITY : d * a.sl2e;
        }
        float mx = sc[0];
#pragma unroll
        for (int k = 1; k < NL; ++k) mx = fmaxf(mx, sc[k]);
        // the reference max is raised lazily (weights up to 2^kSlack)
        if (__builtin_amdgcn_ballot_w64(mx > m[r] + kSlack) != 0) {
          const float mn = fmaxf(m[r], mx);
          const float alpha = ex2(m[r] - mn);
          m[r] = mn;
          l[r] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
        }
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          const float pk = ex2(sc[k] - m[r]);
          l[r] += pk;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] += pk * vf[k][e];
        }
      }
    }
  };
  u32x4 ks[3][NL], vs[3][NL];
  Cursor cs[3] = {first, first, first}, lc = first;
  int issued = 0;
  ring3(
      cnt,
      [&](const int S) {
        if (issued > 0) lc = advance(a, it, meta, lc);
        cs[S] = lc;
        load(ks[S], vs[S], lc);
        ++issued;
      },
      [&](const int S) { tile(ks[S], vs[S], cs[S]); });

  // merge the token groups inside the wave (butterfly: every lane ends with the total)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) {
      float M = m[r];
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
      const float sc = ex2(m[r] - M);
      float lr = l[r] * sc;
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) lr += __shfl_xor(lr, off);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float o = acc[r][e] * sc;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) o += __shfl_xor(o, off);
        acc[r][e] = o;
      }
      m[r] = M;
      l[r] = lr;
    }
  }
  merge_store<D, 8, R>(a, it, g, rows, m, l, acc, sh);
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int D, int R>
__device__ __forceinline__ void run_q4(const TileArgs& a, const kvp_item& it, const int g, MergeLds<D>& sh) {
  constexpr int LPT = D / 16;    // lanes per token row (16 codes = 8 bytes each)
  constexpr int TPL = 64 / LPT;  // tokens per wave-wide load
  constexpr int NL = 16 / TPL;   // loads per lane per 16-token tile
  constexpr int NG = D / 64;     // quantisation groups per row
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int dq = (lane % LPT) * 16;
  const int grp = dq / 64;
  const int tg = lane / LPT;
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;

  float qf[R][16], qsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    qsum[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) qf[r][i] = 0.f;
    if (r < rows) {
      const int c = r / group;
      const int hq = g * group + (r - c * group);
      uint4 h0, h1, l0, l1;
      load_q8<D>(a, it.cons_begin + c, hq, dq, h0, l0);
      load_q8<D>(a, it.cons_begin + c, hq, dq + 8, h1, l1);
      const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      const uint32_t lw[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qf[r][2 * i] = bf16_lo(hw[i]) + bf16_lo(lw[i]);
        qf[r][2 * i + 1] = bf16_hi(hw[i]) + bf16_hi(lw[i]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) qsum[r] += qf[r][i];
    }
  }
  float m[R], l[R], acc[R][16], zacc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegBig;
    l[r] = 0.f;
    zacc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
  }

  constexpr int64_t kRowBytes = D / 2;
  constexpr int64_t kParBytes = NG * 4;
  const int64_t head_codes = (int64_t)a.B * kRowBytes;
  const int64_t head_par = (int64_t)a.B * kParBytes;
  auto load = [&](u32x2* kk, u32x2* vv, uint32_t* kq, uint32_t* vq, const Cursor& c) {
    const int64_t hb = (a.layer_blocks + c.p) * a.Hkv + g;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int tk = c.s * 16 + k * TPL + tg;
      const int64_t co = hb * head_codes + tk * kRowBytes + dq / 2;
      const int64_t po = hb * head_par + tk * kParBytes + grp * 4;
      kk[k] = ld_nt8(a.kpool + co);
      vv[k] = ld_nt8(a.vpool + co);
      kq[k] = ld_nt4(a.kpar + po);
      vq[k] = ld_nt4(a.vpar + po);
    }
  };

  int cnt;
  Cursor first;
  BlockMeta meta;
  wave_range(a, it, w, cnt, first, meta);
  // codes of one 16-code run -> floats (low nibble = even element)
  auto codes = [](const u32x2 c, float (&f)[16]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t lo = c[e] & 0x0f0f0f0fu, hi = (c[e] >> 4) & 0x0f0f0f0fu;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f[8 * e + 2 * b] = (float)((lo >> (8 * b)) & 0xffu);
        f[8 * e + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xffu);
      }
    }
  };
  // K codes are dequantised one token run at a time for every row's score, then
  // V codes for every row's accumulation: the two are never live together
  auto tile = [&](const u32x2* kc, const u32x2* vc, const uint32_t* kp, const uint32_t* vp, const Cursor& cur) {
    const uint32_t rmask = cur.m0;
    const int valid = min(16, cur.nt - cur.s * 16);
    bool act[R];
#pragma unroll
    for (int r = 0; r < R; ++r) act[r] = r < rows && ((rmask >> (r / group)) & 1u);
    float sc[R][NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const bool ok = k * TPL + tg < valid;
      float ck[16];
      codes(kc[k], ck);
      const float sk = half_bits_to_f32(kp[k] & 0xffffu), zk = half_bits_to_f32(kp[k] >> 16);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (act[r]) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) d += qf[r][e] * ck[e];
          d = sk * d + zk * qsum[r];
          d = group_sum<LPT>(d);
          sc[r][k] = ok ? d * a.sl2e : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (act[r]) {
        float mx = sc[r][0];
#pragma unroll
        for (int k = 1; k < NL; ++k) mx = fmaxf(mx, sc[r][k]);
        // the reference max is raised lazily (weights up to 2^kSlack)
        if (__builtin_amdgcn_ballot_w64(mx > m[r] + kSlack) != 0) {
          const float mn = fmaxf(m[r], mx);
          const float alpha = ex2(m[r] - mn);
          m[r] = mn;
          l[r] *= alpha;
          zacc[r] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[r][e] *= alpha;
        }
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          sc[r][k] = ex2(sc[r][k] - m[r]);
          l[r] += sc[r][k];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const bool ok = k * TPL + tg < valid;
      float cv[16];
      codes(vc[k], cv);
      const float sv = ok ? half_bits_to_f32(vp[k] & 0xffffu) : 0.f;
      const float zv = ok ? half_bits_to_f32(vp[k] >> 16) : 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (act[r]) {
          const float ps = sc[r][k] * sv;
          zacc[r] += sc[r][k] * zv;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[r][e] += ps * cv[e];
        }
      }
    }
  };
  // three register sets for up to 4 rows, two above (the row state grows)
  constexpr int NS = R <= 4 ? 3 : 2;
  u32x2 ks[NS][NL], vs[NS][NL];
  uint32_t kps[NS][NL], vps[NS][NL];
  Cursor cs[NS], lc = first;
  int issued = 0;
  auto issue = [&](const int S) {
    if (issued > 0) lc = advance(a, it, meta, lc);
    cs[S] = lc;
    load(ks[S], vs[S], kps[S], vps[S], lc);
    ++issued;
  };
  auto run = [&](const int S) { tile(ks[S], vs[S], kps[S], vps[S], cs[S]); };
  if constexpr (NS == 3) ring3(cnt, issue, run); else ring2(cnt, issue, run);

#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) {
      float M = m[r];
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
      const float sc = ex2(m[r] - M);
      float lr = l[r] * sc;
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) lr += __shfl_xor(lr, off);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float o = (acc[r][e] + zacc[r]) * sc;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) o += __shfl_xor(o, off);
        acc[r][e] = o;
      }
      m[r] = M;
      l[r] = lr;
    }
  }
  merge_store<D, 16, R>(a, it, g, rows, m, l, acc, sh);
}

// ---------------------------------------------------------------------------
// Matrix-core path for items with several query rows (up to 16 per wave): the
// multi-query contraction against each shared block runs on MFMA.
//   S^T (16 tokens x 16 rows) = K (16 x D) . Q^T        v_mfma_f32_16x16x32_bf16
//   O^T (D x 16 rows)        += V^T (D x 16) . P^T      v_mfma_f32_16x16x16_bf16
// Operand layouts (gfx950, checked on the device): for 16x16xK, lane l holds
// A[row l%16][k-run (l/16)], B[k-run (l/16)][col l%16], and the result
// D[rows 4*(l/16)+v][col l%16], v = 0..3.  The token order inside a tile is
// free (the PV contraction sums over it), and it is chosen so that no operand
// needs a transpose: A-row / k-slot 4q+v holds token q+4v.  Then
//  - K goes from HBM straight into A (lane l: token sigma(l%16), dims
//    32m + 8*(l/16) + [0,8)), sigma(4q+v) = q+4v;
//  - the S^T result is P^T's B operand as it stands (lane l: row l%16, tokens
//    l/16 + 4v), and each lane owns one query row for the softmax bookkeeping;
//  - V is read in its natural layout, D/16 consecutive dims of tokens l/16 + 4v
//    per lane, and V^T's A operand for MFMA e takes dim e of those runs, so the
//    output rows of MFMA e are dims i*(D/16) + e, i = 0..15.
// P is split into bf16 hi + lo (two MFMAs) to keep the weights' rounding
// below 2^-16.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct MfmaLds {
  struct Per {
    float acc[16][D];  // the wave's result rows, for the cross-wave merge
  } per[kWaves];
  float ml[kWaves][16][2];
};

// k-slot / A-row 4q+v of a 16-token tile holds token q+4v
__device__ __forceinline__ int tile_token(int i) { return (i >> 2) + 4 * (i & 3); }

// V^T's A operand for output dims i*(D/16) + e: element v is dim e of token
// (l/16) + 4v, taken from the lane's four natural-layout V words
__device__ __forceinline__ s16x4_t v_operand(const u32x4* vz, const int e) {
  const int wd = e >> 1;
  uint32_t a01, a23;
  if (e & 1) {
    a01 = (vz[0][wd] >> 16) | (vz[1][wd] & 0xffff0000u);
    a23 = (vz[2][wd] >> 16) | (vz[3][wd] & 0xffff0000u);
  } else {
    a01 = (vz[0][wd] & 0xffffu) | (vz[1][wd] << 16);
    a23 = (vz[2][wd] & 0xffffu) | (vz[3][wd] << 16);
  }
  return __builtin_bit_cast(s16x4_t, make_uint2(a01, a23));
}

// result rows to row-major memory: acc[e][v] is dim (4*lq + v)*(D/16) + e
template <int D>
__device__ __forceinline__ void store_rows(float* row_base, const int lq, const f32x4_t* acc) {
  constexpr int E = D / 16;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const f32x4_t o = (f32x4_t){acc[4 * h][v], acc[4 * h + 1][v], acc[4 * h + 2][v], acc[4 * h + 3][v]};
      *(f32x4_t*)(row_base + (4 * lq + v) * E + 4 * h) = o;
    }
  }
}




template <int D>
__device__ __forceinline__ void run_mfma(const TileArgs& a, const kvp_item& it, const int g, MfmaLds<D>& sh) {
  constexpr int NM = D / 32;  // QK MFMAs (k = 32 dims each)
  constexpr int NO = D / 16;  // PV MFMAs (16 output dims each)
  constexpr int NL = 4;       // V loads per lane per tile (tokens l/16 + 4v)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15;   // this lane's query row / token in A
  const int lq = lane >> 4;   // k-run index
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;

  bool any_lo = false;
  for (int c = it.cons_begin; c < it.cons_end; ++c) any_lo |= a.cons[c] >= a.n_unshifted;

  // B operand of S^T: Q^T, lane l: row l%16, dims 32m + 8*(l/16) + [0, 8)
  uint4 qh[NM], ql[NM];
  const int crow = lr / group;
#pragma unroll
  for (int m = 0; m < NM; ++m) qh[m] = ql[m] = make_uint4(0, 0, 0, 0);
  if (lr < rows)
#pragma unroll
    for (int m = 0; m < NM / 2; ++m)  // dims 32m + 8*lq and D/2 + 32m + 8*lq: the same rotate-half pairs
      load_q16<D>(a, it.cons_begin + crow, g * group + (lr - crow * group), 32 * m + 8 * lq, qh[m], ql[m],
                  qh[m + NM / 2], ql[m + NM / 2]);

  float mrow = kNegBig, lsum = 0.f;
  f32x4_t acc[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  constexpr int64_t kTileBytes = 16 * D * 2;
  const int64_t head_bytes = (int64_t)a.B * D * 2;
  const int64_t k_lane = (int64_t)tile_token(lr) * D * 2 + 8 * lq * 2;  // A-operand layout
  const int64_t v_lane = (int64_t)lq * D * 2 + lr * (D / 16) * 2;          // natural layout
  auto load = [&](u32x4* kk, u32x4* vv, const Cursor& c) {
    const int64_t off = ((a.layer_blocks + c.p) * a.Hkv + g) * head_bytes + c.s * kTileBytes;
#pragma unroll
    for (int m = 0; m < NM; ++m) kk[m] = ld_nt16(a.kpool + off + k_lane + 64 * m);
#pragma unroll
    for (int v = 0; v < NL; ++v) {
      const uint8_t* src = a.vpool + off + v_lane + (int64_t)v * 4 * D * 2;
      if constexpr (D == 128) {
        vv[v] = ld_nt16(src);
      } else {
        const u32x2 t = ld_nt8(src);
        vv[v] = (u32x4){t.x, t.y, 0u, 0u};
      }
    }
  };

  int cnt;
  Cursor first;
  BlockMeta meta;
  wave_range(a, it, w, cnt, first, meta);
  // one 16-token tile: S^T = K Q^T, online softmax, O^T += V^T P^T
  const int ncons = it.cons_end - it.cons_begin;
  const uint32_t fm0 = ncons >= 32 ? ~0u : ((1u << ncons) - 1u);
  auto tile = [&](const u32x4* kc, const u32x4* vc, const Cursor& cur) {
    const uint32_t rmask = cur.m0;
    const int valid = min(16, cur.nt - cur.s * 16);
    const bool row_reads = lr < rows && ((rmask >> crow) & 1u);
    // a full tile that every row of the item reads needs no masking (wave-uniform;
    // rows past the item's have zero q: finite scores that nothing uses)
    const bool plain = valid == 16 && (rmask & fm0) == fm0;

    // padding tokens are zeroed (they may hold NaN)
    u32x4 vz[NL];
    if (valid == 16) {
#pragma unroll
      for (int v = 0; v < NL; ++v) vz[v] = vc[v];
    } else {
#pragma unroll
      for (int v = 0; v < NL; ++v) vz[v] = lq + 4 * v < valid ? vc[v] : (u32x4){0u, 0u, 0u, 0u};
    }

    // S^T = K Q^T
    f32x4_t s = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const bf16x8_t kA = __builtin_bit_cast(bf16x8_t, kc[m]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8_t, qh[m]), s, 0, 0, 0);
      if (any_lo) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8_t, ql[m]), s, 0, 0, 0);
    }
    // online softmax for row lr over tokens lq + 4v
    float sc[4], mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sc[v] = (plain || (row_reads && lq + 4 * v < valid)) ? s[v] * a.sl2e : -INFINITY;
      mx = fmaxf(mx, sc[v]);
    }
    if (__builtin_amdgcn_ballot_w64(mx > mrow + kSlack) != 0) {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(mrow, mx);
      const float alpha = ex2(mrow - mn);
      mrow = mn;
      lsum *= alpha;
#pragma unroll
      for (int n = 0; n < NO; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = ex2(sc[v] - mrow);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    const uint32_t ph0 = pack_bf16(p[0], p[1]), ph1 = pack_bf16(p[2], p[3]);
    const uint32_t pl0 = pack_bf16(p[0] - bf16_lo(ph0), p[1] - bf16_hi(ph0));
    const uint32_t pl1 = pack_bf16(p[2] - bf16_lo(ph1), p[3] - bf16_hi(ph1));
    const s16x4_t pH = __builtin_bit_cast(s16x4_t, make_uint2(ph0, ph1));
    const s16x4_t pL = __builtin_bit_cast(s16x4_t, make_uint2(pl0, pl1));

    // O^T += V^T P^T
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const s16x4_t vA = v_operand(vz, n);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA, pH, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA, pL, acc[n], 0, 0, 0);
    }
  };
  u32x4 ks[3][NM], vs[3][NL];
  Cursor cs[3] = {first, first, first}, lc = first;
  int issued = 0;
  ring3(
      cnt,
      [&](const int S) {
        if (issued > 0) lc = advance(a, it, meta, lc);
        cs[S] = lc;
        load(ks[S], vs[S], lc);
        ++issued;
      },
      [&](const int S) { tile(ks[S], vs[S], cs[S]); });
  // row totals: the 4 lanes of a row hold disjoint token subsets of the sum
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // cross-wave merge: wave w's rows to LDS, row-major
  store_rows<D>(&sh.per[w].acc[lr][0], lq, acc);
  if (lq == 0) {
    sh.ml[w][lr][0] = mrow;
    sh.ml[w][lr][1] = lsum;
  }
  __syncthreads();
  if (w == 0 && lr < rows) {
    float mx = sh.ml[0][lr][0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) mx = fmaxf(mx, sh.ml[v][lr][0]);
    float scw[kWaves], lt = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      scw[v] = ex2(sh.ml[v][lr][0] - mx);
      lt += scw[v] * sh.ml[v][lr][1];
    }
    const int64_t row = (int64_t)g * a.P + it.part_base + lr;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      f32x4_t o = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) o += scw[v] * *(const f32x4_t*)(&sh.per[v].acc[0][0] + lr * D + 16 * n + 4 * lq);
      *(f32x4_t*)(a.pacc + row * D + 16 * n + 4 * lq) = o;
    }
    if (lq == 0) a.pml[row] = make_float2(mx, lt);
  }
}

// ---------------------------------------------------------------------------
// Wide matrix-core path: a bf16 block read by many consumer rows (a shared
// segment read by every agent of a round, times the GQA heads; the planner makes
// wide items for pools of 16-token blocks only, so a tile is a block).  The 4
// waves of the workgroup load each pair of blocks into LDS once, straight from
// HBM (global_load_lds: no registers), into a ring of kStages pair slots, so that
// the loads of the next kStages - 1 pairs are in flight while a pair is computed;
// every wave multiplies its own 16 or 32 rows against the staged K and V -- one
// HBM read of the block for up to 128 rows.  The item's block table (physical
// id, valid tokens, consumer masks) is staged in LDS once at the start.
//   S^T (16 tokens x 16 rows) = K . Q^T per tile   v_mfma_f32_16x16x32_bf16
//   O^T (D x 16 rows) += V^T (D x 32) . P^T         v_mfma_f32_16x16x32_bf16
// PV contracts over the pair's 32 tokens: k-slot 8q + j holds token 4q + j of
// the first tile (j < 4) or 4q + j - 4 of the second, which are exactly the
// tokens of the two S^T results a lane holds.  V^T's A operand comes from the
// staged natural-layout V by the LDS transpose read (ds_read_b64_tr_b16): in
// each 16-lane group, lane i receives word i%4 of the 8-byte runs addressed by
// lanes 4v + i/4, so lane (q, s) addresses token 4q + s/4, dims 16n + 4(s%4).
// A staged tile keeps its token rows in order, and the 16-byte chunks of row t
// in the order c ^ (t & 7) (an XOR swizzle: the K-operand reads of 16 rows and
// the transpose reads of 4 rows fall on different banks).
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
typedef short s16x8_t __attribute__((ext_vector_type(8)));

template <int D>
struct WideLds {
  static constexpr int kStages = 4;
  static constexpr int kRow = D * 2;        // bytes per token row
  static constexpr int kTile = 16 * kRow;   // one 16-token tile of K or of V
  static constexpr int kStage = 4 * kTile;  // K of tiles a, b, then V of tiles a, b
  static constexpr int kMaxBlocks = kMaxBlocksWide;  // blocks of one wide item (the plan checks it)
  alignas(16) uint8_t ring[kStages][kStage];
  // the item's blocks: physical id, valid tokens, consumer mask words
  alignas(16) uint32_t table[kMaxBlocks][4];
};

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima)
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

template <int NLD>
__device__ __forceinline__ void wait_newer_stages(int k) {
  // k pairs issued after the one awaited, NLD loads each
  switch (k) {
    case 0: __builtin_amdgcn_s_waitcnt(vm_wait(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vm_wait(NLD)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_wait(2 * NLD)); break;
  }
}

// LDS reads of the ring and the workgroup barrier in inline assembly: the
// compiler counts the ring's loads as pending writes to LDS and would otherwise
// wait for all of them (s_waitcnt vmcnt(0)) before any LDS read or barrier,
// which drains the loads in flight for later pairs.  The barrier is a compiler
// memory barrier.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// LDS reads issued without waiting for them, so that their latency overlaps
// other work; lds_wait_* waits for all of them and passes the registers through
// the waiting statement, so that no use of a result can be scheduled before it.
__device__ __forceinline__ void lds_issue_b128(uint32_t addr, u32x4& r) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
}
__device__ __forceinline__ void lds_issue_tr(uint32_t addr, u32x2& r) {
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
}
template <int N>
__device__ __forceinline__ void lds_wait_b128(u32x4 (&r)[N]) {
  if constexpr (N == 12)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]),
                   "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]));
  else if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]));
  else
    static_assert(N == 12 || N == 8, "read batch sizes used by the wide path");
}
template <int N>
__device__ __forceinline__ void lds_wait_b64(u32x2 (&r)[N]) {
  if constexpr (N == 16)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]),
                   "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]), "+v"(r[12]), "+v"(r[13]), "+v"(r[14]),
                   "+v"(r[15]));
  else if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]));
  else
    static_assert(N == 16 || N == 8, "read batch sizes used by the wide path");
}

// Two 16-byte LDS reads (the same addresses in every lane: broadcast).
__device__ __forceinline__ void lds_read2_b128(uint32_t a0, uint32_t a1, u32x4& r0, u32x4& r1) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(r0), "=&v"(r1)
               : "v"(a0), "v"(a1));
}

template <int D, int RT>
__device__ __forceinline__ void run_wide(const TileArgs& a, const kvp_item& it, const int g, WideLds<D>& sh) {
  constexpr int NM = D / 32, NO = D / 16;
  constexpr int NS = WideLds<D>::kStages;
  constexpr int kRow = WideLds<D>::kRow, kTile = WideLds<D>::kTile, kStage = WideLds<D>::kStage;
  constexpr int NLD = kStage / (256 * 16);  // 16-byte loads per thread per pair
  static_assert(NS == 4, "the wait switch covers up to two newer pairs");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;
  const bool active = w * 16 * RT < rows;

  bool any_lo = false;
  for (int c = it.cons_begin; c < it.cons_end; ++c) any_lo |= a.cons[c] >= a.n_unshifted;
  // mask bits of all the item's consumers (a block whose mask words cover them
  // is read by every row)
  const int ncons = it.cons_end - it.cons_begin;
  const uint32_t fm0 = ncons >= 32 ? ~0u : ((1u << ncons) - 1u);
  const uint32_t fm1 = ncons >= 64 ? ~0u : ncons > 32 ? ((1u << (ncons - 32)) - 1u) : 0u;

  // this wave's rows: w*16*RT + 16t + lr for row tile t (B operand of S^T: lane l
  // holds row l%16, dims 32m + 8*(l/16))
  uint4 qh[RT][NM], ql[RT][NM];
  int rr[RT], rc[RT];
  bool rv[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    rr[t] = w * 16 * RT + 16 * t + lr;
    rv[t] = rr[t] < rows;
    rc[t] = rv[t] ? rr[t] / group : 0;
#pragma unroll
    for (int m = 0; m < NM; ++m) qh[t][m] = ql[t][m] = make_uint4(0, 0, 0, 0);
    if (rv[t])
#pragma unroll
      for (int m = 0; m < NM / 2; ++m)  // dims 32m + 8*lq and D/2 + 32m + 8*lq: the same rotate-half pairs
        load_q16<D>(a, it.cons_begin + rc[t], g * group + (rr[t] - rc[t] * group), 32 * m + 8 * lq, qh[t][m],
                    ql[t][m], qh[t][m + NM / 2], ql[t][m + NM / 2]);
  }
  float mrow[RT], lsum[RT];
  f32x4_t acc[RT][NO];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    mrow[t] = kNegBig;
    lsum[t] = 0.f;
#pragma unroll
    for (int n = 0; n < NO; ++n) acc[t][n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }

  // the item's blocks, two per step (pair i = blocks 2i, 2i + 1)
  const int T = it.blk_end - it.blk_begin;
  const int nsteps = (T + 1) >> 1;
  const int64_t head_bytes = (int64_t)16 * D * 2;
  const int64_t head_base = (a.layer_blocks * a.Hkv + g) * head_bytes;  // + p * Hkv * head_bytes
  const int64_t blk_stride = (int64_t)a.Hkv * head_bytes;

  // the item's block table in LDS, filled once: physical id, valid tokens and
  // consumer mask words of each block
  for (int t = tid; t < T; t += 256) {
    const int p = a.plan_blocks[it.blk_begin + t];
    uint32_t m0 = ~0u, m1 = ~0u;
    if (it.mask_base >= 0) {
      const uint32_t* mw = a.mask + it.mask_base + (int64_t)t * it.mask_stride;
      m0 = mw[0];
      if (it.mask_stride > 1) m1 = mw[1];
    }
    *(u32x4*)&sh.table[t][0] = (u32x4){(uint32_t)p, (uint32_t)a.plan_ntok[it.blk_begin + t], m0, m1};
  }
  __syncthreads();
  const uint32_t table_base = lds_addr(&sh.table[0][0]);
  // blocks 2j and 2j + 1 of the table (a missing second block of an odd item
  // reads the first again, with 0 valid tokens)
  auto pair_info = [&](const int j, u32x4& ea, u32x4& eb) {
    const int tb = min(2 * j + 1, T - 1);
    lds_read2_b128(table_base + 32 * j, table_base + 16 * tb, ea, eb);
    if (2 * j + 1 >= T) eb.y = 0u;
  };
  // this thread's 16-byte chunks of a staged pair: byte o = (q*4 + w)*1024 +
  // lane*16 of the slot; part o / kTile (K a, K b, V a, V b), token row and
  // swizzled chunk inside the tile, and the source chunk c = c' ^ (t & 7)
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int src_off[NLD], src_tok[NLD];
  uint32_t src_full[NLD];
#pragma unroll
  for (int q = 0; q < NLD; ++q) {
    const int o = (q * 4 + wu) * 1024 + lane * 16;
    const int r = o % kTile, t = r / kRow, cs = (r % kRow) / 16;
    src_tok[q] = t;
    src_off[q] = ((cs ^ (t & 7)) * 16);
    src_full[q] = (uint32_t)(t * kRow + src_off[q]);
  }
  // loads of pair j into ring slot j % NS, given its two table entries
  // (the block's base address is wave-uniform, in scalar registers; a lane adds
  // a 32-bit offset: the token row's, or row 0's for a padding token)
  auto issue_with = [&](const int j, const u32x4& ea, const u32x4& eb) {
    const int pa = __builtin_amdgcn_readfirstlane((int)ea.x), pb = __builtin_amdgcn_readfirstlane((int)eb.x);
    const int va = min(16, __builtin_amdgcn_readfirstlane((int)ea.y));
    const int vb = min(16, __builtin_amdgcn_readfirstlane((int)eb.y));
    const int64_t oa = head_base + (int64_t)pa * blk_stride;
    const int64_t ob = head_base + (int64_t)pb * blk_stride;
    uint8_t* dst = &sh.ring[j % NS][0];
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int part = (q * 4 + wu) * 1024 / kTile;  // wave-uniform
      const bool second = part & 1;
      // a padding token (or the missing second block of an odd item) loads row 0
      // of its block instead: finite values, whose weights are zero
      const uint32_t off = src_tok[q] < (second ? vb : va) ? src_full[q] : (uint32_t)src_off[q];
      const uint8_t* base = (part >= 2 ? a.vpool : a.kpool) + (second ? ob : oa);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(base + off),
                                       (__attribute__((address_space(3))) void*)(dst + (q * 4 + wu) * 1024), 16, 0,
                                       kWideLoadPolicy);
    }
  };
  auto issue = [&](const int j) {
    u32x4 ea, eb;
    pair_info(j, ea, eb);
    issue_with(j, ea, eb);
  };
  // LDS byte offsets inside a staged tile, through the chunk swizzle: K-operand
  // chunks (token lr, dims 32m + 8*lq) and V transpose-read runs (token vrow,
  // dims 16n + 4*(lr%4))
  const int vrow = 4 * lq + (lr >> 2);
  auto k_off = [&](int m) { return (uint32_t)(lr * kRow + (((4 * m + lq) ^ (lr & 7)) * 16)); };
  auto v_off = [&](int n) {
    return (uint32_t)(vrow * kRow + (((2 * n + ((lr & 3) >> 1)) ^ (vrow & 7)) * 16) + (lr & 1) * 8);
  };
  // S^T of both blocks of a staged pair for every row tile; each block's K
  // operands are read from LDS once and serve every row tile.  Lane l holds row
  // lr, tokens 4*lq + v.
  auto scores = [&](const u32x4* krr, f32x4_t (&svv)[RT][2]) {
    // row tile by row tile, so that the first tile's softmax can start while
    // the second tile's MFMAs run
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4* kr = krr + st * NM;
        f32x4_t acc_s = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        if (any_lo) {
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const bf16x8_t kA = __builtin_bit_cast(bf16x8_t, kr[m]);
            acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8_t, qh[t][m]), acc_s, 0, 0, 0);
            acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8_t, ql[t][m]), acc_s, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int m = 0; m < NM; ++m)
            acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[m]),
                                                            __builtin_bit_cast(bf16x8_t, qh[t][m]), acc_s, 0, 0, 0);
        }
        svv[t][st] = acc_s;
      }
    }
  };

  // the queries are in registers before the ring's loads start (the loop then
  // has only the ring's loads to wait for)
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  // prologue: pairs 0 .. NS-2 in flight; the scores of pair 0
  issue(0);
#pragma unroll
  for (int s = 1; s < NS - 1; ++s)
    if (s < nsteps) issue(s);
  for (int step = 0; step < nsteps; ++step) {
    // this wave's loads of pair `step` have landed; the barrier makes every
    // wave's visible and retires the slot the issue below overwrites (read in
    // the previous step)
    wait_newer_stages<NLD>(__builtin_amdgcn_readfirstlane(min(NS - 2, nsteps - 1 - step)));
    wg_barrier();
    // one batch of LDS reads: the table entries of this pair and of the pair
    // issued below, and both blocks' K operands
    const uint8_t* stg = &sh.ring[step % NS][0];
    const uint32_t kb = lds_addr(stg);
    const int jn = min(step + NS - 1, nsteps - 1);
    u32x4 rd[4 + 2 * NM];
    lds_issue_b128(table_base + 32 * step, rd[0]);
    lds_issue_b128(table_base + 16 * min(2 * step + 1, T - 1), rd[1]);
    lds_issue_b128(table_base + 32 * jn, rd[2]);
    lds_issue_b128(table_base + 16 * min(2 * jn + 1, T - 1), rd[3]);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int m = 0; m < NM; ++m) lds_issue_b128(kb + st * kTile + k_off(m), rd[4 + st * NM + m]);
    lds_wait_b128<4 + 2 * NM>(rd);
    if (2 * jn + 1 >= T) rd[3].y = 0u;
    if (step + NS - 1 < nsteps) issue_with(step + NS - 1, rd[2], rd[3]);
    if (!active) continue;
    f32x4_t s_cur[RT][2];
    scores(&rd[4], s_cur);
    // the V^T operands of the pair: issued now, consumed after the softmax
    const uint32_t vbase = kb + 2 * kTile;
    u32x2 vr[2 * NO];
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      lds_issue_tr(vbase + v_off(n), vr[2 * n]);
      lds_issue_tr(vbase + kTile + v_off(n), vr[2 * n + 1]);
    }
    u32x4 ea = rd[0], eb = rd[1];
    if (2 * step + 1 >= T) eb.y = 0u;
    const int valid[2] = {min(16, __builtin_amdgcn_readfirstlane((int)ea.y)),
                          min(16, __builtin_amdgcn_readfirstlane((int)eb.y))};
    const uint32_t mw0[2] = {(uint32_t)__builtin_amdgcn_readfirstlane((int)ea.z),
                             (uint32_t)__builtin_amdgcn_readfirstlane((int)eb.z)};
    const uint32_t mw1[2] = {(uint32_t)__builtin_amdgcn_readfirstlane((int)ea.w),
                             (uint32_t)__builtin_amdgcn_readfirstlane((int)eb.w)};
    // two full blocks that every row of the item reads need no masking (rows
    // past the item's have zero q: finite scores that nothing uses)
    const bool plain = valid[0] == 16 && valid[1] == 16 && (mw0[0] & mw0[1] & fm0) == fm0 &&
                       (mw1[0] & mw1[1] & fm1) == fm1;
    bf16x8_t pH[RT], pL[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const f32x4_t* sv = s_cur[t];
      float sc[8], mx = -INFINITY;
      if (plain) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            sc[4 * st + v] = sv[st][v] * a.sl2e;
            mx = fmaxf(mx, sc[4 * st + v]);
          }
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bool reads = rv[t];
          if (reads) {
            const uint32_t word = (rc[t] >> 5) ? mw1[st] : mw0[st];
            reads = (word >> (rc[t] & 31)) & 1u;
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            sc[4 * st + v] = (reads && 4 * lq + v < valid[st]) ? sv[st][v] * a.sl2e : -INFINITY;
            mx = fmaxf(mx, sc[4 * st + v]);
          }
        }
      }
      if (__builtin_amdgcn_ballot_w64(mx > mrow[t] + kSlack) != 0) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(mrow[t], mx);
        const float alpha = ex2(mrow[t] - mn);
        mrow[t] = mn;
        lsum[t] *= alpha;
#pragma unroll
        for (int n = 0; n < NO; ++n) acc[t][n] *= alpha;
      }
      float p[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) p[v] = ex2(sc[v] - mrow[t]);
      lsum[t] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[i] = pack_bf16(p[2 * i], p[2 * i + 1]);
        pl[i] = pack_bf16(p[2 * i] - bf16_lo(ph[i]), p[2 * i + 1] - bf16_hi(ph[i]));
      }
      pH[t] = __builtin_bit_cast(bf16x8_t, (u32x4){ph[0], ph[1], ph[2], ph[3]});
      pL[t] = __builtin_bit_cast(bf16x8_t, (u32x4){pl[0], pl[1], pl[2], pl[3]});
      // O^T += V^T P^T over the 32 tokens of the pair for this row tile (its
      // MFMAs run under the next row tile's softmax); the V^T operands serve
      // every row tile
      if (t == 0) lds_wait_b64<2 * NO>(vr);
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        const bf16x8_t vA =
            __builtin_bit_cast(bf16x8_t, (u32x4){vr[2 * n].x, vr[2 * n].y, vr[2 * n + 1].x, vr[2 * n + 1].y});
        acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, pH[t], acc[t][n], 0, 0, 0);
        acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, pL[t], acc[t][n], 0, 0, 0);
      }
    }
  }
  // no load into the ring may outlive the workgroup
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  if (!active) return;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    float l = lsum[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!rv[t]) continue;
    // acc[t][n][v] is dim 16n + 4*lq + v of row rr[t]
    const int64_t row = (int64_t)g * a.P + it.part_base + rr[t];
#pragma unroll
    for (int n = 0; n < NO; ++n) *(f32x4_t*)(a.pacc + row * D + 16 * n + 4 * lq) = acc[t][n];
    if (lq == 0) a.pml[row] = make_float2(mrow[t], l);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path for Q4 items with several rows.  Codes 0..15 are exact in
// bf16, so both contractions run on the codes themselves and the per-token
// scale s and zero z of each 64-dim group are applied outside the MFMAs:
//   score_t = sum_g s_tg (C_g q_g)_t + z_tg sum(q_g)        (one S^T chain per group)
//   o_e     = sum_t (p_t s_tg) c_te + sum_t p_t z_tg,   g = group of dim e
// QK: MFMA m covers dims 64(m/2) + 16(l/16) + 8(m%2) + [0, 8) in lane l (a
// permutation of the dims inside each group, applied to q and K alike), so a
// lane's K codes of one group are 8 contiguous bytes and every MFMA stays in
// one group.  Tokens are in natural order (lane l: token l%16 in A, tokens
// 4(l/16) + v of the result).  PV: each wave converts its tile's V codes to
// bf16 in an LDS stage ([token][dim] layout) and reads V^T's operand with the
// transpose read; the B operand is P' = p * s of the group, split into bf16
// hi + lo.
// Conversion: code c OR 0x4300 is the bf16 of 128 + c (exact), one byte
// permute per pair of codes.  A dword of 8 codes becomes 4 bf16 pairs holding
// its elements in the order (0 2 4 6 1 3 5 7); q is permuted alike once per
// item, V's staged dims carry the permutation into the output positions, which
// the final write undoes.  The offsets are removed exactly where they arise:
// the S chain starts at -128 sum(q) (from the same bf16 q the MFMAs read), and
// one extra MFMA per group against a constant-128 operand accumulates
// 128 sum_t P'_t from the same bf16 P' (subtracted at the end).
template <int D>
struct Q4Lds {
  static constexpr int kVStride = D + 16;  // u16 per staged row (8-row transpose reads hit distinct banks)
  union Per {
    alignas(16) uint16_t v[16 * kVStride];  // the wave's V codes as bf16
    float acc[16][D];                       // the wave's result rows, for the cross-wave merge
  } per[kWaves];
  float ml[kWaves][16][2];
};

// 8 codes (one dword, low nibble = even element) -> 4 packed bf16 pairs of
// 128 + code, elements in the order (0 2 4 6 1 3 5 7)
__device__ __forceinline__ void codes_bf16(const uint32_t x, uint32_t* o) {
  constexpr uint32_t k43 = 0x43434343u;
  const uint32_t lo = x & 0x0f0f0f0fu, hi = (x >> 4) & 0x0f0f0f0fu;
  // byte selectors: 0-3 pick from the codes, 4 picks 0x43
  o[0] = __builtin_amdgcn_perm(k43, lo, 0x04010400u);
  o[1] = __builtin_amdgcn_perm(k43, lo, 0x04030402u);
  o[2] = __builtin_amdgcn_perm(k43, hi, 0x04010400u);
  o[3] = __builtin_amdgcn_perm(k43, hi, 0x04030402u);
}

// 8 bf16 (4 dwords, natural order) -> the order (0 2 4 6 1 3 5 7)
__device__ __forceinline__ uint4 perm8_bf16(const uint4 x) {
  return make_uint4(__builtin_amdgcn_perm(x.y, x.x, 0x05040100u), __builtin_amdgcn_perm(x.w, x.z, 0x05040100u),
                    __builtin_amdgcn_perm(x.y, x.x, 0x07060302u), __builtin_amdgcn_perm(x.w, x.z, 0x07060302u));
}

template <int D>
struct Q4Set {
  static constexpr int NG = D / 64;
  u32x2 kc[NG];  // K codes of token l%16: group g, dims 64g + 16(l/16) + [0, 16)
  u32x4 kp[NG];  // K (s, z) words of tokens 4(l/16) + [0, 4)
  u32x4 vc;      // V codes of token l/4, dims (D/4)(l%4) + [0, D/4)  (D = 64: .xy)
  u32x4 vp[NG];  // V (s, z) words of tokens 4(l/16) + [0, 4)
};

template <int D>
__device__ __forceinline__ void run_q4m(const TileArgs& a, const kvp_item& it, const int g, Q4Lds<D>& sh) {
  constexpr int NG = D / 64;  // quantisation groups per row
  constexpr int NM = D / 32;  // QK MFMAs, two per group
  constexpr int NO = D / 16;  // PV MFMAs (16 dims each), NO / NG per group
  constexpr int SV = Q4Lds<D>::kVStride;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;

  bool any_lo = false;
  for (int c = it.cons_begin; c < it.cons_end; ++c) any_lo |= a.cons[c] >= a.n_unshifted;

  uint4 qh[NM], ql[NM];
  const int crow = lr / group;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    qh[m] = make_uint4(0, 0, 0, 0);
    ql[m] = make_uint4(0, 0, 0, 0);
    if (lr < rows)
      load_q8<D>(a, it.cons_begin + crow, g * group + (lr - crow * group), 64 * (m >> 1) + 16 * lq + 8 * (m & 1),
                 qh[m], ql[m]);
    qh[m] = perm8_bf16(qh[m]);
    ql[m] = perm8_bf16(ql[m]);
  }
  // sum of q over each group for row lr (the row's 4 lanes hold disjoint dims)
  float qs[NG];
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    float t = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 x = qh[2 * gg + h], y = ql[2 * gg + h];
      const uint32_t ws[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) t += bf16_lo(ws[k]) + bf16_hi(ws[k]);
    }
    t += __shfl_xor(t, 16);
    t += __shfl_xor(t, 32);
    qs[gg] = t;
  }

  float mrow = kNegBig, lsum = 0.f, zacc[NG];
  f32x4_t acc[NO], corr[NG];  // corr[g]: 128 sum_t P'_t of row lr (every element alike)
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    zacc[gg] = 0.f;
    corr[gg] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }
  const s16x4_t c128 = (s16x4_t){0x4300, 0x4300, 0x4300, 0x4300};
  f32x4_t s_init[NG];  // the S chains start at -128 sum(q_g)
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const float off = -128.f * qs[gg];
    s_init[gg] = (f32x4_t){off, off, off, off};
  }
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int64_t head_codes = (int64_t)a.B * (D / 2);
  const int64_t head_par = (int64_t)a.B * NG * 4;
  const int kq_lane = lr * (D / 2) + 8 * lq;                   // + 32 per group
  const int par_lane = 16 * NG * lq;                          // + 16 per load
  const int vq_lane = (lane >> 2) * (D / 2) + (lane & 3) * (D / 8);
  auto load = [&](Q4Set<D>& st, const Cursor& c) {
    const int64_t hb = (a.layer_blocks + c.p) * a.Hkv + g;
    const int64_t co = hb * head_codes + (int64_t)c.s * 16 * (D / 2);
    const int64_t po = hb * head_par + (int64_t)c.s * 16 * NG * 4;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      st.kc[gg] = ld_nt8(a.kpool + co + kq_lane + 32 * gg);
      st.kp[gg] = ld_nt16(a.kpar + po + par_lane + 16 * gg);
      st.vp[gg] = ld_nt16(a.vpar + po + par_lane + 16 * gg);
    }
    if constexpr (D == 128) {
      st.vc = ld_nt16(a.vpool + co + vq_lane);
    } else {
      const u32x2 t = ld_nt8(a.vpool + co + vq_lane);
      st.vc = (u32x4){t.x, t.y, 0u, 0u};
    }
  };
  // (s, z) word of token 4 lq + v, group gg
  auto par = [](const u32x4* pw, const int v, const int gg) -> uint32_t {
    const int k = v * NG + gg;
    return pw[k >> 2][k & 3];
  };

  uint16_t* vst = sh.per[w].v;
  int cnt;
  Cursor first;
  BlockMeta meta;
  wave_range(a, it, w, cnt, first, meta);
  auto tile = [&](const Q4Set<D>& st, const Cursor& cur) {
    const int valid = min(16, cur.nt - cur.s * 16);
    const bool row_reads = lr < rows && ((cur.m0 >> crow) & 1u);
    const bool all_read = valid == 16 && it.mask_base < 0;  // wave-uniform
    // stage V codes as bf16 (a padding token's codes are finite; its weight is zero)
    {
      uint32_t o[D / 8];
#pragma unroll
      for (int d = 0; d < D / 32; ++d) codes_bf16(st.vc[d], o + 4 * d);
      uint16_t* dst = vst + (lane >> 2) * SV + (lane & 3) * (D / 4);
#pragma unroll
      for (int d = 0; d < D / 32; ++d) *(u32x4*)(dst + 8 * d) = (u32x4){o[4 * d], o[4 * d + 1], o[4 * d + 2], o[4 * d + 3]};
    }
    // S_g^T = K_g Q_g^T
    bf16x8_t kA[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      uint32_t kb[4];
      codes_bf16(st.kc[m >> 1][m & 1], kb);
      kA[m] = __builtin_bit_cast(bf16x8_t, (u32x4){kb[0], kb[1], kb[2], kb[3]});
    }
    f32x4_t sg[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) sg[gg] = s_init[gg];
    if (any_lo) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        sg[m >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[m], __builtin_bit_cast(bf16x8_t, qh[m]), sg[m >> 1], 0, 0, 0);
        sg[m >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[m], __builtin_bit_cast(bf16x8_t, ql[m]), sg[m >> 1], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m)
        sg[m >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[m], __builtin_bit_cast(bf16x8_t, qh[m]), sg[m >> 1], 0, 0, 0);
    }
    // scores of tokens 4 lq + v for row lr
    float sc[4], mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const uint32_t pw = par(st.kp, v, gg);
        const float t = half_bits_to_f32(pw & 0xffffu) * sg[gg][v] + half_bits_to_f32(pw >> 16) * qs[gg];
        x = gg ? x + t : t;
      }
      // lanes of rows past the item's (zero q: finite scores) need no mask; a
      // full tile of an item without a consumer mask needs none at all
      sc[v] = (all_read || (row_reads && 4 * lq + v < valid)) ? x * a.sl2e : -INFINITY;
      mx = fmaxf(mx, sc[v]);
    }
    if (__builtin_amdgcn_ballot_w64(mx > mrow + kSlack) != 0) {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(mrow, mx);
      const float alpha = ex2(mrow - mn);
      mrow = mn;
      lsum *= alpha;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        zacc[gg] *= alpha;
        corr[gg] *= alpha;
      }
#pragma unroll
      for (int n = 0; n < NO; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = ex2(sc[v] - mrow);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    // P' = p s of each group (hi + lo), and sum p z
    s16x4_t pH[NG], pL[NG];
    // a padding token's (s, z) may be NaN: partial tiles (wave-uniform) take zero
    float vs[4][NG], vz[4][NG];
    if (valid == 16) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const uint32_t pw = par(st.vp, v, gg);
          vs[v][gg] = half_bits_to_f32(pw & 0xffffu);
          vz[v][gg] = half_bits_to_f32(pw >> 16);
        }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const uint32_t pw = par(st.vp, v, gg);
          const bool ok = 4 * lq + v < valid;
          vs[v][gg] = ok ? half_bits_to_f32(pw & 0xffffu) : 0.f;
          vz[v][gg] = ok ? half_bits_to_f32(pw >> 16) : 0.f;
        }
    }
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      float pp[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pp[v] = p[v] * vs[v][gg];
        zacc[gg] += p[v] * vz[v][gg];
      }
      const uint32_t h0 = pack_bf16(pp[0], pp[1]), h1 = pack_bf16(pp[2], pp[3]);
      const uint32_t l0 = pack_bf16(pp[0] - bf16_lo(h0), pp[1] - bf16_hi(h0));
      const uint32_t l1 = pack_bf16(pp[2] - bf16_lo(h1), pp[3] - bf16_hi(h1));
      pH[gg] = __builtin_bit_cast(s16x4_t, make_uint2(h0, h1));
      pL[gg] = __builtin_bit_cast(s16x4_t, make_uint2(l0, l1));
    }
    // the staged V must be visible to this wave's reads (LDS is in order per wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += C^T P'^T; the 16 dims of MFMA n lie in group n / (NO / NG)
    const uint16_t* src = vst + (4 * lq + (lr >> 2)) * SV + 4 * (lr & 3);
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const s16x4_t vA = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + 16 * n));
      const int gg = n / (NO / NG);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA, pH[gg], acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA, pL[gg], acc[n], 0, 0, 0);
    }
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      corr[gg] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(c128, pH[gg], corr[gg], 0, 0, 0);
      corr[gg] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(c128, pL[gg], corr[gg], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  Q4Set<D> ss[3];
  Cursor cs[3], lc = first;
  int issued = 0;
  ring3(
      cnt,
      [&](const int S) {
        if (issued > 0) lc = advance(a, it, meta, lc);
        cs[S] = lc;
        load(ss[S], lc);
        ++issued;
      },
      [&](const int S) { tile(ss[S], cs[S]); });
  // row totals over the row's 4 lanes; the zero terms join the accumulators
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    zacc[gg] += __shfl_xor(zacc[gg], 16);
    zacc[gg] += __shfl_xor(zacc[gg], 32);
  }
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] += zacc[n / (NO / NG)] - corr[n / (NO / NG)][0];

  // cross-wave merge: wave w's rows to LDS (acc[n][v] is position 16n + 4 lq + v
  // of row lr: dim 16n + 8(lq/2) + 2v + lq%2, by the code order above)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* mine = &sh.per[w].acc[0][0];
#pragma unroll
  for (int n = 0; n < NO; ++n) *(f32x4_t*)(mine + lr * D + 16 * n + 4 * lq) = acc[n];
  if (lq == 0) {
    sh.ml[w][lr][0] = mrow;
    sh.ml[w][lr][1] = lsum;
  }
  __syncthreads();
  if (w == 0 && lr < rows) {
    float mx = sh.ml[0][lr][0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) mx = fmaxf(mx, sh.ml[v][lr][0]);
    float scw[kWaves], lt = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      scw[v] = ex2(sh.ml[v][lr][0] - mx);
      lt += scw[v] * sh.ml[v][lr][1];
    }
    const int64_t row = (int64_t)g * a.P + it.part_base + lr;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      f32x4_t o = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) o += scw[v] * *(const f32x4_t*)(&sh.per[v].acc[0][0] + lr * D + 16 * n + 4 * lq);
      // lanes lq and lq ^ 1 (same row) hold the even and the odd dims of one
      // 8-dim run: exchange to natural order
      f32x4_t x;
#pragma unroll
      for (int v = 0; v < 4; ++v) x[v] = __shfl_xor(o[v], 16);
      const f32x4_t nat = (lq & 1) ? (f32x4_t){x[2], o[2], x[3], o[3]} : (f32x4_t){o[0], x[0], o[1], x[1]};
      *(f32x4_t*)(a.pacc + row * D + 16 * n + 4 * lq) = nat;
    }
    if (lq == 0) a.pml[row] = make_float2(mx, lt);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path for Q4 items of 2 to 4 rows whose consumers are all
// unshifted (a GQA group of one agent: the common case of private Q4 caches).
// A 16-row result tile would carry only the item's rows, so a wave takes four
// consecutive tiles of its range at once (slots j = 0..3) and gives result
// column 4j + r to (slot j, row r):
//   QK  S_j^T = K_j Q^T per slot (16 tokens x 16 columns, the same unpadded Q
//       operand for every slot; 4 MFMAs each), and each lane keeps the result
//       of its own column's slot;
//   PV  O^T (D x 16 columns) += V^T P'^T over two slots per 16x16x32 MFMA:
//       k-slot 8q + i holds token 4q + i of the first slot (i < 4) or token
//       4q + i - 4 of the second, which are the tokens of the scores a lane
//       holds; a lane's P' operand holds its column's weights in the half of
//       its own slot and zeros elsewhere, so every column sums its own slot.
// Every column keeps its own online-softmax state; at the end of the item the
// 16 states of a row (4 slots x 4 waves) are merged like split-KV partials.
// The code arithmetic is that of run_q4m: bf16 128 + c operands, the groups'
// s and z applied outside the MFMAs, the S chains started at -128 sum(q_g).
// The 128 offset that V's operand adds is removed with the sum of the same
// bf16 P' values (v_dot2 against ones: exact products, float32 sums).
template <int D>
struct Q4PLds {
  static constexpr int kVRow = D / 2;              // bytes of one token's V codes
  static constexpr int kVSlot = 16 * kVRow + 16;   // bytes per staged slot of 16 tokens (padded)
  union Per {
    alignas(16) uint8_t v[4 * kVSlot];  // the wave's four slots' V codes as stored (4 bits each)
    float acc[16][D];                   // the wave's 16 result columns, for the merge
  } per[kWaves];
  float ml[kWaves][16][2];
};

template <int D>
struct Q4PSet {
  static constexpr int NG = D / 64;
  u32x2 kc[4][NG];  // slot j: K codes of token l%16, group g dims 64g + 16(l/16) + [0, 16)
  u32x4 vc[4];      // slot j: V codes of token l/4, dims (D/4)(l%4) + [0, D/4)  (D = 64: .xy)
  u32x4 kp[NG];     // K (s, z) words of the lane's column slot, tokens 4(l/16) + [0, 4)
  u32x4 vp[NG];     // V (s, z) words, the same tokens
  int valid[4];     // valid tokens of each slot's tile (0: slot past the wave's range)
  uint32_t m0[4];   // consumer mask word of each slot's block
  int64_t pc;       // byte offset of the lane's (s, z) words
};

// Runs a wave's steps with two register sets; a step's loads are issued in two
// parts (codes, then the (s, z) words), each one step before its use: the codes
// of step i + 1 before the first phase of step i (V staging and QK), the words
// of step i + 1 before its second phase (softmax and PV).  The steady loop issues
// the same loads on every path, so the compiler's waits keep one step in flight.
// The caller has issued step 0 into set 0 (both parts).
template <class IssueCodes, class IssuePar, class PhaseA, class PhaseB>
__device__ __forceinline__ void ring2_phased(const int n, IssueCodes&& ic, IssuePar&& ip, PhaseA&& pa, PhaseB&& pb) {
  if (n <= 0) return;
  int i = 0;
  while (i + 3 <= n) {
    ic(1);
    pa(0);
    ip(1);
    pb(0);
    ic(0);
    pa(1);
    ip(0);
    pb(1);
    i += 2;
  }
  // set 0 holds step i; one or two steps are left
  if (n - i == 2) {
    ic(1);
    pa(0);
    ip(1);
    pb(0);
    pa(1);
    pb(1);
  } else {
    pa(0);
    pb(0);
  }
}

template <int D>
__device__ __forceinline__ void run_q4p(const TileArgs& a, const kvp_item& it, const int g, Q4PLds<D>& sh) {
  constexpr int NG = D / 64;
  constexpr int NM = D / 32;  // QK MFMAs per slot, two per group
  constexpr int NO = D / 16;  // 16-dim output chunks
  constexpr int kVRow = Q4PLds<D>::kVRow, kVSlot = Q4PLds<D>::kVSlot;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int jc = lr >> 2, r = lr & 3;  // the lane's result column: slot jc, row r
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;
  const int crow = r / group;

  // Set-up in two rounds of memory latency: (1) the lane row's query row and
  // the item's first 64 blocks (ids, token counts, mask words); (2) the query
  // and the first step's K/V loads, issued back to back.
  BlockMeta meta;
  int qa = 0;
  if (r < rows) qa = a.cons_row[it.cons_begin + crow];  // unshifted consumer: its agent
  const int mbi = it.blk_begin + lane;
  meta.base = it.blk_begin;
  meta.p = 0;
  meta.nt = 0;
  meta.m0 = meta.m1 = 0xffffffffu;
  if (mbi < it.blk_end) {
    meta.p = a.plan_blocks[mbi];
    meta.nt = a.plan_ntok[mbi];
    if (it.mask_base >= 0) {
      const uint32_t* mw = a.mask + it.mask_base + (int64_t)(mbi - it.blk_begin) * it.mask_stride;
      meta.m0 = mw[0];
      if (it.mask_stride > 1) meta.m1 = mw[1];
    }
  }
  // Q operand: row r (zero past the item's rows), the dim order of run_q4m
  uint4 qh[NM];
  {
    const uint16_t* qrow = a.q + ((int64_t)qa * a.Hq + g * group + (r - crow * group)) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      qh[m] = make_uint4(0, 0, 0, 0);
      if (r < rows) qh[m] = *(const uint4*)(qrow + 64 * (m >> 1) + 16 * lq + 8 * (m & 1));
    }
  }

  float mrow = kNegBig, lsum = 0.f, zacc[NG], cacc[NG];
  f32x4_t acc[NO];
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) zacc[gg] = cacc[gg] = 0.f;
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)

  const int64_t head_codes = (int64_t)a.B * (D / 2);
  const int64_t head_par = (int64_t)a.B * NG * 4;
  const int kq_lane = lr * (D / 2) + 8 * lq;  // + 32 per group
  const int par_lane = 16 * NG * lq;          // + 16 per group
  const int vq_lane = (lane >> 2) * (D / 2) + (lane & 3) * (D / 8);

  int cnt;
  Cursor lc;
  wave_range_filled(a, it, w, cnt, lc, meta);
  lc = uniform(lc);
  meta.base = __builtin_amdgcn_readfirstlane(meta.base);
  const int nsteps = (cnt + 3) >> 2;
  int issued = 0;
  float qs[NG];         // sum of the row's q over each group
  f32x4_t s_init[NG];   // the S chains start at -128 sum(q_g)
  auto load_codes = [&](Q4PSet<D>& st) {
    int64_t po[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (issued < cnt) {
        if (issued > 0) lc = uniform(advance(a, it, meta, lc));
        ++issued;
        st.valid[j] = min(16, lc.nt - lc.s * 16);
      } else {
        st.valid[j] = 0;  // past the range: the last tile again, fully masked
      }
      st.m0[j] = lc.m0;
      const int64_t hb = (a.layer_blocks + lc.p) * a.Hkv + g;
      const int64_t co = hb * head_codes + (int64_t)lc.s * 16 * (D / 2);
      po[j] = hb * head_par + (int64_t)lc.s * 16 * NG * 4;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) st.kc[j][gg] = ld_nt8(a.kpool + co + kq_lane + 32 * gg);
      if constexpr (D == 128) {
        st.vc[j] = ld_nt16(a.vpool + co + vq_lane);
      } else {
        const u32x2 t = ld_nt8(a.vpool + co + vq_lane);
        st.vc[j] = (u32x4){t.x, t.y, 0u, 0u};
      }
    }
    st.pc = (jc == 0 ? po[0] : jc == 1 ? po[1] : jc == 2 ? po[2] : po[3]) + par_lane;
  };
  auto load_par = [&](Q4PSet<D>& st) {
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      st.kp[gg] = ld_nt16(a.kpar + st.pc + 16 * gg);
      st.vp[gg] = ld_nt16(a.vpar + st.pc + 16 * gg);
    }
  };
  auto par = [](const u32x4* pw, const int v, const int gg) -> uint32_t {
    const int k = v * NG + gg;
    return pw[k >> 2][k & 3];
  };

  uint8_t* vst = &sh.per[w].v[0];
  // the 8-byte run a lane addresses in the transposed 4-bit reads of a slot pair:
  // lane (lq, lr) takes slot 2pr + bit 2 of lr, token 4 lq + lr % 4, dims of chunk
  // 2c + lr / 8; ds_read_b64_tr_b4 gives lane i of a 16-lane group nibble i of
  // every run its group addresses, i.e. dim 16n + i of tokens 4 lq + [0, 4) of
  // both slots, for chunk 2c (low word) and chunk 2c + 1 (high word)
  const int tr_off = ((lr >> 2) & 1) * kVSlot + (4 * lq + (lr & 3)) * kVRow + (lr >> 3) * 8;
  f32x4_t sg[NG];  // scores of the step: tokens 4 lq + v of the lane's column
  auto phase_a = [&](const Q4PSet<D>& st) {
    // the four slots' V codes to LDS as they are stored (token l/4, dims
    // (D/4)(l%4) + [0, D/4) of each slot; converted after the transposed reads)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint8_t* dst = vst + j * kVSlot + (lane >> 2) * kVRow + (lane & 3) * (D / 8);
      if constexpr (D == 128)
        *(u32x4*)dst = st.vc[j];
      else
        *(u32x2*)dst = (u32x2){st.vc[j].x, st.vc[j].y};
    }
    // S^T of every slot; the lane keeps its column's slot
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4_t cj[NG];
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) cj[gg] = s_init[gg];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        uint32_t kb[4];
        codes_bf16(st.kc[j][m >> 1][m & 1], kb);
        const bf16x8_t kA = __builtin_bit_cast(bf16x8_t, (u32x4){kb[0], kb[1], kb[2], kb[3]});
        cj[m >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8_t, qh[m]), cj[m >> 1], 0, 0, 0);
      }
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) sg[gg] = (j == 0 || jc == j) ? cj[gg] : sg[gg];
    }
  };
  auto phase_b = [&](const Q4PSet<D>& st) {
    const int valid = jc == 0 ? st.valid[0] : jc == 1 ? st.valid[1] : jc == 2 ? st.valid[2] : st.valid[3];
    const uint32_t m0 = jc == 0 ? st.m0[0] : jc == 1 ? st.m0[1] : jc == 2 ? st.m0[2] : st.m0[3];
    const bool full = st.valid[0] == 16 && st.valid[1] == 16 && st.valid[2] == 16 && st.valid[3] == 16;  // wave-uniform
    const bool all_read = full && it.mask_base < 0;
    const bool row_reads = r < rows && ((m0 >> crow) & 1u);
    float sc[4], mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const uint32_t pw = par(st.kp, v, gg);
        const float t = half_bits_to_f32(pw & 0xffffu) * sg[gg][v] + half_bits_to_f32(pw >> 16) * qs[gg];
        x = gg ? x + t : t;
      }
      // columns of rows past the item's have zero q (finite scores): a full
      // step of an item without a consumer mask needs no mask at all
      sc[v] = (all_read || (row_reads && 4 * lq + v < valid)) ? x * a.sl2e : -INFINITY;
      mx = fmaxf(mx, sc[v]);
    }
    if (__builtin_amdgcn_ballot_w64(mx > mrow + kSlack) != 0) {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(mrow, mx);
      const float alpha = ex2(mrow - mn);
      mrow = mn;
      lsum *= alpha;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        zacc[gg] *= alpha;
        cacc[gg] *= alpha;
      }
#pragma unroll
      for (int n = 0; n < NO; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = ex2(sc[v] - mrow);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    // P' = p s of each group (bf16 hi + lo), sum p z, and the sum of P' itself
    float vs[4][NG], vz[4][NG];
    if (full) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const uint32_t pw = par(st.vp, v, gg);
          vs[v][gg] = half_bits_to_f32(pw & 0xffffu);
          vz[v][gg] = half_bits_to_f32(pw >> 16);
        }
    } else {
      // a padding token's (s, z) may be NaN
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const uint32_t pw = par(st.vp, v, gg);
          const bool ok = 4 * lq + v < valid;
          vs[v][gg] = ok ? half_bits_to_f32(pw & 0xffffu) : 0.f;
          vz[v][gg] = ok ? half_bits_to_f32(pw >> 16) : 0.f;
        }
    }
    uint32_t ph[NG][2], pl[NG][2];  // the lane's P' (4 tokens) per group, bf16 hi and lo
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      float pp[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pp[v] = p[v] * vs[v][gg];
        zacc[gg] += p[v] * vz[v][gg];
      }
      // pairs (0, 2) and (1, 3): the token order of the V operand (codes_bf16's)
      const uint32_t h0 = pack_bf16(pp[0], pp[2]), h1 = pack_bf16(pp[1], pp[3]);
      const uint32_t l0 = pack_bf16(pp[0] - bf16_lo(h0), pp[2] - bf16_hi(h0));
      const uint32_t l1 = pack_bf16(pp[1] - bf16_lo(h1), pp[3] - bf16_hi(h1));
      cacc[gg] = dot2_bf16(l1, kOnes, dot2_bf16(l0, kOnes, dot2_bf16(h1, kOnes, dot2_bf16(h0, kOnes, cacc[gg]))));
      ph[gg][0] = h0;
      ph[gg][1] = h1;
      pl[gg][0] = l0;
      pl[gg][1] = l1;
    }
    // the staged V must be visible to this wave's reads (LDS is in order per wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P'^T, two slots per MFMA; the 16 dims of chunk n lie in group n / (NO / NG)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      // P' operands of slots 2pr, 2pr + 1 in the V operand's k order (slot a
      // tokens 0 2, slot b 0 2, slot a 1 3, slot b 1 3 of the lane's four): the
      // lane's weights at its own slot's places, zeros at the other's
      u32x4 bH[NG], bL[NG];
      const bool f = jc == 2 * pr, s = jc == 2 * pr + 1;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        bH[gg] = (u32x4){f ? ph[gg][0] : 0u, s ? ph[gg][0] : 0u, f ? ph[gg][1] : 0u, s ? ph[gg][1] : 0u};
        bL[gg] = (u32x4){f ? pl[gg][0] : 0u, s ? pl[gg][0] : 0u, f ? pl[gg][1] : 0u, s ? pl[gg][1] : 0u};
      }
#pragma unroll
      for (int c = 0; c < NO / 2; ++c) {
        // V^T operands of chunks 2c and 2c + 1: lane l holds dim 16n + l%16 of
        // tokens 4(l/16) + [0, 4) of both slots, converted in codes_bf16's order
        const v2i_t r = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_v2i_t*)(vst + 2 * pr * kVSlot + tr_off + 16 * c));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t o[4];
          codes_bf16((uint32_t)(h ? r.y : r.x), o);
          const bf16x8_t vA = __builtin_bit_cast(bf16x8_t, (u32x4){o[0], o[1], o[2], o[3]});
          const int n = 2 * c + h, gg = n / (NO / NG);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, __builtin_bit_cast(bf16x8_t, bH[gg]), acc[n], 0, 0, 0);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, __builtin_bit_cast(bf16x8_t, bL[gg]), acc[n], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  Q4PSet<D> s0, s1;
  if (nsteps > 0) {
    load_codes(s0);
    load_par(s0);
  }
  // the query's sums per group, under the first step's loads
#pragma unroll
  for (int m = 0; m < NM; ++m) qh[m] = perm8_bf16(qh[m]);
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    float t = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 x = qh[2 * gg + h];
      const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) t += bf16_lo(ws[k]) + bf16_hi(ws[k]);
    }
    t += __shfl_xor(t, 16);
    t += __shfl_xor(t, 32);
    qs[gg] = t;
    const float off = -128.f * t;
    s_init[gg] = (f32x4_t){off, off, off, off};
  }
  ring2_phased(
      nsteps, [&](const int S) { S ? load_codes(s1) : load_codes(s0); },
      [&](const int S) { S ? load_par(s1) : load_par(s0); }, [&](const int S) { S ? phase_a(s1) : phase_a(s0); },
      [&](const int S) { S ? phase_b(s1) : phase_b(s0); });
  // column totals over the column's 4 lanes; the zero terms join the accumulators
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    zacc[gg] += __shfl_xor(zacc[gg], 16);
    zacc[gg] += __shfl_xor(zacc[gg], 32);
    cacc[gg] += __shfl_xor(cacc[gg], 16);
    cacc[gg] += __shfl_xor(cacc[gg], 32);
    zacc[gg] -= 128.f * cacc[gg];
  }
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] += zacc[n / (NO / NG)];

  // the wave's columns to LDS (acc[n][v] is position 16n + 4 lq + v of column lr)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* mine = &sh.per[w].acc[0][0];
#pragma unroll
  for (int n = 0; n < NO; ++n) *(f32x4_t*)(mine + lr * D + 16 * n + 4 * lq) = acc[n];
  if (lq == 0) {
    sh.ml[w][lr][0] = mrow;
    sh.ml[w][lr][1] = lsum;
  }
  __syncthreads();
  // wave w merges row w (w < rows): lane c < D/8 takes dims 8c + [0, 8) over the
  // row's 16 columns (4 waves x 4 slots)
  constexpr int CPR = D / 8;
  const int rr = w, c = lane;
  if (rr < rows && c < CPR) {
    float mx = kNegBig;
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sh.ml[v][4 * j + rr][0]);
    float o[8], lt = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float scw = ex2(sh.ml[v][4 * j + rr][0] - mx);
        lt += scw * sh.ml[v][4 * j + rr][1];
        const float* src = &sh.per[v].acc[4 * j + rr][8 * c];
        const f32x4_t x0 = *(const f32x4_t*)src, x1 = *(const f32x4_t*)(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] += scw * x0[e];
          o[4 + e] += scw * x1[e];
        }
      }
    const int64_t row = (int64_t)g * a.P + it.part_base + rr;
    float* dst = a.pacc + row * D + 8 * c;
    *(f32x4_t*)dst = (f32x4_t){o[0], o[1], o[2], o[3]};
    *(f32x4_t*)(dst + 4) = (f32x4_t){o[4], o[5], o[6], o[7]};
    if (c == 0) a.pml[row] = make_float2(mx, lt);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path for bf16 items of 5 to 7 rows (a GQA group of 5-7 heads of
// one agent, or a few agents' smaller groups): the two-tile form of run_mfma.
// A 16-row result tile would carry only the item's R rows, so a wave takes two
// consecutive tiles of its range at once (slots j = 0, 1) and gives result
// column R*j + r to (slot j, row r); columns from 2R on are idle.
//   QK  S_j^T = K_j Q^T per slot against the same Q operand (all 16 columns
//       computed), each lane keeping the result of its own column's slot;
//   PV  O^T += V^T P^T over both slots in one 16x16x32 MFMA per 16 output dims:
//       k-slot 8q + i holds k-slot 4q + i of the first slot's tile (i < 4) or
//       4q + i - 4 of the second's -- the tokens of the scores a lane holds --
//       and a lane's P operand carries its column's weights in its own slot's
//       half and zeros in the other.
// Operand layouts are run_mfma's (K loaded straight into the A operand in
// k-slot order, V's natural rows repacked into V^T's A operand); each column
// keeps its own online-softmax state, and the 8 states of a row (2 slots x 4
// waves) are merged at the end of the item like split-KV partials.
template <int D>
struct MfmaPSet {
  static constexpr int NM = D / 32;
  u32x4 k[2][NM];  // slot j: K in A-operand order
  u32x4 v[2][4];   // slot j: V rows, tokens l/16 + 4u, dims (l%16)(D/16) + [0, D/16)
  int valid[2];    // valid tokens of each slot's tile (0: slot past the wave's range)
  uint32_t m0[2], m1[2];  // consumer mask words of each slot's block
};

template <int D>
__device__ __forceinline__ void run_mfma_p(const TileArgs& a, const kvp_item& it, const int g, MfmaLds<D>& sh) {
  constexpr int NM = D / 32;  // QK MFMAs per slot (k = 32 dims each)
  constexpr int NO = D / 16;  // PV MFMAs (16 output dims each)
  constexpr int NL = 4;       // V loads per lane per tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;  // 5..7
  const int jc = lr / rows, r = lr - jc * rows;  // the lane's column: slot jc (2: idle), row r
  const bool live = jc < 2;
  const int crow = r / group;

  bool any_lo = false;
  for (int c = it.cons_begin; c < it.cons_end; ++c) any_lo |= a.cons[c] >= a.n_unshifted;

  // B operand of S^T: Q^T, lane l: column l%16 (row r), dims 32m + 8*(l/16) + [0, 8)
  uint4 qh[NM], ql[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) qh[m] = ql[m] = make_uint4(0, 0, 0, 0);
  if (live)
#pragma unroll
    for (int m = 0; m < NM / 2; ++m)  // dims 32m + 8*lq and D/2 + 32m + 8*lq: the same rotate-half pairs
      load_q16<D>(a, it.cons_begin + crow, g * group + (r - crow * group), 32 * m + 8 * lq, qh[m], ql[m],
                  qh[m + NM / 2], ql[m + NM / 2]);

  float mrow = kNegBig, lsum = 0.f;
  f32x4_t acc[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  constexpr int64_t kTileBytes = 16 * D * 2;
  const int64_t head_bytes = (int64_t)a.B * D * 2;
  const int64_t k_lane = (int64_t)tile_token(lr) * D * 2 + 8 * lq * 2;  // A-operand layout
  const int64_t v_lane = (int64_t)lq * D * 2 + lr * (D / 16) * 2;          // natural layout

  int cnt;
  Cursor lc;
  BlockMeta meta;
  wave_range(a, it, w, cnt, lc, meta);
  lc = uniform(lc);
  meta.base = __builtin_amdgcn_readfirstlane(meta.base);
  const int nsteps = (cnt + 1) >> 1;
  int issued = 0;
  // K of both slots (advancing the cursor); V of both slots from the offsets saved
  auto load_k = [&](MfmaPSet<D>& st, int64_t (&vo)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (issued < cnt) {
        if (issued > 0) lc = uniform(advance(a, it, meta, lc));
        ++issued;
        st.valid[j] = min(16, lc.nt - lc.s * 16);
      } else {
        st.valid[j] = 0;  // past the range: the last tile again, fully masked
      }
      st.m0[j] = lc.m0;
      st.m1[j] = lc.m1;
      const int64_t off = ((a.layer_blocks + lc.p) * a.Hkv + g) * head_bytes + lc.s * kTileBytes;
      vo[j] = off;
#pragma unroll
      for (int m = 0; m < NM; ++m) st.k[j][m] = ld_nt16(a.kpool + off + k_lane + 64 * m);
    }
  };
  auto load_v = [&](MfmaPSet<D>& st, const int64_t (&vo)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const uint8_t* src = a.vpool + vo[j] + v_lane + (int64_t)u * 4 * D * 2;
        if constexpr (D == 128) {
          st.v[j][u] = ld_nt16(src);
        } else {
          const u32x2 t = ld_nt8(src);
          st.v[j][u] = (u32x4){t.x, t.y, 0u, 0u};
        }
      }
  };
  const int ncons = it.cons_end - it.cons_begin;
  const uint32_t fm0 = ncons >= 32 ? ~0u : ((1u << ncons) - 1u);
  uint32_t ph[2], pl[2];  // the lane's weights (tokens lq + 4u of its slot), bf16 hi and lo
  // scores, online softmax, weights
  auto phase_a = [&](const MfmaPSet<D>& st) {
    f32x4_t s;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4_t sj = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x8_t kA = __builtin_bit_cast(bf16x8_t, st.k[j][m]);
        sj = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8_t, qh[m]), sj, 0, 0, 0);
        if (any_lo) sj = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, __builtin_bit_cast(bf16x8_t, ql[m]), sj, 0, 0, 0);
      }
      s = (j == 0 || jc == j) ? sj : s;
    }
    const int valid = jc == 0 ? st.valid[0] : st.valid[1];
    const uint32_t rmask = jc == 0 ? st.m0[0] : st.m0[1];
    const bool row_reads = live && ((rmask >> crow) & 1u);
    // two full tiles that every row of the item reads need no masking (idle
    // columns have zero q: finite scores that nothing uses)
    const bool plain = st.valid[0] == 16 && st.valid[1] == 16 && (st.m0[0] & st.m0[1] & fm0) == fm0;
    float sc[4], mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sc[u] = (plain || (row_reads && lq + 4 * u < valid)) ? s[u] * a.sl2e : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    if (__builtin_amdgcn_ballot_w64(mx > mrow + kSlack) != 0) {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(mrow, mx);
      const float alpha = ex2(mrow - mn);
      mrow = mn;
      lsum *= alpha;
#pragma unroll
      for (int n = 0; n < NO; ++n) acc[n] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = ex2(sc[u] - mrow);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    ph[0] = pack_bf16(p[0], p[1]);
    ph[1] = pack_bf16(p[2], p[3]);
    pl[0] = pack_bf16(p[0] - bf16_lo(ph[0]), p[1] - bf16_hi(ph[0]));
    pl[1] = pack_bf16(p[2] - bf16_lo(ph[1]), p[3] - bf16_hi(ph[1]));
  };
  // O^T += V^T P^T over both slots
  auto phase_b = [&](const MfmaPSet<D>& st) {
    // padding tokens are zeroed (they may hold NaN)
    u32x4 vz[2][NL];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (st.valid[j] == 16) {
#pragma unroll
        for (int u = 0; u < NL; ++u) vz[j][u] = st.v[j][u];
      } else {
#pragma unroll
        for (int u = 0; u < NL; ++u) vz[j][u] = lq + 4 * u < st.valid[j] ? st.v[j][u] : (u32x4){0u, 0u, 0u, 0u};
      }
    }
    const bool f = jc == 0, s = jc == 1;
    const bf16x8_t bH = __builtin_bit_cast(bf16x8_t, (u32x4){f ? ph[0] : 0u, f ? ph[1] : 0u, s ? ph[0] : 0u, s ? ph[1] : 0u});
    const bf16x8_t bL = __builtin_bit_cast(bf16x8_t, (u32x4){f ? pl[0] : 0u, f ? pl[1] : 0u, s ? pl[0] : 0u, s ? pl[1] : 0u});
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const s16x4_t v0 = v_operand(vz[0], n), v1 = v_operand(vz[1], n);
      const bf16x8_t vA = __builtin_bit_cast(bf16x8_t, (s16x8_t){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, bH, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, bL, acc[n], 0, 0, 0);
    }
  };
  MfmaPSet<D> s0, s1;
  int64_t vo0[2], vo1[2];
  if (nsteps > 0) {
    load_k(s0, vo0);
    load_v(s0, vo0);
  }
  // K of step i+1 before the scores of step i, V of step i+1 before its P.V
  ring2_phased(
      nsteps, [&](const int S) { S ? load_k(s1, vo1) : load_k(s0, vo0); },
      [&](const int S) { S ? load_v(s1, vo1) : load_v(s0, vo0); }, [&](const int S) { S ? phase_a(s1) : phase_a(s0); },
      [&](const int S) { S ? phase_b(s1) : phase_b(s0); });
  // column totals: the 4 lanes of a column hold disjoint token subsets
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // the wave's columns to LDS, row-major by column
  store_rows<D>(&sh.per[w].acc[lr][0], lq, acc);
  if (lq == 0) {
    sh.ml[w][lr][0] = mrow;
    sh.ml[w][lr][1] = lsum;
  }
  __syncthreads();
  // wave w merges rows w and w + 4 (< rows): lane l takes dims 2l, 2l + 1 (D = 128)
  // or dim l (D = 64) over the row's 8 columns (2 slots x 4 waves)
  constexpr int EPL = D / 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = w + 4 * h;
    if (rr >= rows) break;
    float mx = kNegBig;
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
#pragma unroll
      for (int j = 0; j < 2; ++j) mx = fmaxf(mx, sh.ml[v][rows * j + rr][0]);
    float o[EPL], lt = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float scw = ex2(sh.ml[v][rows * j + rr][0] - mx);
        lt += scw * sh.ml[v][rows * j + rr][1];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] += scw * sh.per[v].acc[rows * j + rr][EPL * lane + e];
      }
    const int64_t row = (int64_t)g * a.P + it.part_base + rr;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a.pacc[row * D + EPL * lane + e] = o[e];
    if (lane == 0) a.pml[row] = make_float2(mx, lt);
  }
}

#ifdef KVP_DEVICE_CHECKS
// The checked build's test of a work item, by the whole workgroup before it
// reads anything through the item: its block, consumer, partial-row and mask
// ranges against the plan's extents (and the row limits of the paths), every
// physical id and valid token count of its blocks, and every consumer's entry
// (query pair in range, agent in range, shifted pairs last, query row as the
// plan derives it).  False (and the bits in g_dev_err) when anything is out.
__device__ bool item_in_bounds(const TileArgs& a, const kvp_item& it, const bool q4) {
  __shared__ uint32_t s_bad;
  const int nb = it.blk_end - it.blk_begin, nc = it.cons_end - it.cons_begin;
  const int group = a.Hq / a.Hkv;
  const bool wide_ok = !q4 && a.B == 16;
  uint32_t bad = 0;
  if (it.blk_begin < 0 || nb < 1 || it.blk_end > a.n_plan_blocks || it.cons_begin < 0 || nc < 1 ||
      it.cons_end > a.n_cons || it.rows != nc * group || it.rows > (wide_ok ? kMaxRowsWide : kMaxRowsValu) ||
      (it.rows > kMaxRowsValu && (nc > kMaxConsWide || nb > kMaxBlocksWide)) || it.part_base < 0 ||
      it.part_base > a.P - it.rows ||
      (it.mask_base != -1 && (it.mask_base < 0 || it.mask_stride != (nc + 31) / 32 ||
                              (int64_t)it.mask_base + (int64_t)nb * it.mask_stride > a.n_mask_words)))
    bad = 1u;
  if (!bad) {
    for (int i = it.blk_begin + (int)threadIdx.x; i < it.blk_end; i += (int)blockDim.x) {
      const int p = a.plan_blocks[i], nt = a.plan_ntok[i];
      if (p < 0 || p >= a.n_phys || nt < 0 || nt > a.B) bad |= 2u;
    }
    for (int c = it.cons_begin + (int)threadIdx.x; c < it.cons_end; c += (int)blockDim.x) {
      const int qc = a.cons[c];
      if (qc < 0 || qc >= a.n_qcons) {
        bad |= 4u;
        continue;
      }
      const int j = a.qcons[2 * qc], shift = a.qcons[2 * qc + 1], row = a.cons_row[c];
      const bool shifted = qc >= a.n_unshifted;
      if (j < 0 || j >= a.n_agents || (shift != 0) != shifted || row != (shifted ? qc - a.n_unshifted : j))
        bad |= 4u;
    }
  }
  if (threadIdx.x == 0) s_bad = 0u;
  __syncthreads();
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  bad = s_bad;
  if (bad && threadIdx.x == 0) atomicOr(&g_dev_err, bad);
  return bad == 0u;
}
#endif

// One launch for every item: each workgroup dispatches on its item's row count.
// bf16 items with more than 4 rows and Q4 items with more than 1 take a
// matrix-core path.
template <int D, int RMAX, bool Q4>
__global__ __launch_bounds__(256, 2) void tile_kernel(const TileArgs a) {
  int ii, g;
  if (!unit_of(a.n_items, a.Hkv, a.xcd_span, ii, g)) return;
  const kvp_item it = a.items[ii];
#ifdef KVP_DEVICE_CHECKS
  if (!item_in_bounds(a, it, Q4)) return;
#endif
  const int rows = it.rows;
  // one LDS region, laid out per path (a workgroup takes exactly one path)
  // (the wide path's ring only in the launches that have wide items)
  struct NoLds {};
  __shared__ union Lds {
    MergeLds<D> merge;
    MfmaLds<D> mfma;
    std::conditional_t<!Q4 && RMAX >= 128, WideLds<D>, NoLds> wide;
    Q4Lds<D> q4;
    std::conditional_t<Q4 && RMAX >= 2, Q4PLds<D>, NoLds> q4p;
  } lds;
  MergeLds<D>& sh = lds.merge;
  if constexpr (!Q4 && RMAX >= 128) {
    // (the planner makes wide items for 16-token blocks only)
    if (rows > 64) {
      run_wide<D, 2>(a, it, g, lds.wide);
      return;
    }
    if (rows > 16) {
      run_wide<D, 1>(a, it, g, lds.wide);
      return;
    }
  }
  if constexpr (!Q4 && RMAX >= 8) {
    // (8 rows fill the 16 columns of two slots too, but such items -- an MHA
    // round's prefix read by 8 agents -- are bound by HBM, and the one-tile path
    // with its deeper prefetch measured faster there)
    if (rows > 7) {
      run_mfma<D>(a, it, g, lds.mfma);
      return;
    }
    if (rows > 4) {
      run_mfma_p<D>(a, it, g, lds.mfma);
      return;
    }
  }
  if constexpr (Q4 && RMAX >= 2) {
    if (rows > 1) {
      bool shifted = false;
      for (int c = it.cons_begin; c < it.cons_end; ++c) shifted |= a.cons[c] >= a.n_unshifted;
      if (rows <= 4 && !shifted)
        run_q4p<D>(a, it, g, lds.q4p);
      else
        run_q4m<D>(a, it, g, lds.q4);
      return;
    }
  }
  if constexpr (!Q4 && RMAX >= 4) {
    if (rows > 2) {
      run_bf16<D, 4>(a, it, g, sh);
      return;
    }
  }
  if constexpr (!Q4 && RMAX >= 2) {
    if (rows > 1) {
      run_bf16<D, 2>(a, it, g, sh);
      return;
    }
  }
  if constexpr (Q4) run_q4<D, 1>(a, it, g, sh); else run_bf16<D, 1>(a, it, g, sh);
}

// ---------------------------------------------------------------------------
// 2. combine

// One wave per (agent, q head).  Its partials are the entries comb_ptr[j] ..
// comb_ptr[j+1] of comb_rows, taken 64 at a time: lane e loads entry e's row
// index and (max, sum), and the loads of the accumulators are issued as soon as
// the row indices are known, so a merge costs three dependent rounds of loads
// (the CSR bounds, the row indices, then the partials).  The log-sum-exp merge
// (MemDecay blog sec. 4.2: float32 softmax) rescales the running sums when a
// later chunk raises the maximum; entries are added in comb_rows order.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ pacc, const float2* __restrict__ pml,
                                                     const int32_t* __restrict__ comb_ptr,
                                                     const int32_t* __restrict__ comb_rows, int Hq, int Hkv, int P,
                                                     int n_comb, float* __restrict__ out) {
  constexpr int E = D / 64;  // dims per lane
  constexpr int U = 16;      // accumulator loads in flight per lane
  typedef float vecE __attribute__((ext_vector_type(E)));
  const int j = blockIdx.x / Hq, h = blockIdx.x - j * Hq;
  const int group = Hq / Hkv, g = h / group, hh = h - g * group;
  const int e0 = comb_ptr[j], e1 = comb_ptr[j + 1];
  const int64_t base = (int64_t)g * P + hh;
  const int lane = threadIdx.x;
#ifdef KVP_DEVICE_CHECKS
  {
    // the checked build: the agent's entries and their partial rows in range
    bool bad = e0 < 0 || e1 < e0 || e1 > n_comb;
    if (!bad)
      for (int e = e0 + lane; e < e1; e += 64) {
        const int r = comb_rows[e];
        bad |= r < 0 || r > P - group;
      }
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      if (lane == 0) atomicOr(&g_dev_err, 8u);
      return;
    }
  }
#endif
  const float* col = pacc + lane * E;
  float M = -INFINITY, L = 0.f;
  vecE o = {};
  for (int c0 = e0; c0 < e1; c0 += 64) {
    const int n = min(64, e1 - c0);
    // lanes past the chunk repeat its last entry (every load stays in bounds
    // and no load waits behind a branch); they weigh 0
    const int row = comb_rows[c0 + min(lane, n - 1)];
    const float2 ml = pml[base + row];
    vecE v[U];
    auto load = [&](int s0) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = *(const vecE*)(col + (base + __builtin_amdgcn_readlane(row, min(s0 + u, n - 1))) * D);
    };
    load(0);  // in flight while the maximum and the weights are formed
    __builtin_amdgcn_sched_barrier(0);
    float cm = lane < n ? ml.x : -INFINITY;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float Mn = fmaxf(M, cm);
    const float sc = ex2(M - Mn);  // M = -inf on the first chunk: 0, and o, L are 0
    o *= sc;
    L *= sc;
    M = Mn;
    const float w = lane < n ? ex2(ml.x - M) : 0.f;  // lane e: entry e's weight
    float t = w * ml.y;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
    L += t;
    int s0 = 0;  // (n >= 1: the first sub-chunk is always used)
    do {
      if (s0 > 0) load(s0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(s0 + u, 63)));
        o += (s0 + u < n ? wu : 0.f) * v[u];
      }
      s0 += U;
    } while (s0 < n);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *(vecE*)(out + ((int64_t)j * Hq + h) * D + lane * E) = o * inv;
}

// ---------------------------------------------------------------------------
// host side

struct WsLayout {
  size_t pacc, pml, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const kvp_shape* sh, const kvp_plan_dev* pl) {
  WsLayout w{};
  w.pacc = 0;
  w.pml = w.pacc + align256((size_t)sh->n_kv_heads * pl->n_part_rows * sh->head_dim * 4);
  w.total = w.pml + align256((size_t)sh->n_kv_heads * pl->n_part_rows * 8);
  return w;
}

int check_plan(const kvp_plan_dev* pl) {
  if (!pl) return fail(KVP_EINVAL, "plan is NULL");
  if (pl->n_agents < 0 || pl->n_phys < 0 || pl->n_items < 0 || pl->n_qcons < 0 || pl->n_part_rows < 0 ||
      pl->n_qcons_shifted < 0 || pl->n_qcons_shifted > pl->n_qcons || pl->unit_span < 1 || pl->unit_span > 4096 ||
      pl->n_plan_blocks < 0 || pl->n_cons < 0 || pl->n_mask_words < 0 || pl->n_comb < 0)
    return fail(KVP_EINVAL, "bad plan counts");
  int sum = 0;
  for (int i = 0; i < kRowClasses; ++i) {
    if (pl->class_items[i] < 0) return fail(KVP_EINVAL, "negative class count");
    sum += pl->class_items[i];
  }
  if (sum != pl->n_items) return fail(KVP_EINVAL, "class counts do not add up to n_items");
  if (pl->n_items > 0 &&
      (!pl->items || !pl->plan_blocks || !pl->cons || !pl->qcons || !pl->phys_ntok || !pl->plan_ntok || !pl->cons_row))
    return fail(KVP_EINVAL, "plan pointer is NULL");
  if (pl->n_agents > 0 && (!pl->comb_ptr || !pl->comb_rows)) return fail(KVP_EINVAL, "plan combine pointer is NULL");
  if (pl->n_items > 0 && pl->n_qcons_shifted > 0 && !pl->rope_cs)
    return fail(KVP_EINVAL, "plan rope_cs is NULL with shifted consumers");
  return KVP_OK;
}

template <int D, int RMAX>
void launch_tiles(const TileArgs& a, bool q4, hipStream_t st) {
  const int total = a.n_items * a.Hkv;
  const int win = (a.Hkv & 7) == 0 ? 8 : 8 * a.xcd_span;
  const int grid = win * ((total + win - 1) / win);
  if (q4)
    hipLaunchKernelGGL((tile_kernel<D, RMAX, true>), dim3(grid), dim3(64 * kWaves), 0, st, a);
  else
    hipLaunchKernelGGL((tile_kernel<D, RMAX, false>), dim3(grid), dim3(64 * kWaves), 0, st, a);
}

// rmax_class: index of the largest row class present (0: wide ... 5: 1 row)
template <int D>
void launch_all(int rmax_class, const TileArgs& a, bool q4, hipStream_t st) {
  switch (rmax_class) {
    case 0: launch_tiles<D, 128>(a, q4, st); break;
    case 1: launch_tiles<D, 16>(a, q4, st); break;
    case 2: launch_tiles<D, 8>(a, q4, st); break;
    case 3: launch_tiles<D, 4>(a, q4, st); break;
    case 4: launch_tiles<D, 2>(a, q4, st); break;
    default: launch_tiles<D, 1>(a, q4, st); break;
  }
}

}  // namespace

// Workspace of paged_decode_attn_noalloc: the partials of one call, for callers
// that cannot allocate device memory.  Every device the library runs on holds
// its own copy from the first use of this code object until the process ends.
static __device__ __align__(256) uint8_t scratch[KVP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.  In host code
// the array's name is only a stand-in for the symbol, never an address.
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(KVP_EINVAL, "device index out of range for the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
    if (!p) return fail(KVP_EHIP, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVP_OK;
}
}  // namespace

extern "C" int paged_decode_attn_workspace_bytes(const kvp_shape* shape, const kvp_plan_dev* plan, size_t* bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  rc = check_plan(plan);
  if (rc) return rc;
  if (!bytes) return fail(KVP_EINVAL, "bytes is NULL");
  *bytes = ws_layout(shape, plan).total;
  return KVP_OK;
}

static int decode_phases(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q, const void* k_pool,
                         const void* v_pool, const void* k_params, const void* v_params, int32_t layer, float scale,
                         float* out, void* workspace, size_t ws_bytes, uint32_t phases, void* stream) {
  if (phases < 1 || phases > 7) return fail(KVP_EINVAL, "phases must be in 1..7");
  int rc = check_shape(shape);
  if (rc) return rc;
  rc = check_plan(plan);
  if (rc) return rc;
  const bool q4 = shape->kv_dtype == KVP_Q4G64;
  if (layer < 0 || layer >= shape->n_layers) return fail(KVP_EINVAL, "layer out of range");
  if (!std::isfinite(scale)) return fail(KVP_EINVAL, "scale");
  if ((int64_t)plan->n_items * shape->n_kv_heads + 16LL * shape->n_kv_heads > 0x7fffffffLL)
    return fail(KVP_EINVAL, "too many work items");
  const WsLayout w = ws_layout(shape, plan);
  if (ws_bytes < w.total) return fail(KVP_EWORKSPACE, "workspace too small");
  // only the pointers the call reads or writes must be set: none without agents,
  // no pool without work items (every agent is empty), no workspace of size 0
  if (plan->n_agents == 0) return KVP_OK;
  if (!q || !out) return fail(KVP_EINVAL, "null device pointer (q or out)");
  if (plan->n_items > 0 && (!k_pool || !v_pool)) return fail(KVP_EINVAL, "null device pointer (pool)");
  if (plan->n_items > 0 && q4 && (!k_params || !v_params))
    return fail(KVP_EINVAL, "Q4 pools need k_params and v_params");
  if (w.total > 0 && !workspace) return fail(KVP_EINVAL, "null device pointer (workspace)");
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  const int D = shape->head_dim;
  const int n_unshifted = plan->n_qcons - plan->n_qcons_shifted;

  TileArgs a{};
  a.items = plan->items;
  a.plan_blocks = plan->plan_blocks;
  a.cons = plan->cons;
  a.qcons = plan->qcons;
  a.mask = plan->mask;
  a.phys_ntok = plan->phys_ntok;
  a.plan_ntok = plan->plan_ntok;
  a.cons_row = plan->cons_row;
  a.q = (const uint16_t*)q;
  a.rope_cs = plan->rope_cs;
  a.n_unshifted = n_unshifted;
  a.kpool = (const uint8_t*)k_pool;
  a.vpool = (const uint8_t*)v_pool;
  a.kpar = (const uint8_t*)k_params;
  a.vpar = (const uint8_t*)v_params;
  a.layer_blocks = (int64_t)layer * plan->n_phys;
  a.Hq = shape->n_q_heads;
  a.Hkv = shape->n_kv_heads;
  a.B = shape->block_tokens;
  a.sl2e = scale * kLog2e;
  a.pacc = (float*)(ws + w.pacc);
  a.pml = (float2*)(ws + w.pml);
  a.P = plan->n_part_rows;
  a.n_items = plan->n_items;
  a.xcd_span = plan->unit_span;
  a.n_agents = plan->n_agents;
  a.n_phys = plan->n_phys;
  a.n_plan_blocks = plan->n_plan_blocks;
  a.n_cons = plan->n_cons;
  a.n_qcons = plan->n_qcons;
  a.n_mask_words = plan->n_mask_words;
  int rmax_class = kRowClasses - 1;
  for (int cls = 0; cls < kRowClasses; ++cls)
    if (plan->class_items[cls] > 0) {
      rmax_class = cls;
      break;
    }
  if ((phases & 2u) && plan->n_items > 0) {
    if (D == 128)
      launch_all<128>(rmax_class, a, q4, st);
    else
      launch_all<64>(rmax_class, a, q4, st);
  }
  const int nw = plan->n_agents * shape->n_q_heads;
  if (phases & 4u) {
    if (D == 128)
      hipLaunchKernelGGL(combine_kernel<128>, dim3(nw), dim3(64), 0, st, a.pacc, (const float2*)a.pml,
                         plan->comb_ptr, plan->comb_rows, shape->n_q_heads, shape->n_kv_heads, plan->n_part_rows,
                         plan->n_comb, out);
    else
      hipLaunchKernelGGL(combine_kernel<64>, dim3(nw), dim3(64), 0, st, a.pacc, (const float2*)a.pml,
                         plan->comb_ptr, plan->comb_rows, shape->n_q_heads, shape->n_kv_heads, plan->n_part_rows,
                         plan->n_comb, out);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
  return KVP_OK;
}

extern "C" int paged_decode_attn(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q, const void* k_pool,
                                 const void* v_pool, const void* k_params, const void* v_params, int32_t layer,
                                 float scale, float* out, void* workspace, size_t ws_bytes, void* stream) {
  return decode_phases(shape, plan, q, k_pool, v_pool, k_params, v_params, layer, scale, out, workspace, ws_bytes, 7u,
                       stream);
}

extern "C" int paged_decode_attn_phases(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q,
                                        const void* k_pool, const void* v_pool, const void* k_params,
                                        const void* v_params, int32_t layer, float scale, float* out, void* workspace,
                                        size_t ws_bytes, uint32_t phases, void* stream) {
  return decode_phases(shape, plan, q, k_pool, v_pool, k_params, v_params, layer, scale, out, workspace, ws_bytes,
                       phases, stream);
}

extern "C" int paged_decode_attn_noalloc(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q,
                                         const void* k_pool, const void* v_pool, const void* k_params,
                                         const void* v_params, int32_t layer, float scale, float* out, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  rc = check_plan(plan);
  if (rc) return rc;
  const size_t need = ws_layout(shape, plan).total;
  if (need > (size_t)KVP_NOALLOC_SCRATCH_BYTES) {
    char msg[160];
    snprintf(msg, sizeof msg, "the plan needs %zu bytes of workspace; paged_decode_attn_noalloc holds at most %zu",
             need, (size_t)KVP_NOALLOC_SCRATCH_BYTES);
    return fail(KVP_EWORKSPACE, msg);
  }
  void* ws = nullptr;
  if (plan->n_agents > 0 && need > 0) {
    rc = scratch_ptr(&ws);
    if (rc) return rc;
  }
  return decode_phases(shape, plan, q, k_pool, v_pool, k_params, v_params, layer, scale, out, ws,
                       ws ? (size_t)KVP_NOALLOC_SCRATCH_BYTES : 0, 7u, stream);
}

extern "C" int kvpool_device_checks_enabled(void) {
#ifdef KVP_DEVICE_CHECKS
  return 1;
#else
  return 0;
#endif
}

namespace {
__global__ void take_err_kernel(uint32_t* dst) {
  if (threadIdx.x == 0) *dst = atomicExch(&g_dev_err, 0u);
}
}  // namespace

extern "C" int kvpool_debug_take_device_errors(uint32_t* dst, void* stream) {
  if (!dst) return fail(KVP_EINVAL, "dst is NULL");
  hipLaunchKernelGGL(take_err_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
  return KVP_OK;
}
