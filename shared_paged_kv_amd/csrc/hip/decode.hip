// paged_decode_attn on gfx950: one decode step of attention for many agents
// over a deduplicated, paged KV pool.
//
// Three kernels per call, all on the caller's stream:
//   1. qprep   -- every distinct (agent, shift) consumer's query, moved by
//                 R(-shift) so that (R(-s) q) . k == q . (R(s) k) (INMS
//                 walkthrough sec. 3.2: the compensation depends on the position
//                 difference only), split into a bf16 hi + lo pair.
//   2. tile    -- one wave per (work item, kv head): streams the item's physical
//                 blocks from HBM once with 16-byte loads straight into
//                 registers, and every query row the item carries (all agents
//                 and GQA heads that read those blocks) is scored against the
//                 same registers: the block is fetched once for all of them.
//                 Online softmax per row (MemDecay blog sec. 4.2: scaled dot
//                 product, float32 softmax); delta blocks are ordinary blocks of
//                 their owner, and the owner is masked out of the master block
//                 (TokenDance write-up sec. 3, the correction fused into the
//                 load); Q4 blocks are dequantised in registers (Q4 KV paper
//                 summary sec. 2.2).  Writes a partial (max, sum, acc) per row.
//   3. combine -- log-sum-exp merge of each (agent, q head)'s partials in a
//                 fixed order.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../host/kvpool_internal.h"
#include "device_common.h"
#include "kvpool.h"

namespace {
using namespace kvp;

constexpr float kNegBig = -1e30f;  // finite "no score yet" (keeps exp2 arguments finite)
constexpr float kLog2e = 1.4426950408889634f;

struct TileArgs {
  const kvp_item* items;
  const int32_t* plan_blocks;
  const int32_t* cons;
  const int32_t* qcons;
  const uint32_t* mask;
  const int32_t* phys_ntok;
  const uint16_t* qhi;  // [n_qcons][Hq][D] bf16
  const uint16_t* qlo;
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
  int item0, n_items;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 1. query preparation

__global__ __launch_bounds__(256) void qprep_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ qcons,
                                                    int n_qcons, int Hq, int D, float base,
                                                    uint16_t* __restrict__ qhi, uint16_t* __restrict__ qlo) {
  const int half = D / 2;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_qcons * half) return;
  const int qc = t / half, i = t % half;
  const int j = qcons[2 * qc], delta = qcons[2 * qc + 1];
  float c, s;
  rope_cs(-delta, i, D, base, &c, &s);
  for (int h = 0; h < Hq; ++h) {
    const uint16_t* src = q + ((int64_t)j * Hq + h) * D;
    float y1, y2;
    rope_apply(bf16_to_f32(src[i]), bf16_to_f32(src[i + half]), c, s, &y1, &y2);
    const uint16_t h1 = f32_to_bf16_rne(y1), h2 = f32_to_bf16_rne(y2);
    const int64_t o = ((int64_t)qc * Hq + h) * D;
    qhi[o + i] = h1;
    qhi[o + i + half] = h2;
    qlo[o + i] = f32_to_bf16_rne(y1 - bf16_to_f32(h1));
    qlo[o + i + half] = f32_to_bf16_rne(y2 - bf16_to_f32(h2));
  }
}

// ---------------------------------------------------------------------------
// 2. tile pass

// XCD-aware item mapping: workgroups are dealt round-robin over the 8 XCDs, so
// workgroup b runs on XCD b % 8.  Map it to logical unit (b % 8) * per + b / 8:
// consecutive logical units (the same kv head, neighbouring items) share an XCD
// and its L2.  The grid is padded to 8 * per; units past the end exit.
__device__ __forceinline__ int xcd_logical(int total) {
  const int per = (total + 7) >> 3;
  return (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
}

template <int D, int R>
__global__ __launch_bounds__(64) void tile_bf16_kernel(const TileArgs a) {
  constexpr int LPT = D / 8;     // lanes per token row (8 bf16 = 16 bytes each)
  constexpr int TPL = 64 / LPT;  // tokens per wave-wide load
  constexpr int NL = 16 / TPL;   // loads per lane per 16-token tile
  const int lane = threadIdx.x;
  const int dsl = (lane % LPT) * 8;
  const int tg = lane / LPT;

  const int total = a.n_items * a.Hkv;
  const int logical = xcd_logical(total);
  if (logical >= total) return;
  const int g = logical / a.n_items;
  const kvp_item it = a.items[a.item0 + logical % a.n_items];
  const int group = a.Hq / a.Hkv;
  const int rows = it.rows;

  bool any_lo = false;
  for (int c = it.cons_begin; c < it.cons_end; ++c) any_lo |= a.qcons[2 * a.cons[c] + 1] != 0;

  uint4 qh[R], ql[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    qh[r] = make_uint4(0, 0, 0, 0);
    ql[r] = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      const int c = r / group;
      const int hq = g * group + (r - c * group);
      const int qc = a.cons[it.cons_begin + c];
      const int64_t o = ((int64_t)qc * a.Hq + hq) * D + dsl;
      qh[r] = *(const uint4*)(a.qhi + o);
      if (any_lo) ql[r] = *(const uint4*)(a.qlo + o);
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
  auto tile_base = [&](int p, int s) -> int64_t {
    return ((a.layer_blocks + p) * a.Hkv + g) * head_bytes + s * kTileBytes + lane_off;
  };
  uint4 kc[NL], vc[NL], kn[NL], vn[NL];
  auto load = [&](uint4* kk, uint4* vv, int64_t off) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      kk[k] = *(const uint4*)(a.kpool + off + (int64_t)k * TPL * D * 2);
      vv[k] = *(const uint4*)(a.vpool + off + (int64_t)k * TPL * D * 2);
    }
  };

  int bi = it.blk_begin, s = 0;
  int p = a.plan_blocks[bi];
  int nt = a.phys_ntok[p];
  load(kc, vc, tile_base(p, 0));
  while (true) {
    int s2 = s + 1, bi2 = bi, p2 = p, nt2 = nt;
    if (s2 * 16 >= nt) {
      bi2 = bi + 1;
      s2 = 0;
      if (bi2 < it.blk_end) {
        p2 = a.plan_blocks[bi2];
        nt2 = a.phys_ntok[p2];
      }
    }
    const bool more = bi2 < it.blk_end;
    if (more) load(kn, vn, tile_base(p2, s2));

    const uint32_t rmask = it.mask_base < 0 ? 0xffffffffu : a.mask[it.mask_base + (bi - it.blk_begin) * it.mask_stride];
    const int valid = min(16, nt - s * 16);
    const bool partial = valid < 16;
    float vf[NL][8];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const uint32_t w[4] = {vc[k].x, vc[k].y, vc[k].z, vc[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[k][2 * i] = bf16_lo(w[i]);
        vf[k][2 * i + 1] = bf16_hi(w[i]);
      }
      if (partial && k * TPL + tg >= valid) {
#pragma unroll
        for (int i = 0; i < 8; ++i) vf[k][i] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rows && ((rmask >> (r / group)) & 1u)) {
        float sc[NL];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          float d = 0.f;
          d = dot2_bf16(qh[r].x, kc[k].x, d);
          d = dot2_bf16(qh[r].y, kc[k].y, d);
          d = dot2_bf16(qh[r].z, kc[k].z, d);
          d = dot2_bf16(qh[r].w, kc[k].w, d);
          if (any_lo) {
            d = dot2_bf16(ql[r].x, kc[k].x, d);
            d = dot2_bf16(ql[r].y, kc[k].y, d);
            d = dot2_bf16(ql[r].z, kc[k].z, d);
            d = dot2_bf16(ql[r].w, kc[k].w, d);
          }
          d = group_sum<LPT>(d);
          sc[k] = (partial && k * TPL + tg >= valid) ? -INFINITY : d * a.sl2e;
        }
        float mx = sc[0];
#pragma unroll
        for (int k = 1; k < NL; ++k) mx = fmaxf(mx, sc[k]);
        const float mn = fmaxf(m[r], mx);
        const float alpha = ex2(m[r] - mn);
        m[r] = mn;
        l[r] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r][i] *= alpha;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          const float pk = ex2(sc[k] - mn);
          l[r] += pk;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[r][i] += pk * vf[k][i];
        }
      }
    }
    if (!more) break;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      kc[k] = kn[k];
      vc[k] = vn[k];
    }
    bi = bi2;
    s = s2;
    p = p2;
    nt = nt2;
  }

  // merge the token groups of the wave and write one partial per row
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
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[i] = acc[r][i] * sc;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) o[i] += __shfl_xor(o[i], off);
      }
      const int64_t row = (int64_t)g * a.P + it.part_base + r;
      if (tg == 0) {
        float4* dst = (float4*)(a.pacc + row * D + dsl);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
      if (lane == 0) a.pml[row] = make_float2(M, lr);
    }
  }
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int D, int R>
__global__ __launch_bounds__(64) void tile_q4_kernel(const TileArgs a) {
  constexpr int LPT = D / 16;    // lanes per token row (16 codes = 8 bytes each)
  constexpr int TPL = 64 / LPT;  // tokens per wave-wide load
  constexpr int NL = 16 / TPL;   // loads per lane per 16-token tile
  constexpr int NG = D / 64;     // quantisation groups per row
  const int lane = threadIdx.x;
  const int dq = (lane % LPT) * 16;
  const int grp = dq / 64;
  const int tg = lane / LPT;

  const int total = a.n_items * a.Hkv;
  const int logical = xcd_logical(total);
  if (logical >= total) return;
  const int g = logical / a.n_items;
  const kvp_item it = a.items[a.item0 + logical % a.n_items];
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
      const int qc = a.cons[it.cons_begin + c];
      const int64_t o = ((int64_t)qc * a.Hq + hq) * D + dq;
      const uint4 h0 = *(const uint4*)(a.qhi + o), h1 = *(const uint4*)(a.qhi + o + 8);
      const uint4 l0 = *(const uint4*)(a.qlo + o), l1 = *(const uint4*)(a.qlo + o + 8);
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
  uint2 kc[NL], vc[NL], kn[NL], vn[NL];
  uint32_t kp[NL], vp[NL], kpn[NL], vpn[NL];
  auto load = [&](uint2* kk, uint2* vv, uint32_t* kq, uint32_t* vq, int p, int s) {
    const int64_t hb = (a.layer_blocks + p) * a.Hkv + g;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int tk = s * 16 + k * TPL + tg;
      const int64_t co = hb * head_codes + tk * kRowBytes + dq / 2;
      const int64_t po = hb * head_par + tk * kParBytes + grp * 4;
      kk[k] = *(const uint2*)(a.kpool + co);
      vv[k] = *(const uint2*)(a.vpool + co);
      kq[k] = *(const uint32_t*)(a.kpar + po);
      vq[k] = *(const uint32_t*)(a.vpar + po);
    }
  };

  int bi = it.blk_begin, s = 0;
  int p = a.plan_blocks[bi];
  int nt = a.phys_ntok[p];
  load(kc, vc, kp, vp, p, 0);
  while (true) {
    int s2 = s + 1, bi2 = bi, p2 = p, nt2 = nt;
    if (s2 * 16 >= nt) {
      bi2 = bi + 1;
      s2 = 0;
      if (bi2 < it.blk_end) {
        p2 = a.plan_blocks[bi2];
        nt2 = a.phys_ntok[p2];
      }
    }
    const bool more = bi2 < it.blk_end;
    if (more) load(kn, vn, kpn, vpn, p2, s2);

    const uint32_t rmask = it.mask_base < 0 ? 0xffffffffu : a.mask[it.mask_base + (bi - it.blk_begin) * it.mask_stride];
    const int valid = min(16, nt - s * 16);
    float ck[NL][16], cv[NL][16], sk[NL], zk[NL], sv[NL], zv[NL];
    bool ok[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      ok[k] = k * TPL + tg < valid;
      const uint32_t kw[2] = {kc[k].x, kc[k].y}, vw[2] = {vc[k].x, vc[k].y};
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t klo = kw[w] & 0x0f0f0f0fu, khi = (kw[w] >> 4) & 0x0f0f0f0fu;
        const uint32_t vlo = vw[w] & 0x0f0f0f0fu, vhi = (vw[w] >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          ck[k][8 * w + 2 * b] = (float)((klo >> (8 * b)) & 0xffu);
          ck[k][8 * w + 2 * b + 1] = (float)((khi >> (8 * b)) & 0xffu);
          cv[k][8 * w + 2 * b] = (float)((vlo >> (8 * b)) & 0xffu);
          cv[k][8 * w + 2 * b + 1] = (float)((vhi >> (8 * b)) & 0xffu);
        }
      }
      sk[k] = half_bits_to_f32(kp[k] & 0xffffu);
      zk[k] = half_bits_to_f32(kp[k] >> 16);
      sv[k] = ok[k] ? half_bits_to_f32(vp[k] & 0xffffu) : 0.f;
      zv[k] = ok[k] ? half_bits_to_f32(vp[k] >> 16) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rows && ((rmask >> (r / group)) & 1u)) {
        float sc[NL];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) d += qf[r][i] * ck[k][i];
          d = sk[k] * d + zk[k] * qsum[r];
          d = group_sum<LPT>(d);
          sc[k] = ok[k] ? d * a.sl2e : -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int k = 1; k < NL; ++k) mx = fmaxf(mx, sc[k]);
        const float mn = fmaxf(m[r], mx);
        const float alpha = ex2(m[r] - mn);
        m[r] = mn;
        l[r] *= alpha;
        zacc[r] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][i] *= alpha;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          const float pk = ex2(sc[k] - mn);
          l[r] += pk;
          const float ps = pk * sv[k];
          zacc[r] += pk * zv[k];
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[r][i] += ps * cv[k][i];
        }
      }
    }
    if (!more) break;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      kc[k] = kn[k];
      vc[k] = vn[k];
      kp[k] = kpn[k];
      vp[k] = vpn[k];
    }
    bi = bi2;
    s = s2;
    p = p2;
    nt = nt2;
  }

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
      float o[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o[i] = (acc[r][i] + zacc[r]) * sc;
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) o[i] += __shfl_xor(o[i], off);
      }
      const int64_t row = (int64_t)g * a.P + it.part_base + r;
      if (tg == 0) {
        float4* dst = (float4*)(a.pacc + row * D + dq);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
      }
      if (lane == 0) a.pml[row] = make_float2(M, lr);
    }
  }
}

// ---------------------------------------------------------------------------
// 3. combine

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ pacc, const float2* __restrict__ pml,
                                                     const int32_t* __restrict__ comb_ptr,
                                                     const int32_t* __restrict__ comb_rows, int Hq, int Hkv, int P,
                                                     float* __restrict__ out) {
  constexpr int E = D / 64;  // dims per lane
  const int j = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const int group = Hq / Hkv, g = h / group, hh = h - g * group;
  const int e0 = comb_ptr[j], e1 = comb_ptr[j + 1];
  const int64_t base = (int64_t)g * P + hh;
  float M = -INFINITY;
  for (int e = e0; e < e1; ++e) M = fmaxf(M, pml[base + comb_rows[e]].x);
  float L = 0.f, o[E];
#pragma unroll
  for (int i = 0; i < E; ++i) o[i] = 0.f;
  for (int e = e0; e < e1; ++e) {
    const int64_t row = base + comb_rows[e];
    const float2 ml = pml[row];
    const float w = ex2(ml.x - M);
    L += w * ml.y;
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] += w * pacc[row * D + threadIdx.x * E + i];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* dst = out + ((int64_t)j * Hq + h) * D + threadIdx.x * E;
#pragma unroll
  for (int i = 0; i < E; ++i) dst[i] = o[i] * inv;
}

// ---------------------------------------------------------------------------
// host side

struct WsLayout {
  size_t qhi, qlo, pacc, pml, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const kvp_shape* sh, const kvp_plan_dev* pl) {
  WsLayout w{};
  const size_t qb = align256((size_t)pl->n_qcons * sh->n_q_heads * sh->head_dim * 2);
  w.qhi = 0;
  w.qlo = qb;
  w.pacc = 2 * qb;
  w.pml = w.pacc + align256((size_t)sh->n_kv_heads * pl->n_part_rows * sh->head_dim * 4);
  w.total = w.pml + align256((size_t)sh->n_kv_heads * pl->n_part_rows * 8);
  return w;
}

int check_plan(const kvp_plan_dev* pl) {
  if (!pl) return fail(KVP_EINVAL, "plan is NULL");
  if (pl->n_agents < 0 || pl->n_phys < 0 || pl->n_items < 0 || pl->n_qcons < 0 || pl->n_part_rows < 0)
    return fail(KVP_EINVAL, "negative plan counts");
  int sum = 0;
  for (int i = 0; i < 5; ++i) {
    if (pl->class_items[i] < 0) return fail(KVP_EINVAL, "negative class count");
    sum += pl->class_items[i];
  }
  if (sum != pl->n_items) return fail(KVP_EINVAL, "class counts do not add up to n_items");
  if (pl->n_items > 0 && (!pl->items || !pl->plan_blocks || !pl->cons || !pl->qcons || !pl->phys_ntok))
    return fail(KVP_EINVAL, "plan pointer is NULL");
  if (pl->n_agents > 0 && (!pl->comb_ptr || !pl->comb_rows)) return fail(KVP_EINVAL, "plan combine pointer is NULL");
  return KVP_OK;
}

template <int D, int R>
void launch_tile(const TileArgs& a, bool q4, hipStream_t st) {
  const int total = a.n_items * a.Hkv;
  const int grid = 8 * ((total + 7) / 8);
  if (q4)
    hipLaunchKernelGGL((tile_q4_kernel<D, R>), dim3(grid), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((tile_bf16_kernel<D, R>), dim3(grid), dim3(64), 0, st, a);
}

template <int D>
void launch_class(int cls, const TileArgs& a, bool q4, hipStream_t st) {
  switch (cls) {
    case 0: launch_tile<D, 16>(a, q4, st); break;
    case 1: launch_tile<D, 8>(a, q4, st); break;
    case 2: launch_tile<D, 4>(a, q4, st); break;
    case 3: launch_tile<D, 2>(a, q4, st); break;
    default: launch_tile<D, 1>(a, q4, st); break;
  }
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

extern "C" int paged_decode_attn(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q, const void* k_pool,
                                 const void* v_pool, const void* k_params, const void* v_params, int32_t layer,
                                 float scale, float* out, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  rc = check_plan(plan);
  if (rc) return rc;
  const bool q4 = shape->kv_dtype == KVP_Q4G64;
  if (!q || !k_pool || !v_pool || !out || !workspace) return fail(KVP_EINVAL, "null device pointer");
  if (q4 && (!k_params || !v_params)) return fail(KVP_EINVAL, "Q4 pools need k_params and v_params");
  if (layer < 0 || layer >= shape->n_layers) return fail(KVP_EINVAL, "layer out of range");
  if (!std::isfinite(scale)) return fail(KVP_EINVAL, "scale");
  const WsLayout w = ws_layout(shape, plan);
  if (ws_bytes < w.total) return fail(KVP_EWORKSPACE, "workspace too small");
  if (plan->n_agents == 0) return KVP_OK;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  const int D = shape->head_dim;

  if (plan->n_qcons > 0) {
    const int threads = plan->n_qcons * (D / 2);
    hipLaunchKernelGGL(qprep_kernel, dim3((threads + 255) / 256), dim3(256), 0, st, (const uint16_t*)q, plan->qcons,
                       plan->n_qcons, shape->n_q_heads, D, shape->rope_theta, (uint16_t*)(ws + w.qhi),
                       (uint16_t*)(ws + w.qlo));
  }
  TileArgs a{};
  a.items = plan->items;
  a.plan_blocks = plan->plan_blocks;
  a.cons = plan->cons;
  a.qcons = plan->qcons;
  a.mask = plan->mask;
  a.phys_ntok = plan->phys_ntok;
  a.qhi = (const uint16_t*)(ws + w.qhi);
  a.qlo = (const uint16_t*)(ws + w.qlo);
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
  int first = 0;
  for (int cls = 0; cls < 5; ++cls) {
    const int n = plan->class_items[cls];
    if (n == 0) continue;
    a.item0 = first;
    a.n_items = n;
    if (D == 128)
      launch_class<128>(cls, a, q4, st);
    else
      launch_class<64>(cls, a, q4, st);
    first += n;
  }
  const int nw = plan->n_agents * shape->n_q_heads;
  if (D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(nw), dim3(64), 0, st, a.pacc, (const float2*)a.pml, plan->comb_ptr,
                       plan->comb_rows, shape->n_q_heads, shape->n_kv_heads, plan->n_part_rows, out);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(nw), dim3(64), 0, st, a.pacc, (const float2*)a.pml, plan->comb_ptr,
                       plan->comb_rows, shape->n_q_heads, shape->n_kv_heads, plan->n_part_rows, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
  return KVP_OK;
}
