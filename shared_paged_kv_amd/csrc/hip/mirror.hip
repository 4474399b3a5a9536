// Master/mirror device steps on gfx950 (include/kvpool_mirror.h).
//
// TokenDance write-up, sec. 3: one dense master, every other cache a mirror of
// block-sparse differences; the restore applies the differences and restores
// the RoPE positions inside the one pass that moves the blocks, instead of
// copying the master and overwriting it afterwards.
//
// Both kernels are streaming passes over whole blocks ([Hkv][B][d] bf16 per
// layer, contiguous).  Many agents take the same master block, so a workgroup
// owns a run of up to kRun consecutive entries and splits it into sub-runs that
// share a source: each 16-byte chunk of the source is loaded once per sub-run
// and written (restore) or compared (diff) for every entry of it.  Callers that
// order entries by source get one source read per sub-run instead of one per
// destination; any order is correct.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../host/kvpool_internal.h"
#include "device_common.h"
#include "kvpool.h"
#include "kvpool_mirror.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRun = 8;  // entries per workgroup

__device__ __forceinline__ bool words_differ(uint32_t a, uint32_t b, float tau) {
  if (tau == 0.f) return a != b;
  // a NaN on either side makes the comparison false, hence "differs"
  return !(fabsf(kvp::bf16_lo(a) - kvp::bf16_lo(b)) <= tau) || !(fabsf(kvp::bf16_hi(a) - kvp::bf16_hi(b)) <= tau);
}

__device__ __forceinline__ bool chunk_differs(u32x4 a, u32x4 b, float tau) {
  bool d = false;
#pragma unroll
  for (int w = 0; w < 4; ++w) d |= words_differ(a[w], b[w], tau);
  return d;
}

// End of the sub-run that starts at e: the following entries with the same
// source (and, where given, the same valid-token count).
__device__ __forceinline__ int sub_run_end(const int* src, const int* nt, int e, int ne) {
  int e1 = e + 1;
  while (e1 < ne && src[e1] == src[e] && (!nt || nt[e1] == nt[e])) ++e1;
  return e1;
}

// Workgroup (run of entries, layer).  A thread owns 8 rotate-half pairs of one
// token row: 16 bytes at i0 and 16 bytes at i0 + D/2, for K and for V.  cos/sin
// of every (entry, pair) are formed once per workgroup (float64 angle) into LDS.
template <int D>
__global__ __launch_bounds__(256) void restore_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                                                      int pool_blocks, const int32_t* __restrict__ entries, int n,
                                                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                      int dst_blocks, int Hkv, int B, float base) {
  constexpr int H = D / 2, Q = H / 8, RPP = 256 / Q;
  __shared__ int s_src[kRun], s_shift[kRun], s_nt[kRun], s_dst[kRun];
  __shared__ float2 s_cs[kRun][H];
  const int e0 = blockIdx.x * kRun, ne = min(kRun, n - e0);
  const int64_t layer = blockIdx.y;
  const int t = threadIdx.x;
  if (t < ne) {
    const int32_t* E = entries + 4 * (int64_t)(e0 + t);
    const int src = E[0], shift = E[1], nt = E[2], dst = E[3];
    const bool ok = src >= 0 && src < pool_blocks && nt >= 0 && nt <= B && dst >= 0 && dst < dst_blocks;
    s_src[t] = ok ? src : -1;  // a sub-run of -1 is skipped
    s_shift[t] = shift;
    s_nt[t] = nt;
    s_dst[t] = dst;
  }
  __syncthreads();
  for (int x = t; x < ne * H; x += 256) {
    const int e = x / H, i = x % H;
    float c = 1.f, s = 0.f;
    if (s_shift[e] != 0) kvp::rope_cs(s_shift[e], i, D, base, &c, &s);
    s_cs[e][i] = make_float2(c, s);
  }
  __syncthreads();
  const int64_t blk = (int64_t)Hkv * B * D;
  const int i0 = 8 * (t % Q), r0 = t / Q;
  for (int e = 0; e < ne;) {
    const int e1 = sub_run_end(s_src, s_nt, e, ne);
    const int src = s_src[e], nt = s_nt[e];
    if (src >= 0) {
      const uint16_t* ks = kp + (layer * pool_blocks + src) * blk;
      const uint16_t* vs = vp + (layer * pool_blocks + src) * blk;
      for (int row = r0; row < Hkv * B; row += RPP) {
        const int64_t o = (int64_t)row * D + i0;
        const bool valid = row % B < nt;
        u32x4 k1 = {0u, 0u, 0u, 0u}, k2 = k1, v1 = k1, v2 = k1;
        if (valid) {
          k1 = *(const u32x4*)(ks + o);
          k2 = *(const u32x4*)(ks + o + H);
          v1 = *(const u32x4*)(vs + o);
          v2 = *(const u32x4*)(vs + o + H);
        }
        for (int k = e; k < e1; ++k) {
          u32x4 a = k1, b = k2;
          if (valid && s_shift[k] != 0) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              uint32_t ra = 0, rb = 0;
#pragma unroll
              for (int hw = 0; hw < 2; ++hw) {
                const float2 cs = s_cs[k][i0 + 2 * w + hw];
                const float x1 = hw ? kvp::bf16_hi(k1[w]) : kvp::bf16_lo(k1[w]);
                const float x2 = hw ? kvp::bf16_hi(k2[w]) : kvp::bf16_lo(k2[w]);
                float y1, y2;
                kvp::rope_apply(x1, x2, cs.x, cs.y, &y1, &y2);
                ra |= (uint32_t)kvp::f32_to_bf16_rne(y1) << (16 * hw);
                rb |= (uint32_t)kvp::f32_to_bf16_rne(y2) << (16 * hw);
              }
              a[w] = ra;
              b[w] = rb;
            }
          }
          const int64_t d0 = (layer * dst_blocks + s_dst[k]) * blk + o;
          *(u32x4*)(dk + d0) = a;
          *(u32x4*)(dk + d0 + H) = b;
          *(u32x4*)(dv + d0) = v1;
          *(u32x4*)(dv + d0 + H) = v2;
        }
      }
    }
    e = e1;
  }
}

// Workgroup = run of pairs, over every layer.  Per layer and sub-run (pairs with
// the same master): every thread loads its 16-byte chunks of the master once
// and of each undecided candidate, and compares the valid tokens.  A pair is
// decided once a difference is seen; the workgroup stops when all are.
__global__ __launch_bounds__(256) void diff_blocks_kernel(const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
                                                          int pool_blocks, const uint8_t* __restrict__ ck,
                                                          const uint8_t* __restrict__ cv, int cand_blocks,
                                                          const int32_t* __restrict__ pairs, int n, float tau,
                                                          int32_t* __restrict__ flags, int L, int Hkv, int B, int d) {
  __shared__ int s_m[kRun], s_c[kRun], s_nt[kRun];
  __shared__ unsigned s_found;
  const int e0 = blockIdx.x * kRun, ne = min(kRun, n - e0);
  const int t = threadIdx.x;
  if (t == 0) s_found = 0u;
  if (t < ne) {
    const int32_t* P = pairs + 3 * (int64_t)(e0 + t);
    const int m = P[0], c = P[1], nt = P[2];
    const bool ok = m >= 0 && m < pool_blocks && c >= 0 && c < cand_blocks && nt >= 0 && nt <= B;
    s_m[t] = ok ? m : -1;
    s_c[t] = c;
    s_nt[t] = nt;
  }
  __syncthreads();
  unsigned valid = 0u;
  for (int e = 0; e < ne; ++e) valid |= (s_m[e] >= 0 ? 1u : 0u) << e;
  const int64_t block_bytes = (int64_t)Hkv * B * d * 2;
  const int64_t units = block_bytes / 16;
  const int row_units = d / 8;
  unsigned found = 0u;  // uniform: pairs decided in earlier layers
  for (int layer = 0; layer < L && (valid & ~found); ++layer) {
    unsigned mine = 0u;
    for (int e = 0; e < ne;) {
      const int e1 = sub_run_end(s_m, nullptr, e, ne);
      unsigned todo = 0u;
      for (int k = e; k < e1; ++k) todo |= ((valid & ~found) >> k & 1u) << (k - e);
      if (todo) {
        const int64_t mo = ((int64_t)layer * pool_blocks + s_m[e]) * block_bytes;
        for (int64_t u = t; u < units; u += 256) {
          const int tok = (int)((u / row_units) % B);
          const u32x4 mk = *(const u32x4*)(kp + mo + 16 * u), mv = *(const u32x4*)(vp + mo + 16 * u);
          u32x4 xk[kRun], xv[kRun];
#pragma unroll
          for (int k = 0; k < kRun; ++k) {
            if (todo >> k & 1u) {
              const int64_t co = ((int64_t)layer * cand_blocks + s_c[e + k]) * block_bytes + 16 * u;
              xk[k] = *(const u32x4*)(ck + co);
              xv[k] = *(const u32x4*)(cv + co);
            }
          }
#pragma unroll
          for (int k = 0; k < kRun; ++k) {
            if ((todo >> k & 1u) && tok < s_nt[e + k] && (chunk_differs(mk, xk[k], tau) || chunk_differs(mv, xv[k], tau)))
              mine |= 1u << (e + k);
          }
        }
      }
      e = e1;
    }
    if (mine) atomicOr(&s_found, mine);
    __syncthreads();
    found = s_found;
    __syncthreads();
  }
  if (t < ne) flags[e0 + t] = s_m[t] < 0 ? -1 : (int)(found >> t & 1u);
}

}  // namespace

extern "C" int kv_diff_blocks(const kvp_shape* shape, const void* k_pool, const void* v_pool, int32_t pool_blocks,
                              const void* cand_k, const void* cand_v, int32_t cand_blocks, const int32_t* pairs,
                              int32_t n, float tau, int32_t* flags, void* stream) {
  int rc = kvp::check_shape(shape);
  if (rc) return rc;
  if (shape->kv_dtype != KVP_BF16) return kvp::fail(KVP_EINVAL, "kv_diff_blocks supports bf16 pools");
  if (n < 0 || pool_blocks < 1 || cand_blocks < 1) return kvp::fail(KVP_EINVAL, "negative count or block count");
  if (!(tau >= 0.f) || !std::isfinite(tau)) return kvp::fail(KVP_EINVAL, "tau must be finite and >= 0");
  if (n > 0 && (!k_pool || !v_pool || !cand_k || !cand_v || !pairs || !flags))
    return kvp::fail(KVP_EINVAL, "a device pointer is NULL");
  if (n == 0) return KVP_OK;
  if (n > INT32_MAX - kRun) return kvp::fail(KVP_EINVAL, "too many pairs");
  const unsigned runs = (unsigned)((n + kRun - 1) / kRun);
  hipLaunchKernelGGL(diff_blocks_kernel, dim3(runs), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)k_pool,
                     (const uint8_t*)v_pool, pool_blocks, (const uint8_t*)cand_k, (const uint8_t*)cand_v, cand_blocks,
                     pairs, n, tau, flags, shape->n_layers, shape->n_kv_heads, shape->block_tokens, shape->head_dim);
  if (hipGetLastError() != hipSuccess) return kvp::fail(KVP_EHIP, "kv_diff_blocks launch failed");
  return KVP_OK;
}

extern "C" int kv_restore(const kvp_shape* shape, const void* k_pool, const void* v_pool, int32_t pool_blocks,
                          const int32_t* entries, int32_t n, void* dst_k, void* dst_v, int32_t dst_blocks,
                          void* stream) {
  int rc = kvp::check_shape(shape);
  if (rc) return rc;
  if (shape->kv_dtype != KVP_BF16) return kvp::fail(KVP_EINVAL, "kv_restore supports bf16 pools");
  if (n < 0 || pool_blocks < 1 || dst_blocks < 1) return kvp::fail(KVP_EINVAL, "negative count or block count");
  if (n > 0 && (!k_pool || !v_pool || !entries || !dst_k || !dst_v)) return kvp::fail(KVP_EINVAL, "a device pointer is NULL");
  if (shape->n_layers > 65535 || n > INT32_MAX - kRun) return kvp::fail(KVP_EINVAL, "too many layers or entries");
  if (n == 0) return KVP_OK;
  const dim3 grid((unsigned)((n + kRun - 1) / kRun), (unsigned)shape->n_layers);
  hipStream_t st = (hipStream_t)stream;
  const int Hkv = shape->n_kv_heads, B = shape->block_tokens;
  if (shape->head_dim == 128)
    hipLaunchKernelGGL(restore_kernel<128>, grid, dim3(256), 0, st, (const uint16_t*)k_pool, (const uint16_t*)v_pool,
                       pool_blocks, entries, n, (uint16_t*)dst_k, (uint16_t*)dst_v, dst_blocks, Hkv, B,
                       shape->rope_theta);
  else
    hipLaunchKernelGGL(restore_kernel<64>, grid, dim3(256), 0, st, (const uint16_t*)k_pool, (const uint16_t*)v_pool,
                       pool_blocks, entries, n, (uint16_t*)dst_k, (uint16_t*)dst_v, dst_blocks, Hkv, B,
                       shape->rope_theta);
  if (hipGetLastError() != hipSuccess) return kvp::fail(KVP_EHIP, "kv_restore launch failed");
  return KVP_OK;
}
