// Master/mirror device steps on gfx950 (include/kvpool_mirror.h).
//
// TokenDance write-up, sec. 3: one dense master, every other cache a mirror of
// block-sparse differences; the restore applies the differences and restores
// the RoPE positions inside the one pass that moves the blocks, instead of
// copying the master and overwriting it afterwards.  Both kernels are streaming
// passes over whole blocks ([Hkv][B][d] per layer, contiguous): 16-byte (diff)
// or 8-byte (restore) accesses, consecutive threads on consecutive bytes.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../host/kvpool_internal.h"
#include "device_common.h"
#include "kvpool.h"
#include "kvpool_mirror.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bool words_differ(uint32_t a, uint32_t b, float tau) {
  if (tau == 0.f) return a != b;
  const float a0 = __uint_as_float(a << 16), a1 = __uint_as_float(a & 0xffff0000u);
  const float b0 = __uint_as_float(b << 16), b1 = __uint_as_float(b & 0xffff0000u);
  // a NaN on either side makes the comparison false, hence "differs"
  return !(fabsf(a0 - b0) <= tau) || !(fabsf(a1 - b1) <= tau);
}

// One workgroup per pair, over every layer; it stops once a difference is seen.
__global__ __launch_bounds__(256) void diff_blocks_kernel(const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
                                                          int pool_blocks, const uint8_t* __restrict__ ck,
                                                          const uint8_t* __restrict__ cv, int cand_blocks,
                                                          const int32_t* __restrict__ pairs, float tau,
                                                          int32_t* __restrict__ flags, int L, int Hkv, int B, int d) {
  const int i = blockIdx.x;
  const int master = pairs[3 * i], cand = pairs[3 * i + 1], nt = pairs[3 * i + 2];
  if (master < 0 || master >= pool_blocks || cand < 0 || cand >= cand_blocks || nt < 0 || nt > B) {
    if (threadIdx.x == 0) flags[i] = -1;
    return;
  }
  __shared__ int s_diff;
  if (threadIdx.x == 0) s_diff = 0;
  __syncthreads();
  const int64_t block_bytes = (int64_t)Hkv * B * d * 2;
  const int row_chunks = d / 8;  // 16-byte chunks per token row
  for (int layer = 0; layer < L; ++layer) {
    const int64_t mo = ((int64_t)layer * pool_blocks + master) * block_bytes;
    const int64_t co = ((int64_t)layer * cand_blocks + cand) * block_bytes;
    int found = 0;
    for (int64_t c = threadIdx.x; c < block_bytes / 16; c += 256) {
      const int tok = (int)((c / row_chunks) % B);
      if (tok >= nt) continue;
      const u32x4 a = *(const u32x4*)(kp + mo + 16 * c), b = *(const u32x4*)(ck + co + 16 * c);
      const u32x4 e = *(const u32x4*)(vp + mo + 16 * c), f = *(const u32x4*)(cv + co + 16 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) found |= words_differ(a[w], b[w], tau) | words_differ(e[w], f[w], tau);
    }
    if (found) s_diff = 1;  // benign race: every writer stores 1
    __syncthreads();
    const int any = s_diff;
    __syncthreads();
    if (any) break;
  }
  if (threadIdx.x == 0) flags[i] = s_diff;
}

// One workgroup per (destination block, layer); a thread owns 4 consecutive
// rotate-half pairs (cos/sin formed once, float64 angles) of one token row per
// pass.
__global__ __launch_bounds__(256) void restore_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                                                      int pool_blocks, const int32_t* __restrict__ blocks, int n,
                                                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int Hkv,
                                                      int B, int d, float base) {
  const int bi = (int)(blockIdx.x % (unsigned)n);
  const int64_t layer = blockIdx.x / (unsigned)n;
  const int src = blocks[3 * bi], shift = blocks[3 * bi + 1], nt = blocks[3 * bi + 2];
  if (src < 0 || src >= pool_blocks || nt < 0 || nt > B) return;  // not a valid entry
  const int half = d / 2, q = half / 4, rows_per_pass = 256 / q;
  const int i0 = 4 * (threadIdx.x % q), r0 = threadIdx.x / q;
  float c[4], s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    c[k] = 1.f;
    s[k] = 0.f;
    if (shift != 0) kvp::rope_cs(shift, i0 + k, d, base, &c[k], &s[k]);
  }
  const int64_t sb = (layer * pool_blocks + src) * Hkv * B * d;
  const int64_t db = (layer * n + bi) * Hkv * B * d;
  for (int row = r0; row < Hkv * B; row += rows_per_pass) {
    const int64_t o = (int64_t)row * d;
    u32x2 k1 = (u32x2){0u, 0u}, k2 = (u32x2){0u, 0u}, v1 = (u32x2){0u, 0u}, v2 = (u32x2){0u, 0u};
    if (row % B < nt) {
      k1 = *(const u32x2*)(kp + sb + o + i0);
      k2 = *(const u32x2*)(kp + sb + o + half + i0);
      v1 = *(const u32x2*)(vp + sb + o + i0);
      v2 = *(const u32x2*)(vp + sb + o + half + i0);
      if (shift != 0) {
        uint16_t a[4], b[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wa = k1[k >> 1], wb = k2[k >> 1];
          const float x1 = kvp::bf16_to_f32((uint16_t)(k & 1 ? wa >> 16 : wa & 0xffffu));
          const float x2 = kvp::bf16_to_f32((uint16_t)(k & 1 ? wb >> 16 : wb & 0xffffu));
          float y1, y2;
          kvp::rope_apply(x1, x2, c[k], s[k], &y1, &y2);
          a[k] = kvp::f32_to_bf16_rne(y1);
          b[k] = kvp::f32_to_bf16_rne(y2);
        }
        k1 = (u32x2){(uint32_t)a[0] | ((uint32_t)a[1] << 16), (uint32_t)a[2] | ((uint32_t)a[3] << 16)};
        k2 = (u32x2){(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16)};
      }
    }
    *(u32x2*)(dk + db + o + i0) = k1;
    *(u32x2*)(dk + db + o + half + i0) = k2;
    *(u32x2*)(dv + db + o + i0) = v1;
    *(u32x2*)(dv + db + o + half + i0) = v2;
  }
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
  hipLaunchKernelGGL(diff_blocks_kernel, dim3((unsigned)n), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)k_pool,
                     (const uint8_t*)v_pool, pool_blocks, (const uint8_t*)cand_k, (const uint8_t*)cand_v, cand_blocks,
                     pairs, tau, flags, shape->n_layers, shape->n_kv_heads, shape->block_tokens, shape->head_dim);
  if (hipGetLastError() != hipSuccess) return kvp::fail(KVP_EHIP, "kv_diff_blocks launch failed");
  return KVP_OK;
}

extern "C" int kv_restore(const kvp_shape* shape, const void* k_pool, const void* v_pool, int32_t pool_blocks,
                          const int32_t* blocks, int32_t n, void* dst_k, void* dst_v, void* stream) {
  int rc = kvp::check_shape(shape);
  if (rc) return rc;
  if (shape->kv_dtype != KVP_BF16) return kvp::fail(KVP_EINVAL, "kv_restore supports bf16 pools");
  if (n < 0 || pool_blocks < 1) return kvp::fail(KVP_EINVAL, "negative count or block count");
  if (n > 0 && (!k_pool || !v_pool || !blocks || !dst_k || !dst_v)) return kvp::fail(KVP_EINVAL, "a device pointer is NULL");
  if ((int64_t)n * shape->n_layers > INT32_MAX) return kvp::fail(KVP_EINVAL, "too many blocks");
  if (n == 0) return KVP_OK;
  hipLaunchKernelGGL(restore_kernel, dim3((unsigned)(n * shape->n_layers)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)k_pool, (const uint16_t*)v_pool, pool_blocks, blocks, n, (uint16_t*)dst_k,
                     (uint16_t*)dst_v, shape->n_kv_heads, shape->block_tokens, shape->head_dim, shape->rope_theta);
  if (hipGetLastError() != hipSuccess) return kvp::fail(KVP_EHIP, "kv_restore launch failed");
  return KVP_OK;
}
