// kv_rerotate: batched RoPE offset compensation on gfx950.
//
// INMS walkthrough, sec. 2.3 / 3.2: a stored key reused at another position is
// rotated by an angle that depends only on the position difference; values are
// not rotated.  TokenDance write-up, sec. 2: the rotation is done in one batched
// call for all requests of a round.  A row's heads share its shift, so cos/sin
// of shift * theta_i (float64 angle) are formed once per (row, pair) and applied
// in every head.  Two kernels: a vector one (8 pairs per thread, 16-byte
// accesses) for head_dim a multiple of 16 on 16-byte aligned buffers, and a
// per-pair one for everything else; both round identically.
#include <hip/hip_runtime.h>

#include "../host/kvpool_internal.h"
#include "device_common.h"
#include "kvpool.h"

namespace {

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == KVP_BF16) return kvp::bf16_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}
__device__ __forceinline__ void store_elem(void* base, int64_t idx, int dtype, float v) {
  if (dtype == KVP_BF16)
    ((uint16_t*)base)[idx] = kvp::f32_to_bf16_rne(v);
  else
    ((float*)base)[idx] = v;
}

__global__ __launch_bounds__(256) void rerotate_kernel(const void* __restrict__ x, void* y,
                                                       const int32_t* __restrict__ shift, int64_t n_rows,
                                                       int n_heads, int d, float base, int in_dt, int out_dt) {
  const int half = d / 2;
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_rows * half) return;
  int64_t r = t / half;
  int i = (int)(t % half);
  float c, s;
  kvp::rope_cs(shift[r], i, d, base, &c, &s);
  for (int h = 0; h < n_heads; ++h) {
    int64_t o = (r * n_heads + h) * d;
    float x1 = load_elem(x, o + i, in_dt), x2 = load_elem(x, o + i + half, in_dt);
    float y1, y2;
    kvp::rope_apply(x1, x2, c, s, &y1, &y2);
    store_elem(y, o + i, out_dt, y1);
    store_elem(y, o + i + half, out_dt, y2);
  }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const u32x4 w = *(const u32x4*)p;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = kvp::bf16_lo(w[k]);
    v[2 * k + 1] = kvp::bf16_hi(w[k]);
  }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[k] = a[k];
    v[4 + k] = b[k];
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = (uint32_t)kvp::f32_to_bf16_rne(v[2 * k]) | ((uint32_t)kvp::f32_to_bf16_rne(v[2 * k + 1]) << 16);
  *(u32x4*)p = w;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *(f32x4*)p = (f32x4){v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = (f32x4){v[4], v[5], v[6], v[7]};
}

// Vector path (head_dim a multiple of 16, 16-byte aligned buffers): a thread
// owns 8 consecutive rotate-half pairs of one row, forms their cos/sin once
// (theta_i from LDS, the same float64 steps as the scalar path) and rotates
// them in every head of the row with 16-byte accesses.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void rerotate_vec_kernel(const TI* x, TO* y, const int32_t* __restrict__ shift,
                                                           int64_t n_rows, int n_heads, int d, float base) {
  __shared__ double s_th[256];
  const int half = d / 2, G = half / 8, rows_per_wg = 256 / G;
  for (int i = threadIdx.x; i < half; i += 256) s_th[i] = kvp::rope_theta(i, d, base);
  __syncthreads();
  const int slot = threadIdx.x / G, g = threadIdx.x % G;
  const int64_t r = (int64_t)blockIdx.x * rows_per_wg + slot;
  if (slot >= rows_per_wg || r >= n_rows) return;
  const int i0 = 8 * g;
  const int32_t sh = shift[r];
  float c[8], s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) kvp::rope_cs_theta(sh, s_th[i0 + k], &c[k], &s[k]);
  for (int h = 0; h < n_heads; ++h) {
    const int64_t o = (r * n_heads + h) * d + i0;
    float x1[8], x2[8], y1[8], y2[8];
    load8(x + o, x1);
    load8(x + o + half, x2);
#pragma unroll
    for (int k = 0; k < 8; ++k) kvp::rope_apply(x1[k], x2[k], c[k], s[k], &y1[k], &y2[k]);
    store8(y + o, y1);
    store8(y + o + half, y2);
  }
}

template <typename TI, typename TO>
void launch_vec(const void* x, void* y, const int32_t* shift, int64_t n_rows, int n_heads, int d, float base,
                hipStream_t st) {
  const int rows_per_wg = 256 / (d / 16);
  const int64_t blocks = (n_rows + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((rerotate_vec_kernel<TI, TO>), dim3((unsigned)blocks), dim3(256), 0, st, (const TI*)x, (TO*)y,
                     shift, n_rows, n_heads, d, base);
}

}  // namespace

extern "C" int kv_rerotate(const void* x, void* y, const int32_t* shift, int64_t n_rows, int32_t n_heads,
                           int32_t head_dim, float rope_theta, int32_t in_dtype, int32_t out_dtype, void* stream) {
  using namespace kvp;
  if (!x || !y || !shift) return fail(KVP_EINVAL, "kv_rerotate: null pointer");
  if (n_rows < 0 || n_heads < 1 || head_dim < 2 || head_dim % 2 || head_dim > 512)
    return fail(KVP_EINVAL, "kv_rerotate: bad sizes");
  if ((in_dtype != KVP_BF16 && in_dtype != KVP_F32) || (out_dtype != KVP_BF16 && out_dtype != KVP_F32))
    return fail(KVP_EINVAL, "kv_rerotate: dtype must be KVP_BF16 or KVP_F32");
  if (!(rope_theta > 0.f)) return fail(KVP_EINVAL, "kv_rerotate: rope_theta");
  if (x == y && in_dtype != out_dtype) return fail(KVP_EINVAL, "kv_rerotate: in-place needs equal dtypes");
  if (n_rows == 0) return KVP_OK;
  hipStream_t st = (hipStream_t)stream;
  if (head_dim % 16 == 0 && ((uintptr_t)x | (uintptr_t)y) % 16 == 0 && n_rows / (256 / (head_dim / 16)) < 0x7fffffff) {
    if (in_dtype == KVP_BF16 && out_dtype == KVP_BF16)
      launch_vec<uint16_t, uint16_t>(x, y, shift, n_rows, n_heads, head_dim, rope_theta, st);
    else if (in_dtype == KVP_BF16)
      launch_vec<uint16_t, float>(x, y, shift, n_rows, n_heads, head_dim, rope_theta, st);
    else if (out_dtype == KVP_BF16)
      launch_vec<float, uint16_t>(x, y, shift, n_rows, n_heads, head_dim, rope_theta, st);
    else
      launch_vec<float, float>(x, y, shift, n_rows, n_heads, head_dim, rope_theta, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
    return KVP_OK;
  }
  int64_t threads = n_rows * (head_dim / 2);
  int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return fail(KVP_EINVAL, "kv_rerotate: too many rows");
  hipLaunchKernelGGL(rerotate_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, y, shift,
                     n_rows, (int)n_heads, (int)head_dim, rope_theta, (int)in_dtype, (int)out_dtype);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
  return KVP_OK;
}
