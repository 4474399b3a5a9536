// kv_rerotate: batched RoPE offset compensation on gfx950.
//
// INMS walkthrough, sec. 2.3 / 3.2: a stored key reused at another position is
// rotated by an angle that depends only on the position difference; values are
// not rotated.  TokenDance write-up, sec. 2: the rotation is done in one batched
// call for all requests of a round.  One thread per (row, rotate-half pair): it
// forms cos/sin of shift * theta_i once (float64 angle) and rotates that pair in
// every head of the row.
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
  int64_t threads = n_rows * (head_dim / 2);
  int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return fail(KVP_EINVAL, "kv_rerotate: too many rows");
  hipLaunchKernelGGL(rerotate_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, x, y, shift,
                     n_rows, (int)n_heads, (int)head_dim, rope_theta, (int)in_dtype, (int)out_dtype);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVP_EHIP, hipGetErrorString(e));
  return KVP_OK;
}
