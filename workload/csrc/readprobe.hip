// Plain HBM read probe (gfx950): the read ceiling a decode step's tile pass is
// compared against.  Every thread reads 16-byte words, U loads in flight, and
// folds them into one XOR kept only to stop the loads from being dropped.  Two
// access patterns: a grid stride (the whole grid sweeps the buffer front to
// back) and per-workgroup contiguous chunks (each workgroup streams its own
// share); which one is faster depends on the box.  Holds no part of the
// attention method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, int64_t n, uint32_t* out) {
  const int64_t st = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * st < n; i += U * st) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = NT ? __builtin_nontemporal_load(p + i + k * st) : p[i + k * st];
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += st) {
    const u32x4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // the stored value never matters; a thread writes only on a chance match
  if (acc == 0x9E3779B9u) out[0] = acc;
}

// workgroup b reads 16-byte words [b chunk, min(n, (b + 1) chunk)) with a
// workgroup stride
template <int U>
__global__ __launch_bounds__(256) void chunk_kernel(const u32x4* __restrict__ p, int64_t n, int64_t chunk,
                                                    uint32_t* out) {
  const int64_t b0 = (int64_t)blockIdx.x * chunk;
  const int64_t b1 = b0 + chunk < n ? b0 + chunk : n;
  int64_t i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * 256 < b1; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + i + k * 256);
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < b1; i += 256) {
    const u32x4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16, buf 16-byte aligned) of buf once; out: 4
// device bytes.  grid: workgroups of 256 threads (1 .. 65536); nontemporal:
// 0 or 1; chunked: 0 (grid stride) or 1 (contiguous chunk per workgroup,
// non-temporal loads).  Returns 0, -1 (bad argument) or -5 (launch error).
int kvgen_read_probe(const void* buf, int64_t bytes, void* out, int grid, int nontemporal, int chunked,
                     void* stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 || ((uintptr_t)buf & 15) || grid < 1 || grid > 65536) return -1;
  const int64_t n = bytes / 16;
  if (chunked)
    hipLaunchKernelGGL((chunk_kernel<16>), dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf, n,
                       (n + grid - 1) / grid, (uint32_t*)out);
  else if (nontemporal)
    hipLaunchKernelGGL((read_kernel<8, true>), dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf, n,
                       (uint32_t*)out);
  else
    hipLaunchKernelGGL((read_kernel<8, false>), dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf, n,
                       (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
