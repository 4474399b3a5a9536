// Device filler for the synthetic KV pools and queries (gfx950).
//
// Produces exactly the values workload/rng.py and workload/spec.py produce on
// the host: Philox4x32-10 (Salmon et al., SC'11) keyed by a block's 16-byte
// content seed, one word per element, Irwin-Hall byte sum scaled by 7/1024,
// rounded to bf16; slots past a block's valid tokens hold NaN; the Q4 variant
// encodes those bf16 values groupwise (64 elements, fp16 scale and zero).
// Holds no part of the attention method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

__device__ __forceinline__ float ih_value(uint32_t w) {
  const int s = (int)(w & 0xff) + (int)((w >> 8) & 0xff) + (int)((w >> 16) & 0xff) + (int)(w >> 24) - 510;
  return (float)(s * 7) * (1.0f / 1024.0f);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// words for elements 4*qd .. 4*qd+3 of a tile
__device__ __forceinline__ void tile_quad(const uint32_t* sd, int layer, int sel, uint32_t qd, uint32_t out[4]) {
  out[0] = qd;
  out[1] = sd[3];
  out[2] = (uint32_t)(sel & 0xff) | ((uint32_t)layer << 8);
  out[3] = sd[2];
  philox(out, sd[0], sd[1]);
}

// one thread per 4 consecutive elements of one (block, layer) tile [H][B][D]
__global__ __launch_bounds__(256) void fill_bf16_kernel(uint16_t* __restrict__ pool, const uint32_t* __restrict__ seeds,
                                                        const int32_t* __restrict__ ntok, int n_phys, int stride,
                                                        int layer, int H, int B, int D, int sel) {
  const int64_t quads_per_tile = (int64_t)H * B * D / 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= quads_per_tile * n_phys) return;
  const int p = (int)(t / quads_per_tile);
  const uint32_t qd = (uint32_t)(t % quads_per_tile);
  uint32_t w[4];
  tile_quad(seeds + 4 * (int64_t)p, layer, sel, qd, w);
  const int tok = (int)((qd * 4 / D) % B);
  const bool pad = tok >= ntok[p];
  uint16_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pad ? (uint16_t)0x7fc0 : bf16_rne(ih_value(w[i]));
  uint2 pk;
  pk.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  pk.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  *(uint2*)(pool + ((int64_t)layer * stride + p) * H * B * D + (int64_t)qd * 4) = pk;
}

// one thread per (block, head, token, group of 64): draw, then encode
__global__ __launch_bounds__(256) void fill_q4_kernel(uint8_t* __restrict__ codes, uint16_t* __restrict__ params,
                                                      const uint32_t* __restrict__ seeds,
                                                      const int32_t* __restrict__ ntok, int n_phys, int stride,
                                                      int layer, int H, int B, int D, int sel) {
  const int NG = D / 64;
  const int64_t per_tile = (int64_t)H * B * NG;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= per_tile * n_phys) return;
  const int p = (int)(t / per_tile);
  const int64_t r = t % per_tile;  // (h * B + tok) * NG + grp
  const int grp = (int)(r % NG);
  const int tok = (int)((r / NG) % B);
  const int64_t row = ((int64_t)layer * stride + p) * H * B + r / NG;  // row index in the pool
  uint8_t* cdst = codes + row * (D / 2) + grp * 32;
  uint16_t* pdst = params + (row * NG + grp) * 2;
  if (tok >= ntok[p]) {
    for (int i = 0; i < 32; i += 4) *(uint32_t*)(cdst + i) = 0u;
    pdst[0] = 0x7e00;
    pdst[1] = 0x7e00;
    return;
  }
  float x[64];
  const uint32_t e0 = (uint32_t)((r / NG) * D + grp * 64);
#pragma unroll
  for (int qd = 0; qd < 16; ++qd) {
    uint32_t w[4];
    tile_quad(seeds + 4 * (int64_t)p, layer, sel, e0 / 4 + qd, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * qd + i] = __uint_as_float((uint32_t)bf16_rne(ih_value(w[i])) << 16);
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 64; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  const _Float16 s16 = (_Float16)((mx - mn) / 15.0f);
  const _Float16 z16 = (_Float16)mn;
  const float s = (float)s16, z = (float)z16;
  uint32_t packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    uint32_t c = 0;
    if (s != 0.f) {
      float f = rintf((x[i] - z) / s);
      f = fminf(fmaxf(f, 0.f), 15.f);
      c = (uint32_t)f;
    }
    packed[i / 8] |= c << (4 * (i % 8));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) *(uint32_t*)(cdst + 4 * i) = packed[i];
  pdst[0] = __builtin_bit_cast(uint16_t, s16);
  pdst[1] = __builtin_bit_cast(uint16_t, z16);
}

// queries: one thread per 4 elements of agent j's [Hq][D] tile
__global__ __launch_bounds__(256) void fill_q_kernel(uint16_t* __restrict__ q, const uint32_t* __restrict__ seeds,
                                                     int n_agents, int layer, int Hq, int D) {
  const int64_t quads = (int64_t)Hq * D / 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= quads * n_agents) return;
  const int j = (int)(t / quads);
  const uint32_t qd = (uint32_t)(t % quads);
  uint32_t w[4];
  tile_quad(seeds + 4 * (int64_t)j, layer, 2, qd, w);
  uint2 pk;
  pk.x = (uint32_t)bf16_rne(ih_value(w[0])) | ((uint32_t)bf16_rne(ih_value(w[1])) << 16);
  pk.y = (uint32_t)bf16_rne(ih_value(w[2])) | ((uint32_t)bf16_rne(ih_value(w[3])) << 16);
  *(uint2*)(q + (int64_t)j * Hq * D + (int64_t)qd * 4) = pk;
}

inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

extern "C" {

// pool: [n_layers][stride][H][B][D] bf16 (stride >= n_phys blocks per layer);
// fills blocks [0, n_phys) of layer `layer`.
int kvgen_fill_bf16(void* pool, const void* seeds, const void* ntok, int n_phys, int stride, int layer, int H, int B,
                    int D, int sel, void* stream) {
  if (n_phys <= 0) return 0;
  if (stride < n_phys) return -1;
  if ((int64_t)H * B * D % 4) return -1;
  const int64_t threads = (int64_t)H * B * D / 4 * n_phys;
  hipLaunchKernelGGL(fill_bf16_kernel, dim3(grid_for(threads)), dim3(256), 0, (hipStream_t)stream, (uint16_t*)pool,
                     (const uint32_t*)seeds, (const int32_t*)ntok, n_phys, stride, layer, H, B, D, sel);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// codes: [n_layers][stride][H][B][D/2] uint8; params: [...][D/64][2] fp16
// (stride >= n_phys blocks per layer); fills blocks [0, n_phys) of one layer.
int kvgen_fill_q4(void* codes, void* params, const void* seeds, const void* ntok, int n_phys, int stride, int layer,
                  int H, int B, int D, int sel, void* stream) {
  if (n_phys <= 0) return 0;
  if (D % 64 || stride < n_phys) return -1;
  const int64_t threads = (int64_t)H * B * (D / 64) * n_phys;
  hipLaunchKernelGGL(fill_q4_kernel, dim3(grid_for(threads)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)codes,
                     (uint16_t*)params, (const uint32_t*)seeds, (const int32_t*)ntok, n_phys, stride, layer, H, B, D,
                     sel);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// q: [n_agents][Hq][D] bf16 for one layer.
int kvgen_fill_q(void* q, const void* seeds, int n_agents, int layer, int Hq, int D, void* stream) {
  if (n_agents <= 0) return 0;
  const int64_t threads = (int64_t)Hq * D / 4 * n_agents;
  hipLaunchKernelGGL(fill_q_kernel, dim3(grid_for(threads)), dim3(256), 0, (hipStream_t)stream, (uint16_t*)q,
                     (const uint32_t*)seeds, n_agents, layer, Hq, D);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
