// kv_append: the device work of one decode-time append on gfx950.
//
// INMS walkthrough, sec. 2.2: a write into a shared block first copies it
// (copy-on-write), then writes into the private copy.  The host side
// (kvpool_append) decides which blocks to copy and where each new token goes;
// here every copy runs first (one launch), then every token write (a second
// launch on the same stream, so a write never races a copy of its block).
// A token's K arrives post-RoPE at its logical position and is stored in the
// block's frame, rotated by -shift (INMS walkthrough, sec. 2.3: the
// compensation depends only on the position difference; V is not rotated).
#include <hip/hip_runtime.h>

#include "../host/kvpool_internal.h"
#include "device_common.h"
#include "kvpool.h"
#include "kvpool_lifecycle.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (copy, layer): the block's K and V of every kv head are one
// contiguous run each ([Hkv][B][d] bf16) -- a plain 16-byte streaming copy.  The
// source is often shared by many copies (cached loads); the copies are not read
// again before the next decode (non-temporal stores).
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ kp, uint8_t* __restrict__ vp,
                                                          const int32_t* __restrict__ copies, int n_copies,
                                                          int capacity, int64_t block_bytes) {
  const int c = (int)(blockIdx.x % (unsigned)n_copies);
  const int64_t layer = blockIdx.x / (unsigned)n_copies;
  const int src = copies[2 * c], dst = copies[2 * c + 1];
  if (src < 0 || src >= capacity || dst < 0 || dst >= capacity || src == dst) return;  // not a valid copy
  const int64_t so = (layer * capacity + src) * block_bytes, dof = (layer * capacity + dst) * block_bytes;
  for (int64_t o = (int64_t)threadIdx.x * 16; o < block_bytes; o += 256 * 16) {
    const u32x4 k = *(const u32x4*)(kp + so + o);
    const u32x4 v = *(const u32x4*)(vp + so + o);
    __builtin_nontemporal_store(k, (u32x4*)(kp + dof + o));
    __builtin_nontemporal_store(v, (u32x4*)(vp + dof + o));
  }
}

// One workgroup per (write, chunk of kLayerChunk layers).  The rotation depends
// only on the shift and the pair index, so a thread forms cos/sin of its pair
// once (float64 angle) and applies it to its kv heads in every layer of the
// chunk; consecutive threads touch consecutive elements.
constexpr int kLayerChunk = 8;

__global__ __launch_bounds__(256) void write_tokens_kernel(uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                           const int32_t* __restrict__ writes, int n_writes,
                                                           const uint16_t* __restrict__ knew,
                                                           const uint16_t* __restrict__ vnew, int n_rows,
                                                           int capacity, int L, int Hkv, int B, int d, float base) {
  const int wi = (int)(blockIdx.x % (unsigned)n_writes);
  const int l0 = (int)(blockIdx.x / (unsigned)n_writes) * kLayerChunk;
  const int phys = writes[4 * wi], slot = writes[4 * wi + 1], row = writes[4 * wi + 2], shift = writes[4 * wi + 3];
  if (phys < 0 || phys >= capacity || slot < 0 || slot >= B || row < 0 || row >= n_rows) return;  // not a valid write
  const int half = d / 2, hs = blockDim.x / half;  // head slots per pass
  const int i = threadIdx.x % half, h0 = threadIdx.x / half;
  float c = 1.f, s = 0.f;
  if (shift != 0) kvp::rope_cs(-shift, i, d, base, &c, &s);
  for (int64_t layer = l0; layer < min(L, l0 + kLayerChunk); ++layer) {
    for (int h = h0; h < Hkv; h += hs) {
      const int64_t src = ((layer * n_rows + row) * Hkv + h) * d;
      const int64_t dst = (((layer * capacity + phys) * Hkv + h) * B + slot) * d;
      uint16_t k1 = knew[src + i], k2 = knew[src + i + half];
      if (shift != 0) {
        float y1, y2;
        kvp::rope_apply(kvp::bf16_to_f32(k1), kvp::bf16_to_f32(k2), c, s, &y1, &y2);
        k1 = kvp::f32_to_bf16_rne(y1);
        k2 = kvp::f32_to_bf16_rne(y2);
      }
      kp[dst + i] = k1;
      kp[dst + i + half] = k2;
      vp[dst + i] = vnew[src + i];
      vp[dst + i + half] = vnew[src + i + half];
    }
  }
}

}  // namespace

extern "C" int kv_append(const kvp_shape* shape, void* k_pool, void* v_pool, int32_t capacity, const int32_t* copies,
                         int32_t n_copies, const int32_t* writes, int32_t n_writes, const void* k_new,
                         const void* v_new, int32_t n_rows, void* stream) {
  int rc = kvp::check_shape(shape);
  if (rc) return rc;
  if (shape->kv_dtype != KVP_BF16) return kvp::fail(KVP_EINVAL, "kv_append supports bf16 pools");
  if (capacity < 1 || n_copies < 0 || n_writes < 0 || n_rows < 0) return kvp::fail(KVP_EINVAL, "negative count or capacity");
  if ((n_copies > 0 || n_writes > 0) && (!k_pool || !v_pool)) return kvp::fail(KVP_EINVAL, "pool pointer is NULL");
  if (n_copies > 0 && !copies) return kvp::fail(KVP_EINVAL, "copies is NULL");
  if (n_writes > 0 && (!writes || !k_new || !v_new || n_rows < 1)) return kvp::fail(KVP_EINVAL, "writes or new rows missing");
  const int L = shape->n_layers, Hkv = shape->n_kv_heads, B = shape->block_tokens, d = shape->head_dim;
  if ((int64_t)n_copies * L > INT32_MAX || (int64_t)n_writes * (L + kLayerChunk - 1) / kLayerChunk > INT32_MAX)
    return kvp::fail(KVP_EINVAL, "too many operations");
  hipStream_t st = (hipStream_t)stream;
  const int64_t block_bytes = (int64_t)Hkv * B * d * 2;
  if (n_copies > 0)
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)(n_copies * L)), dim3(256), 0, st, (uint8_t*)k_pool,
                       (uint8_t*)v_pool, copies, n_copies, capacity, block_bytes);
  if (n_writes > 0) {
    const int chunks = (L + kLayerChunk - 1) / kLayerChunk;
    hipLaunchKernelGGL(write_tokens_kernel, dim3((unsigned)(n_writes * chunks)), dim3(256), 0, st, (uint16_t*)k_pool,
                       (uint16_t*)v_pool, writes, n_writes, (const uint16_t*)k_new, (const uint16_t*)v_new, n_rows,
                       capacity, L, Hkv, B, d, shape->rope_theta);
  }
  if (hipGetLastError() != hipSuccess) return kvp::fail(KVP_EHIP, "kv_append launch failed");
  return KVP_OK;
}
