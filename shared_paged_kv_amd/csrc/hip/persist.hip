// Persistent Q4 block pool, device side: moves blocks between the Q4 pool and a
// host image with DMA copies (include/kvpool_persist.h).  Q4 KV paper summary,
// sec. 2.2: one agent's cache is loaded while another agent decodes; these
// copies run on the copy engines, so a load issued on its own stream overlaps
// the decode's kernels.
//
// Per tensor (K codes, V codes, K params, V params) a block is one contiguous
// run per layer; the ids are cut into runs of consecutive physical ids and each
// run of each tensor is one 2-D copy over the layers (the image's layer pitch
// is n blocks, the pool's is pool_blocks).
#include <hip/hip_runtime.h>


#include "../host/kvpool_internal.h"
#include "kvpool.h"
#include "kvpool_persist.h"

namespace {

struct Plan {
  int64_t blk[4];    // bytes per block and layer of each tensor
  int64_t off[4];    // offset of each tensor in the image
  int L = 0;
};

int make_plan(const kvp_shape* s, int32_t n, int32_t pool_blocks, const int32_t* ids, Plan* p) {
  const int64_t bytes = kvpool_q4_image_bytes(s, n);
  if (bytes < 0) return (int)bytes;
  if (pool_blocks < 1 || (n > 0 && !ids)) return kvp::fail(KVP_EINVAL, "pool_blocks < 1 or ids NULL");
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= pool_blocks) return kvp::fail(KVP_EINVAL, "block id out of range");
  const int64_t cb = (int64_t)s->n_kv_heads * s->block_tokens * (s->head_dim / 2);
  const int64_t pb = (int64_t)s->n_kv_heads * s->block_tokens * (s->head_dim / 64) * 4;
  p->L = s->n_layers;
  p->blk[0] = p->blk[1] = cb;
  p->blk[2] = p->blk[3] = pb;
  p->off[0] = 0;
  p->off[1] = cb * n * p->L;
  p->off[2] = 2 * cb * n * p->L;
  p->off[3] = 2 * cb * n * p->L + pb * n * p->L;
  return KVP_OK;
}

// One copy of a run: r blocks from image block i / pool block id, every layer.
hipError_t copy_run(bool to_pool, uint8_t* pool, uint8_t* img, int64_t blk, int64_t n, int64_t pool_blocks, int L,
                    int64_t i, int64_t id, int64_t r, hipStream_t st) {
  uint8_t* dp = pool + id * blk;
  uint8_t* hp = img + i * blk;
  const size_t w = (size_t)(r * blk), hpitch = (size_t)(n * blk), dpitch = (size_t)(pool_blocks * blk);
  const hipMemcpyKind kind = to_pool ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  if (L == 1) return hipMemcpyAsync(to_pool ? dp : hp, to_pool ? hp : dp, w, kind, st);
  if (dpitch <= (size_t)INT32_MAX && hpitch <= (size_t)INT32_MAX)
    return to_pool ? hipMemcpy2DAsync(dp, dpitch, hp, hpitch, w, (size_t)L, kind, st)
                   : hipMemcpy2DAsync(hp, hpitch, dp, dpitch, w, (size_t)L, kind, st);
  for (int l = 0; l < L; ++l) {
    hipError_t e = hipMemcpyAsync(to_pool ? dp + l * dpitch : hp + l * hpitch, to_pool ? hp + l * hpitch : dp + l * dpitch,
                                  w, kind, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int move(bool to_pool, const kvp_shape* s, int32_t n, void* const pools[4], int32_t pool_blocks, const int32_t* ids,
         void* image, void* stream) {
  Plan p;
  int rc = make_plan(s, n, pool_blocks, ids, &p);
  if (rc) return rc;
  if (n == 0) return KVP_OK;
  if (!image) return kvp::fail(KVP_EINVAL, "image is NULL");
  for (int t = 0; t < 4; ++t)
    if (!pools[t]) return kvp::fail(KVP_EINVAL, "a pool pointer is NULL");
  hipStream_t st = (hipStream_t)stream;
  for (int32_t i = 0; i < n;) {
    int32_t r = 1;
    while (i + r < n && ids[i + r] == ids[i] + r) ++r;
    for (int t = 0; t < 4; ++t) {
      hipError_t e = copy_run(to_pool, (uint8_t*)pools[t], (uint8_t*)image + p.off[t], p.blk[t], n, pool_blocks, p.L,
                              i, ids[i], r, st);
      if (e != hipSuccess) return kvp::fail(KVP_EHIP, hipGetErrorString(e));
    }
    i += r;
  }
  return KVP_OK;
}

}  // namespace

extern "C" int kv_q4_gather(const kvp_shape* shape, const void* k_codes, const void* v_codes, const void* k_params,
                            const void* v_params, int32_t pool_blocks, const int32_t* ids, int32_t n, void* image,
                            void* stream) {
  void* const pools[4] = {(void*)k_codes, (void*)v_codes, (void*)k_params, (void*)v_params};
  return move(false, shape, n, pools, pool_blocks, ids, image, stream);
}

extern "C" int kv_q4_scatter(const kvp_shape* shape, const void* image, int32_t n, void* k_codes, void* v_codes,
                             void* k_params, void* v_params, int32_t pool_blocks, const int32_t* ids, void* stream) {
  void* const pools[4] = {k_codes, v_codes, k_params, v_params};
  return move(true, shape, n, pools, pool_blocks, ids, (void*)image, stream);
}
