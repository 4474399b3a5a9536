/* Master/mirror storage, the two device steps around the decode read
 * (TokenDance write-up, sec. 3): one dense master cache, every other agent a
 * mirror = a reference to the master plus block-sparse differences.
 *
 *  - kv_diff_blocks (diff construction): flags the candidate blocks of the
 *    mirrors that differ from their master block, so that only those become
 *    delta blocks (the write-up, sec. 3: differences cluster in contiguous
 *    blocks; sec. 2: the cached values that differ from the new ones).
 *  - kv_restore (fused diff restore): materialises agents' contexts into paged
 *    buffers in one pass -- each logical block is read once from its delta
 *    block if it has one, else from the master block, its K is moved to the
 *    agent's positions (RoPE offset compensation), and it is written once.
 *    The write-up contrasts this with loading the master, copying it and then
 *    overwriting the differing blocks (sec. 3, fused restore).
 *
 * Device buffers are the caller's; both calls enqueue on the stream and return.
 * Layouts: a pool is [n_layers][pool_blocks][Hkv][B][d] bf16 (K and V apart).
 */
#ifndef KVPOOL_MIRROR_H
#define KVPOOL_MIRROR_H

#include "kvpool.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Diff construction.  pairs: device int32 [n][3] = (master physical id in the
 * pool, candidate block index in cand, valid tokens); cand_k / cand_v: device
 * [n_layers][cand_blocks][Hkv][B][d] bf16, the mirrors' blocks in the master's
 * stored frame.  flags[i] (device int32) becomes 1 if some valid token of pair
 * i differs in K or V in some layer and kv head, else 0: with tau == 0 a value
 * differs when its bits differ; with tau > 0 when |cand - master| > tau (float32,
 * a NaN on either side differs).  Padding slots are not compared.  Entries with
 * an id or token count out of range get flag -1.
 * Errors: KVP_EINVAL (null pointer with n > 0, bad shape, kv_dtype not bf16,
 * n < 0, tau < 0 or not finite, non-positive block counts), KVP_EHIP. */
int kv_diff_blocks(const kvp_shape* shape, const void* k_pool, const void* v_pool, int32_t pool_blocks,
                   const void* cand_k, const void* cand_v, int32_t cand_blocks, const int32_t* pairs, int32_t n,
                   float tau, int32_t* flags, void* stream);

/* Fused restore.  blocks: device int32 [n][3] = (physical id in the pool, shift,
 * valid tokens) for destination blocks 0..n-1 of dst_k / dst_v ([n_layers][n]
 * [Hkv][B][d] bf16): destination block i receives the valid tokens of the
 * source block, K rotated by R(shift) (float64 angle, float32 rotation,
 * round to nearest even), V as stored; its padding slots are zeroed.
 * kvpool_restore_list fills these entries for one agent.  Entries out of range
 * are skipped.  Errors: KVP_EINVAL (null pointer with n > 0, bad shape,
 * kv_dtype not bf16, n < 0, pool_blocks < 1), KVP_EHIP. */
int kv_restore(const kvp_shape* shape, const void* k_pool, const void* v_pool, int32_t pool_blocks,
               const int32_t* blocks, int32_t n, void* dst_k, void* dst_v, void* stream);

/* Host: the restore entries of agent j from built tables, one per logical block
 * in order: (effective physical id = delta if present else block, shift, valid
 * tokens) into out[3*i..3*i+2].  Returns the number of logical blocks (also
 * when it exceeds max_blocks, in which case only max_blocks entries are
 * written) or KVP_EINVAL (null tables, agent out of range, max_blocks < 0 or
 * out NULL with max_blocks > 0). */
int kvpool_restore_list(const kvp_tables* t, int32_t agent, int32_t* out, int32_t max_blocks);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_MIRROR_H */
