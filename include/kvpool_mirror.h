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
 * an id or token count out of range get flag -1.  Pairs that name the same
 * master should be adjacent: the master is then read once for up to 8 of them.
 * Errors: KVP_EINVAL (null pointer with n > 0, bad shape, kv_dtype not bf16,
 * n < 0, tau < 0 or not finite, non-positive block counts), KVP_EHIP. */
int kv_diff_blocks(const kvp_shape* shape, const void* k_pool, const void* v_pool, int32_t pool_blocks,
                   const void* cand_k, const void* cand_v, int32_t cand_blocks, const int32_t* pairs, int32_t n,
                   float tau, int32_t* flags, void* stream);

/* Fused restore.  entries: device int32 [n][4] = (physical id in the pool,
 * shift, valid tokens, destination block); dst_k / dst_v: device [n_layers]
 * [dst_blocks][Hkv][B][d] bf16.  The destination block of each entry receives
 * the valid tokens of the source block, K rotated by R(shift) (float64 angle,
 * float32 rotation, round to nearest even), V as stored; its padding slots are
 * zeroed.  Entries with an id, token count or destination out of range are
 * skipped; two entries with one destination race.  Entries that share (source,
 * valid tokens) should be adjacent: the source is then read once for up to 8
 * destinations.  kvpool_restore_list orders them so.  Errors: KVP_EINVAL (null
 * pointer with n > 0, bad shape, kv_dtype not bf16, n < 0, non-positive block
 * counts), KVP_EHIP. */
int kv_restore(const kvp_shape* shape, const void* k_pool, const void* v_pool, int32_t pool_blocks,
               const int32_t* entries, int32_t n, void* dst_k, void* dst_v, int32_t dst_blocks, void* stream);

/* Host: the restore entries of the listed agents from built tables.  Destination
 * blocks are numbered in list order, each agent's logical blocks in order
 * (agent agents[0] takes 0..n_blocks-1, the next agent follows); an entry is
 * (effective physical id = delta if present else block, shift, valid tokens,
 * destination).  The entries are ordered by (source, valid tokens, shift), ties
 * in destination order.  Returns the number of entries; writes them only when
 * max_entries is at least that number (so max_entries = 0 asks for the size).
 * Errors: KVP_EINVAL (null tables, agent out of range, n_agents < 0, agents
 * NULL with n_agents > 0, max_entries < 0, out NULL with max_entries > 0),
 * KVP_ENOMEM. */
int kvpool_restore_list(const kvp_tables* t, const int32_t* agents, int32_t n_agents, int32_t* out,
                        int32_t max_entries);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_MIRROR_H */
