/* Block lifecycle of the deduplicated pool: decode-time append with
 * copy-on-write, sequence destruction, and a reference-leak audit.
 *
 * The INMS walkthrough (sec. 2.2) gives the rules: shared blocks are read-only;
 * a sequence that writes into a block whose reference count is above one gets
 * a private copy first (the old block's count drops by one), else it writes in
 * place; a count that reaches zero returns the block to the pool.  Sec. 3.3
 * gives the three engine-facing calls (register a sequence, write KV blocks
 * through the dedup logic, destroy a sequence: decrement its blocks' counts and
 * reclaim), and sec. 5.3 the failure mode this header also covers: an agent
 * that exits without its destroy call leaks its references until a scan finds
 * them and a forced reclamation returns them.
 *
 * Host state lives in an opaque kvp_pool (library-owned).  Device memory stays
 * the caller's: the pool tensors [L][capacity][Hkv][B][d] (bf16), the new
 * token rows, and the device copies of the operation lists.
 *
 * Readings taken where the pages are silent:
 *  - one appended token goes to the agent's last logical block while it has
 *    room, else to a new logical block whose first position follows the last;
 *  - a copy-on-write copy keeps the source's stored frame (src_pos0) and bytes;
 *    a new block's frame is its own first logical position (shift 0);
 *  - the token's K arrives post-RoPE at its logical position and is stored in
 *    the block's frame: bf16(R(-shift) k), round to nearest even; V as given;
 *  - a freed physical id is reused smallest first, otherwise the smallest id
 *    never allocated, below the pool's capacity;
 *  - an entry overlaid by a delta block writes into the delta (count 1).
 */
#ifndef KVPOOL_LIFECYCLE_H
#define KVPOOL_LIFECYCLE_H

#include "kvpool.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvp_pool kvp_pool; /* opaque, owned by the library */

/* Device work of one kvpool_append call, in host memory owned by the pool
 * (valid until the next call on it).  copies[2i] -> copies[2i+1]: whole-block
 * copies (every layer, kv head, slot, K and V), to run before any write.
 * writes[4i..4i+3] = (physical id, slot, new-row index, shift): new row r of
 * the caller's arrays goes to slot of the block, its K rotated by -shift. */
typedef struct kvp_append_ops {
  int32_t n_copies;
  const int32_t* copies;
  int32_t n_writes;
  const int32_t* writes;
} kvp_append_ops;

/* Result of kvpool_audit.  A block is allocated from its first use until it
 * is freed; its recount is the number of live agents' effective references. */
typedef struct kvp_audit {
  int32_t n_allocated;    /* allocated physical blocks                       */
  int32_t n_leaked;       /* allocated, refcount > 0, recount == 0            */
  int32_t n_mismatched;   /* allocated, refcount != recount (leaked included) */
  int32_t n_live_agents;
  int64_t leaked_tokens;  /* valid tokens held by the leaked blocks           */
} kvp_audit;

/* Creates a pool from built tables (copied; t may be freed afterwards) with
 * room for capacity physical blocks (capacity >= the tables' n_phys).
 * Errors: KVP_EINVAL (null pointer, capacity too small), KVP_ENOMEM. */
int kvpool_pool_create(const kvp_tables* t, const kvp_shape* shape, int32_t capacity, kvp_pool** out);
void kvpool_pool_free(kvp_pool* pool);

/* Appends one token to each listed agent, in list order (an agent listed k
 * times gets k tokens); the token of agents[i] is new row i.  All or nothing:
 * on error the pool is unchanged.  Errors: KVP_EINVAL (null pointer, n < 0,
 * agent out of range or not live), KVP_EFULL (not enough free blocks for the
 * copies and new blocks the call needs), KVP_ENOMEM. */
int kvpool_append(kvp_pool* pool, int32_t n, const int32_t* agents, kvp_append_ops* ops);

/* Destroys a live agent: each effective reference is released; blocks reaching
 * zero are freed.  Errors: KVP_EINVAL (out of range or not live). */
int kvpool_destroy(kvp_pool* pool, int32_t agent);

/* Marks a live agent as lost (it exited without its destroy call): its table is
 * dropped and its references are left in place -- a leak, for kvpool_audit to
 * find.  Errors: KVP_EINVAL (out of range or not live). */
int kvpool_lose(kvp_pool* pool, int32_t agent);

/* Recounts the live agents' references against the stored counts.  If ids is
 * not NULL, the ids of up to max_ids leaked blocks are written to it, ascending.
 * Errors: KVP_EINVAL (null pool or audit, max_ids < 0). */
int kvpool_audit(const kvp_pool* pool, kvp_audit* audit, int32_t* ids, int32_t max_ids);

/* Forced reclamation: every stored count becomes its recount and the blocks at
 * zero are freed.  Returns the number of blocks freed (>= 0) or KVP_EINVAL. */
int kvpool_reclaim(kvp_pool* pool);

/* Snapshot of the pool's current tables and work plan, for paged_decode_attn
 * on the pool tensors [L][capacity][Hkv][B][d]: n_phys is the capacity (free
 * ids have refcount 0 and no valid tokens; dead agents have no blocks;
 * phys_agent/phys_block are -1 for blocks created by the lifecycle calls).
 * Free with kvpool_tables_free.  Errors: KVP_EINVAL, KVP_ENOMEM. */
int kvpool_pool_tables(const kvp_pool* pool, kvp_tables** out);

/* Runs one kvpool_append's device work on a bf16 pool: first every block copy
 * (all layers and kv heads), then every token write.  k_pool, v_pool: device
 * [n_layers][capacity][Hkv][B][d] bf16.  copies, writes: device copies of the
 * ops' arrays.  k_new, v_new: device [n_layers][n_rows][Hkv][d] bf16, the new
 * tokens' K post-RoPE at their logical positions and V.  Enqueued on stream.
 * Errors: KVP_EINVAL (null pointer with a non-zero count, bad shape, kv_dtype
 * not bf16, negative counts or capacity), KVP_EHIP. */
int kv_append(const kvp_shape* shape, void* k_pool, void* v_pool, int32_t capacity, const int32_t* copies,
              int32_t n_copies, const int32_t* writes, int32_t n_writes, const void* k_new, const void* v_new,
              int32_t n_rows, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_LIFECYCLE_H */
