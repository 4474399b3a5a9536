/*
 * kvpool.h -- C ABI of the deduplicated paged KV pool and its decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * One decode step of attention for many agents whose KV caches share blocks:
 *   1. kvpool_build_tables  (host)   fingerprint dedup + refcounts -> block tables,
 *                                    master/mirror delta overlay, RoPE shifts, and
 *                                    the device work plan.
 *   2. kv_rerotate          (device) batched RoPE re-rotation of K or Q rows.
 *   3. paged_decode_attn    (device) decode attention over the pool (online softmax,
 *                                    GQA, delta overlay and Q4 dequantisation fused
 *                                    into the load, split-KV merge).
 *
 * Conventions for every entry point:
 *   - returns 0 (KVP_OK) or a negative kvp_status; never throws, never aborts;
 *     kvpool_last_error() gives a thread-local message for the last failure;
 *   - on error, outputs are left untouched;
 *   - "device" pointers are HIP device allocations owned by the caller; the
 *     library never allocates, frees or synchronises device memory;
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream); device
 *     entry points only enqueue work on it and return.
 */
#ifndef KVPOOL_H
#define KVPOOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvp_status {
  KVP_OK = 0,
  KVP_EINVAL = -1,     /* bad shape, range, ordering or null pointer            */
  KVP_ETIER = -2,      /* a GROUP span without a group id (group < 0)           */
  KVP_ENOMEM = -3,     /* host allocation failed                                */
  KVP_EWORKSPACE = -4, /* workspace too small                                   */
  KVP_EHIP = -5,       /* a HIP launch or runtime error                         */
  KVP_EFULL = -6,      /* the pool has no free physical block (lifecycle calls) */
  KVP_EIO = -7         /* a file could not be opened, read or written, or is
                          malformed (persistence calls)                          */
} kvp_status;

/* element types */
enum { KVP_BF16 = 0, KVP_Q4G64 = 1, KVP_F32 = 2 };
/* memory tiers (INMS walkthrough, sec. 2.1: global read-only, group shared, private) */
enum { KVP_GLOBAL = 0, KVP_GROUP = 1, KVP_PRIVATE = 2 };
/* span kinds: PREFIX continues the chain of the block before it; SEGMENT restarts
 * it, so its blocks are indexed by their own content wherever they are placed
 * (TokenDance write-up, sec. 1: segment hashing behind a separator token). */
enum { KVP_PREFIX = 0, KVP_SEGMENT = 1 };

/* Model-agnostic cache shape (Q4 KV paper summary, sec. 3: a cache spec per model).
 * n_q_heads % n_kv_heads == 0 (q head h reads kv head h / (n_q_heads/n_kv_heads));
 * head_dim in {64, 128}; block_tokens in {16, 256}; kv_dtype KVP_BF16 or
 * KVP_Q4G64; rope_theta > 0 is the RoPE base. */
typedef struct kvp_shape {
  int32_t n_layers, n_q_heads, n_kv_heads, head_dim, block_tokens, kv_dtype;
  float rope_theta;
} kvp_shape;

/* A run of tokens with one tier and kind.  group is the group id of a GROUP span
 * (ignored otherwise).  tokens: host array of n_tokens ids, borrowed for the call. */
typedef struct kvp_span {
  int32_t tier, group, kind, n_tokens;
  const int32_t* tokens;
} kvp_span;

/* One agent (one decode sequence): its spans in order, and the logical block
 * indices (strictly increasing) that its mirror replaces with a delta block.  A
 * delta may only replace a block of a SEGMENT span of a shared tier (TokenDance
 * write-up, sec. 3: mirrors are block-sparse differences against the master). */
typedef struct kvp_agent {
  int32_t n_spans;
  const kvp_span* spans;
  int32_t n_delta;
  const int32_t* delta_blocks;
} kvp_agent;

/* One unit of decode work: a chunk of physical blocks read by a set of consumers
 * (agent, shift).  The tile pass runs one workgroup per (item, kv head) unit in a
 * one-dimensional grid; units are dealt over the 8 XCDs so that the units of one
 * kv head (when n_kv_heads is a multiple of 8), or a window of consecutive items
 * over the same blocks (otherwise), stay on one XCD and share its L2. */
typedef struct kvp_item {
  int32_t blk_begin, blk_end;   /* range in plan_blocks                          */
  int32_t cons_begin, cons_end; /* range in cons                                 */
  int32_t part_base;            /* first partial row (per kv head) it writes     */
  int32_t mask_base;            /* first mask word, or -1: all consumers read all blocks */
  int32_t mask_stride;          /* mask words per block                          */
  int32_t rows;                 /* (cons_end - cons_begin) * (n_q_heads / n_kv_heads);
                                   up to 16, or up to 128 (at most 64 consumers) for
                                   bf16 blocks read by many consumers (the
                                   matrix-core "wide" items)                        */
} kvp_item;

typedef struct kvp_tables kvp_tables; /* opaque, owned by the library */

/* Borrowed views of every array of a kvp_tables (valid until kvpool_tables_free).
 * Table arrays are [n_agents][max_blocks] int32, row-major, padded with -1 (ids)
 * or 0 (ntok, dst_pos0, shift). */
typedef struct kvp_tables_view {
  int32_t n_agents, max_blocks, n_phys, n_dedup, n_delta;
  const int32_t* n_blocks;    /* [n_agents] logical blocks per agent                   */
  const int32_t* block_table; /* dedup physical id of each logical block               */
  const int32_t* delta_table; /* delta physical id overlaying it, or -1                 */
  const int32_t* ntok;        /* valid tokens of the logical block                     */
  const int32_t* dst_pos0;    /* logical start position in the agent's sequence        */
  const int32_t* shift;       /* dst_pos0 - src_pos0[block_table]                       */
  const int32_t* src_pos0;    /* [n_phys] position of the stored frame                 */
  const int32_t* refcount;    /* [n_phys] effective references                         */
  const int32_t* phys_ntok;   /* [n_phys] valid tokens of the physical block           */
  const int32_t* phys_agent;  /* [n_phys] agent of the first occurrence (delta: owner) */
  const int32_t* phys_block;  /* [n_phys] its logical block index                      */
  /* work plan (device copies of these arrays form a kvp_plan_dev) */
  int32_t n_items, n_plan_blocks, n_cons, n_qcons, n_mask_words, n_part_rows, n_comb;
  const kvp_item* items;       /* [n_items]                                           */
  const int32_t* plan_blocks;  /* [n_plan_blocks] physical ids                         */
  const int32_t* cons;         /* [n_cons] index into qcons                            */
  const int32_t* qcons;        /* [n_qcons][2] (agent, shift), unique pairs; the
                                  n_qcons_shifted pairs with shift != 0 come last       */
  const uint32_t* mask;        /* [n_mask_words] bit c of a block's word(s): consumer c reads it */
  const int32_t* comb_ptr;     /* [n_agents + 1] CSR over comb_rows                    */
  const int32_t* comb_rows;    /* [n_comb] partial row (for the group's first q head)  */
  int32_t n_qcons_shifted;
  int32_t class_items[6];      /* how many items have rows in (16,128], (8,16], (4,8],
                                  (2,4], (1,2] and exactly 1 (items are in dispatch
                                  order: more rows first; a plan without wide items
                                  ends with short items split off its last quarter)  */
  int32_t unit_span;           /* (item, kv head) units of consecutive items that read
                                  the same blocks; kept on one XCD per dispatch window  */
  int64_t unique_kv_bytes;     /* bytes of valid tokens in the pool, per layer         */
  /* lookups derived from the arrays above, so that the device reaches a block's
     token count and a consumer's query row in one load */
  const int32_t* plan_ntok;    /* [n_plan_blocks] phys_ntok[plan_blocks[i]]            */
  const int32_t* cons_row;     /* [n_cons] row of consumer cons[i]'s query: its agent
                                  (rows of q) if unshifted, else cons[i] minus the
                                  number of unshifted pairs (its row of rope_cs)      */
  const float* rope_cs;        /* [n_qcons_shifted][head_dim/2][2] float32 (cos, sin) of
                                  -shift * theta_i, theta_i = rope_theta^(-2i/head_dim),
                                  for the shifted pairs in qcons order: the rotation
                                  R(-shift) applied to their queries (INMS walkthrough
                                  sec. 3.2); the angle is formed in double           */
  int32_t n_rope_cs;           /* floats in rope_cs: n_qcons_shifted * head_dim          */
} kvp_tables_view;

/* Device copy of the work plan: every pointer is a device array holding exactly
 * the corresponding kvp_tables_view array; counts copied from the view. */
typedef struct kvp_plan_dev {
  int32_t n_agents, n_phys, n_items, n_qcons, n_qcons_shifted, n_part_rows;
  int32_t class_items[6];
  int32_t unit_span;
  const kvp_item* items;
  const int32_t* plan_blocks;
  const int32_t* cons;
  const int32_t* qcons;
  const uint32_t* mask;
  const int32_t* phys_ntok;
  const int32_t* comb_ptr;
  const int32_t* comb_rows;
  const int32_t* plan_ntok;
  const int32_t* cons_row;
  const float* rope_cs;  /* may be NULL when n_qcons_shifted is 0 */
  /* extents of the arrays above (copied from the view), read by the kernels'
     bounds checks in the checked build (kvpool_device_checks_enabled) */
  int32_t n_plan_blocks, n_cons, n_mask_words, n_comb;
} kvp_plan_dev;

/* kvpool_build_tables (host, synchronous).
 * Follows: INMS walkthrough sec. 2.2 (fixed blocks, content fingerprint looked up
 * in the pool of the block's tier, hit -> reuse and refcount + 1, miss -> new
 * block) and sec. 3.2 (tier must match); TokenDance write-up sec. 1 (segments
 * indexed by content) and sec. 3 (master plus block-sparse mirrors); the
 * shared-memory prefix cache blog sec. 3.2 (FNV-1a over token ids).
 * Every span starts a new block; a block's key is (tier, group, [agent, span] if
 * PRIVATE, predecessor's physical id or the SEGMENT root, tokens); keys are
 * hashed with word-wise FNV-1a-64 and confirmed by exact comparison.  Physical
 * ids follow first occurrence (agents in order, blocks in order); delta ids follow
 * all dedup ids in (agent, block) order; refcount counts effective references
 * (an overlaid entry does not count toward its master, the copy-on-write
 * decrement); a delta is stored in its master's frame.
 * Also builds the work plan for `shape` (head counts, block size, dtype).
 * shape, agents: host, borrowed.  *out: library-owned, free with
 * kvpool_tables_free.  Errors: KVP_EINVAL (null pointer, bad shape, negative
 * length, unknown tier/kind, delta index out of range / not increasing / not on a
 * shared SEGMENT block), KVP_ETIER, KVP_ENOMEM. */
int kvpool_build_tables(const kvp_shape* shape, const kvp_agent* agents, int32_t n_agents,
                        kvp_tables** out);

/* Fills *v with borrowed pointers into t.  KVP_EINVAL if either is NULL. */
int kvpool_tables_view(const kvp_tables* t, kvp_tables_view* v);

/* Frees t (NULL is a no-op). */
void kvpool_tables_free(kvp_tables* t);

/* kv_rerotate (device, asynchronous): batched RoPE offset compensation.
 * INMS walkthrough sec. 2.3 / 3.2: a stored key moved from position a to b is
 * rotated by an angle that depends on b - a only; V is never rotated.
 * TokenDance write-up sec. 2: one batched rotation call for all requests.
 * y[r, h, :] = R(shift[r]) x[r, h, :] with rotate-half pairs (i, i + d/2),
 * theta_i = rope_theta^(-2i/d), angle shift * theta_i formed in float64; the
 * rotation itself in float32; bf16 output rounded to nearest even.
 * x, y: device [n_rows][n_heads][head_dim] of in_dtype / out_dtype (KVP_BF16 or
 * KVP_F32); x == y allowed when the dtypes match.  shift: device int32 [n_rows].
 * Errors: KVP_EINVAL (null pointer, n_rows < 0, n_heads < 1, head_dim odd or
 * > 512, dtype), KVP_EHIP. */
int kv_rerotate(const void* x, void* y, const int32_t* shift, int64_t n_rows, int32_t n_heads,
                int32_t head_dim, float rope_theta, int32_t in_dtype, int32_t out_dtype, void* stream);

/* Workspace bytes paged_decode_attn needs for this shape and plan. */
int paged_decode_attn_workspace_bytes(const kvp_shape* shape, const kvp_plan_dev* plan, size_t* bytes);

/* paged_decode_attn (device, asynchronous): one decode step of attention for every
 * agent of the plan at one layer.
 * Attention as in the MemDecay blog sec. 4.2: scores q.k * scale (scale normally
 * 1/sqrt(head_dim)), float32 softmax, weighted sum of V; GQA contiguous groups.
 * Each agent attends to all of its cached tokens.  Delta blocks replace their
 * master block for their owner only (TokenDance write-up sec. 3, fused into the
 * load); a consumer with shift s reads the stored K as R(s) K, computed as
 * (R(-s) q) . K (INMS walkthrough sec. 3.2); Q4 blocks are dequantised in the
 * kernel as s * c + z per group of 64 (Q4 KV paper summary sec. 2.2).
 * q: device bf16 [n_agents][n_q_heads][head_dim], post-RoPE at the current position.
 * k_pool, v_pool (KVP_BF16): device bf16 [n_layers][n_phys][n_kv_heads][block_tokens][head_dim].
 * k_pool, v_pool (KVP_Q4G64): device uint8 codes [n_layers][n_phys][n_kv_heads][block_tokens][head_dim/2]
 *   (even element in the low nibble); k_params, v_params: device float16
 *   [n_layers][n_phys][n_kv_heads][block_tokens][head_dim/64][2] = (scale, zero);
 *   NULL for KVP_BF16.  Slots beyond a block's valid tokens are never read into
 *   the result (they may hold NaN).
 * out: device float32 [n_agents][n_q_heads][head_dim]; an agent with no cached
 *   tokens gets zeros.
 * workspace: device, at least paged_decode_attn_workspace_bytes; its contents on
 *   entry do not matter.  plan: host struct of device pointers (kvp_plan_dev),
 *   built from the kvp_tables_view of the same shape.
 * A pointer the call does not use may be NULL: all of them when the plan has no
 * agents (nothing is launched), the pools and params when it has no work items
 * (every agent is empty: out is zero-filled), the workspace when its size is 0.
 * Errors: KVP_EINVAL (a used pointer is NULL, bad shape, layer out of range, bad
 * plan counts), KVP_EWORKSPACE, KVP_EHIP. */
int paged_decode_attn(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q,
                      const void* k_pool, const void* v_pool, const void* k_params,
                      const void* v_params, int32_t layer, float scale, float* out,
                      void* workspace, size_t ws_bytes, void* stream);

/* paged_decode_attn_phases: the work of paged_decode_attn restricted to the phases
 * set in `phases` -- bit 2: tile pass (writes the partials into the workspace),
 * bit 4: combine (merges the partials into out).  Bit 1 (query preparation) is
 * accepted and launches nothing: a shifted consumer's query is rotated by the
 * tile pass as it loads it, with the plan's rope_cs.  Calling it with 1, then 2,
 * then 4 on one stream with the same workspace does exactly what one
 * paged_decode_attn call does; it lets a caller time or schedule the phases
 * apart.  Same arguments and errors as paged_decode_attn, plus KVP_EINVAL for
 * phases outside 1..7. */
int paged_decode_attn_phases(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q,
                             const void* k_pool, const void* v_pool, const void* k_params,
                             const void* v_params, int32_t layer, float scale, float* out,
                             void* workspace, size_t ws_bytes, uint32_t phases, void* stream);

/* Bytes of the library's own per-device scratch array (128 MiB): the largest
 * workspace paged_decode_attn_noalloc can serve. */
#define KVP_NOALLOC_SCRATCH_BYTES (128u << 20)

/* paged_decode_attn_noalloc: paged_decode_attn without a workspace argument and
 * without any device allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a static device array of the library
 * (KVP_NOALLOC_SCRATCH_BYTES, one per device, held from the first use of the
 * library's kernels on that device until the process ends); its address is
 * looked up once per device.  Calls on one device share that array: calls that
 * overlap on one device (several streams or host threads) race and must be
 * serialised by the caller; stream order suffices.  Nothing in it needs to be
 * zero on entry (the call overwrites what it reads).  Same arguments, results
 * and errors as paged_decode_attn, plus KVP_EWORKSPACE when the plan needs more
 * than KVP_NOALLOC_SCRATCH_BYTES (paged_decode_attn_workspace_bytes tells), and
 * KVP_EHIP when the array's address cannot be looked up.  Calls no hipMalloc,
 * hipFree or other allocating routine. */
int paged_decode_attn_noalloc(const kvp_shape* shape, const kvp_plan_dev* plan, const void* q,
                              const void* k_pool, const void* v_pool, const void* k_params,
                              const void* v_params, int32_t layer, float scale, float* out, void* stream);

/* Checked build (test hooks).  The library built with device-side bounds checks
 * (libkvpool_checked.so) tests, in every tile-pass workgroup before it touches a
 * pool, the query or the workspace, that its item's block, consumer, partial-row
 * and mask ranges lie inside the plan's arrays, that every physical id and valid
 * token count it will read is in range, and that every consumer's query row is;
 * the combine tests its agent's entries the same way.  A workgroup or wave that
 * finds a violation sets a bit in a per-device error word (1: item ranges,
 * 2: block ids or token counts, 4: consumers, 8: combine lists) and returns
 * without reading or writing anything else.  The ordinary build has no checks.
 * kvpool_device_checks_enabled: 1 in the checked build, 0 otherwise.
 * kvpool_debug_take_device_errors (device, asynchronous): copies the current
 * device's error word to *dst (device uint32) and clears it, on `stream`.
 * Errors: KVP_EINVAL (dst NULL), KVP_EHIP. */
int kvpool_device_checks_enabled(void);
int kvpool_debug_take_device_errors(uint32_t* dst, void* stream);

/* Thread-local message describing the last non-zero status ("" if none). */
const char* kvpool_last_error(void);

/* Word-wise FNV-1a-64 (shared-memory prefix cache blog, sec. 3.2: offset basis
 * 1469598103934665603, prime 1099511628211, one 32-bit token id per step) over
 * n words of w (host).  Exposed for tests. */
uint64_t kvpool_fnv1a64_words(const uint32_t* w, int64_t n);

/* Test hook: keep only the low `bits` bits (1..64) of every fingerprint, which
 * forces hash collisions; tables must not change.  Process-wide; returns
 * KVP_EINVAL outside 1..64. */
int kvpool_debug_set_hash_bits(int32_t bits);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_H */
