/* Persistent Q4 block pool: save an agent's Q4 blocks to a file and reload them
 * into the pool (Q4 KV paper summary, sec. 2.1: each agent's cache is cut into
 * fixed 256-token blocks kept in 4-bit form in safetensors files that outlive a
 * restart, one namespace per agent; sec. 2.2: one agent's cache is loaded while
 * another agent decodes, which hides the load).
 *
 * The Q4 pool is the one paged_decode_attn reads (kvpool.h): codes
 * [n_layers][pool_blocks][Hkv][B][d/2] uint8, params [n_layers][pool_blocks]
 * [Hkv][B][d/64][2] fp16 (scale, zero), K and V apart.
 *
 * A host image of n blocks is four tensors back to back, each over all layers:
 *   k_codes  uint8 [n_layers][n][Hkv][B][d/2]
 *   v_codes  uint8 [n_layers][n][Hkv][B][d/2]
 *   k_params fp16  [n_layers][n][Hkv][B][d/64][2]
 *   v_params fp16  [n_layers][n][Hkv][B][d/64][2]
 * kv_q4_gather / kv_q4_scatter move blocks between the pool and an image with
 * DMA copies on the caller's stream (one 2-D copy per tensor and run of
 * consecutive block ids; the image should be pinned host memory for the copies
 * to be asynchronous).  A HIP error part-way leaves the copies enqueued before it
 * in place.  kvpool_q4_save_file / kvpool_q4_load_file move an image
 * to and from a file in the safetensors format: an 8-byte little-endian header
 * length, a JSON header naming each tensor's dtype, shape and byte range, then
 * the bytes.  The file also holds ntok (int32 [n], valid tokens per block) and,
 * in the header's metadata, the agent namespace and the shape.
 */
#ifndef KVPOOL_PERSIST_H
#define KVPOOL_PERSIST_H

#include "kvpool.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the image of n blocks for shape (kv_dtype must be KVP_Q4G64), or
 * KVP_EINVAL (bad shape, not Q4, n < 0). */
int64_t kvpool_q4_image_bytes(const kvp_shape* shape, int32_t n);

/* Device -> host: blocks ids[0..n) (host int32, each in [0, pool_blocks)) of
 * the four pool tensors into image (kvpool_q4_image_bytes(shape, n) bytes), in
 * the order of ids.  Asynchronous on stream.  Errors: KVP_EINVAL (bad shape,
 * not Q4, NULL pointer with n > 0, id out of range, n < 0), KVP_EHIP. */
int kv_q4_gather(const kvp_shape* shape, const void* k_codes, const void* v_codes, const void* k_params,
                 const void* v_params, int32_t pool_blocks, const int32_t* ids, int32_t n, void* image, void* stream);

/* Host -> device: the reverse; image block i goes to pool block ids[i].
 * Asynchronous on stream; the image must stay untouched until the copies end.
 * Two ids that are equal race.  Errors as kv_q4_gather. */
int kv_q4_scatter(const kvp_shape* shape, const void* image, int32_t n, void* k_codes, void* v_codes, void* k_params,
                  void* v_params, int32_t pool_blocks, const int32_t* ids, void* stream);

/* Writes image (n blocks) and ntok (host int32 [n], each in [0, B]) as a
 * safetensors file at path (created or truncated), with agent (a namespace
 * string without control characters or quotes, at most 255 bytes) and the
 * shape in its metadata.  Synchronous.  Errors: KVP_EINVAL (bad shape, not Q4,
 * NULL pointer, n < 1, ntok out of range, bad agent string; nothing written),
 * KVP_ENOMEM (nothing written), KVP_EIO (the file may be left partly written). */
int kvpool_q4_save_file(const kvp_shape* shape, const char* path, const char* agent, const void* image,
                        const int32_t* ntok, int32_t n);

/* Reads a file written by kvpool_q4_save_file (or any safetensors file holding
 * tensors k_codes, v_codes, k_params, v_params and ntok of this shape, in any
 * order in the file).  Returns the number of blocks n.  The tensors are read
 * into image and ntok only when image_bytes >= kvpool_q4_image_bytes(shape, n)
 * and max_blocks >= n (image NULL and max_blocks 0 ask for n).  If agent is
 * not NULL the file's metadata must name the same agent (one namespace per
 * agent), else KVP_EINVAL.  Synchronous.  Errors: KVP_EINVAL (bad shape, not
 * Q4, tensors missing or of another shape or dtype, agent mismatch, n != the
 * tensors' block count, ntok out of range; image and ntok untouched), KVP_EIO
 * (cannot open or read; header malformed; a read that fails after the header
 * was checked may leave the image partly written, ntok untouched), KVP_ENOMEM
 * (image and ntok untouched). */
int kvpool_q4_load_file(const kvp_shape* shape, const char* path, const char* agent, void* image,
                        int64_t image_bytes, int32_t* ntok, int32_t max_blocks);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_PERSIST_H */
