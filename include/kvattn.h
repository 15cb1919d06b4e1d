/*
 * kvattn.h - C ABI of a gfx950 (MI355X) KV-cache attention library.
 *
 * The library computes scaled dot-product attention of new query tokens
 * against one layer's KV cache,
 *     out = softmax(Q K^T * scale + mask) V,
 * as defined in "Transformer Attention Masks and KV-Cache Inference"
 * (c86j224s.github.io), section "State of scaled dot-product attention",
 * and "KV Cache" (heepie.pages.dev), section "Self-Attention".
 *
 * Hot calls: kvattn_kv_append (write new K/V into the cache),
 * kvattn_attn_decode (one new token per sequence against the cache),
 * kvattn_attn_decode_append (both in one launch sequence: the decode step)
 * and kvattn_attn_prefill (many new tokens, causal/padding masked,
 * optionally writing the cache).  Plus sizing, validation and status
 * helpers, and the block-table operations of a paged cache: batch/beam
 * reorder, copy-on-write block copies and a host block pool with reference
 * counts.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named as "device" are HIP device pointers owned by the caller;
 *    the library never allocates, frees or keeps them past the call.  Host
 *    pointers (the kvattn_cache descriptor) are read during the call only.
 *  - Every compute call is asynchronous: it validates its host-side
 *    arguments, enqueues kernels on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns without synchronising.  Kernel faults
 *    surface at the caller's next synchronisation.
 *  - Return value: KVATTN_OK (0) or a negative kvattn_status.  On error
 *    nothing is enqueued; kvattn_last_error() returns a message for the
 *    calling thread.  No C++ exception crosses this boundary.
 *  - Positions are 0-based absolute token positions ("Transformer
 *    Attention Masks and KV-Cache Inference", sections "Causal mask and
 *    future positions" and "Position IDs and the append contract").
 *  - Masks are uint8 with 1 = the query may attend the key, 0 = blocked;
 *    a blocked key gets weight exactly 0 and its K/V bytes are never used
 *    (so non-finite padding cannot leak into the output).  A query row that
 *    can attend no key outputs 0.
 *  - Grouped-query attention: query head h reads KV head
 *    h / (num_q_heads / num_kv_heads) ("KV Cache Fully Explained",
 *    section "(2) GQA"); num_q_heads must be a multiple of num_kv_heads
 *    with a group size of 1, 2, 4 or 8.
 *  - Device-supplied indices (positions, lengths, block ids) are bounds
 *    checked in the kernels: an out-of-range write is skipped, an
 *    out-of-range block is read as fully masked, and lengths are clamped to
 *    the cache's capacity.  kvattn_validate reports such inputs.
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tokens per block of the paged layout: the 16-token blocks behind a page
 * table of "KV Cache, Flash Attention and Inference Optimization"
 * (factory.pai-world.com), section "PagedAttention", and "KV Cache Fully
 * Explained" (techblog.paldyn.com), section "(4) PagedAttention". */
#define KVATTN_BLOCK_TOKENS 16

typedef enum kvattn_status {
  KVATTN_OK = 0,
  KVATTN_EINVAL = -1,       /* null pointer, bad size, bad enum, misalignment */
  KVATTN_EUNSUPPORTED = -2, /* valid request this build has no kernel for   */
  KVATTN_EWORKSPACE = -3,   /* decode workspace missing or too small        */
  KVATTN_ELAUNCH = -4,      /* the HIP runtime refused a kernel launch      */
  KVATTN_ENOSPACE = -5      /* a block pool has too few free blocks         */
} kvattn_status;

typedef enum kvattn_dtype {
  KVATTN_F32 = 0,      /* IEEE binary32                                      */
  KVATTN_BF16 = 1,     /* bfloat16                                           */
  KVATTN_FP8_E4M3 = 2  /* OCP FP8 E4M3FN, cache only; real = code * scale    */
} kvattn_dtype;

typedef enum kvattn_layout {
  /* k, v: [num_rows, num_kv_heads, capacity, head_dim]: the
   * [batch, kv_heads, seq, head_dim] cache shape of "KV Cache"
   * (heepie.pages.dev), section "Tensor", and "Transformer Attention Masks
   * and KV-Cache Inference", section "Cache shape and memory calculation".
   * Sequence b uses row b. */
  KVATTN_CONTIGUOUS = 0,
  /* k, v: [num_blocks, num_kv_heads, 16, head_dim] pools; position p of
   * sequence b lives in block block_table[b * max_blocks + p / 16], slot
   * p % 16. */
  KVATTN_PAGED = 1
} kvattn_layout;

/* One layer's KV cache.  All memory is caller-owned device memory.
 * k and v must be 16-byte aligned.  Element type `dtype`; fp8 caches carry
 * one fp32 dequantisation scale per KV head for K and for V ("KV Cache
 * Fully Explained", section "(1) FP8 quantization" stores the cache at 8
 * bits; the per-head scale is this library's reading). */
typedef struct kvattn_cache {
  int32_t dtype;         /* kvattn_dtype                                   */
  int32_t layout;        /* kvattn_layout                                  */
  int32_t num_kv_heads;  /* >= 1                                           */
  int32_t head_dim;      /* 64 or 128                                      */
  int64_t capacity;      /* contiguous: positions per row; paged: ignored  */
  int64_t num_rows;      /* contiguous: rows allocated; paged: ignored     */
  int64_t num_blocks;    /* paged: blocks in each pool; contiguous: ignored*/
  void* k;               /* device                                         */
  void* v;               /* device                                         */
  const float* k_scale;  /* device [num_kv_heads]; fp8 only, else NULL     */
  const float* v_scale;  /* device [num_kv_heads]; fp8 only, else NULL     */
} kvattn_cache;

/* Library version string, e.g. "kvattn 0.1.0 gfx950". */
const char* kvattn_version(void);

/* Text for a kvattn_status value. */
const char* kvattn_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* kvattn_last_error(void);

/* Exact KV-cache bytes: 2 (K and V) * layers * batch * kv_heads * seq *
 * head_dim * elem_bytes ("Transformer Attention Masks and KV-Cache
 * Inference", section "Cache shape and memory calculation"; "KV Cache Fully
 * Explained", section "KV cache memory size calculation").  Pure host
 * arithmetic; returns 0 if the product overflows 64 bits. */
uint64_t kvattn_cache_bytes(uint64_t layers, uint64_t batch, uint64_t kv_heads,
                            uint64_t seq, uint64_t head_dim, uint64_t elem_bytes);

/* kvattn_kv_append - write n_new tokens' K and V per sequence into the cache.
 *
 * Append-then-attend: the new token's K/V join the cache before its query
 * attends ("Transformer Attention Masks and KV-Cache Inference", section
 * "Prefill and decode stages"; "KV Cache", section "TO-BE").  Token i of
 * sequence b goes to position p = positions[b] + i:
 *   contiguous: cache[b, g, p, :] = x[b, g, i, :]
 *   paged:      pool[block_table[b * max_blocks + p / 16], g, p % 16, :] = x[b, g, i, :]
 * Same element type in and out: the bits are copied.  f32 or bf16 input
 * into an fp8 cache: code = E4M3FN(fp32(x) / k_scale[g]) (or v_scale[g])
 * with round-to-nearest-even, saturation to +-448 and NaN -> 0x7F.
 *
 *  cache        host descriptor of the destination layer
 *  batch        sequences (contiguous: <= cache->num_rows)
 *  n_new        tokens per sequence in k_new / v_new (>= 0; 0 is a no-op)
 *  k_new, v_new device [batch, num_kv_heads, n_new, head_dim] of in_dtype,
 *               16-byte aligned
 *  in_dtype     KVATTN_F32 or KVATTN_BF16; equal to cache->dtype unless the
 *               cache is fp8
 *  positions    device int32 [batch]: position of token 0 of each sequence
 *               (the caller's stored length, per the append contract of
 *               "Position IDs and the append contract"; checked by
 *               kvattn_validate, not here)
 *  n_valid      device int32 [batch] or NULL: tokens of sequence b to write
 *               (clamped to [0, n_new]); NULL = all n_new
 *  block_table  device int32 [batch, max_blocks] (paged) or NULL (contiguous)
 * Writes whose position or block falls outside the cache are skipped.
 */
int kvattn_kv_append(const kvattn_cache* cache, int32_t batch, int32_t n_new,
                     const void* k_new, const void* v_new, int32_t in_dtype,
                     const int32_t* positions, const int32_t* n_valid,
                     const int32_t* block_table, int32_t max_blocks,
                     void* stream);

/* Bytes of device workspace kvattn_attn_decode needs for these sizes
 * (split-K partials: per (sequence, query head, partition) an fp32 output
 * vector plus the running max and sum).  part_tokens as in
 * kvattn_attn_decode (0 = default).  Returns 0 for invalid sizes. */
size_t kvattn_decode_workspace_bytes(int32_t cache_dtype, int32_t batch, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                     int32_t part_tokens);

/* Keys per split-K partition that part_tokens == 0 selects for these sizes
 * and this cache element type (measured per partition kernel: enough
 * workgroups for the current device's compute units - 256 on a whole
 * MI355X, and 256 is assumed when no device is visible - few enough
 * partials for the merge).
 * Returns 0 for invalid sizes. */
int32_t kvattn_decode_default_part_tokens(int32_t cache_dtype, int32_t batch, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t max_seq_len);

/* kvattn_attn_decode - one new query token per sequence against the cache.
 *
 * For sequence b and query head h (KV head g = h / G):
 *   keys s in [0, seq_lens[b]) with key_mask[b * key_mask_stride + s] != 0,
 *   z_s = scale * q[b, h, :] . K[b, g, s, :],
 *   out[b, h, :] = sum_s softmax(z)_s V[b, g, s, :]   (0 if no key allowed).
 * seq_lens counts the cached keys INCLUDING the token just appended: the new
 * query sees itself ("KV Cache", section "TO-BE"; "Transformer Attention
 * Masks and KV-Cache Inference", section "Causal mask and future
 * positions").  The scan is split into partitions of part_tokens keys whose
 * (max, sum, output) partial states are merged exactly afterwards - the
 * running max/sum renormalisation of "KV Cache, Flash Attention and
 * Inference Optimization", section "Flash Attention", numerical trick.
 *
 *  q           device [batch, num_q_heads, head_dim]: f32 for an f32 cache,
 *              bf16 for bf16 and fp8 caches; 16-byte aligned
 *  seq_lens    device int32 [batch]; values are clamped to [0, max_seq_len]
 *              and to the cache capacity (kvattn_validate reports it)
 *  max_seq_len host int32 upper bound of seq_lens (sizes the launch)
 *  block_table device int32 [batch, max_blocks] (paged) or NULL
 *  key_mask    device uint8 [batch, key_mask_stride] or NULL (no mask);
 *              key_mask_stride >= max_seq_len
 *  scale       score scale, normally 1/sqrt(head_dim)
 *  out         device fp32 [batch, num_q_heads, head_dim]
 *  workspace   device, >= kvattn_decode_workspace_bytes(...) bytes, 16-byte
 *              aligned; contents on entry are ignored
 *  part_tokens keys per partition: 0 = default, else a multiple of 64 in
 *              [64, 8192]; also part_tokens * G <= 8192 for the passes
 *              that keep every key's scores in LDS (f32 caches, bf16 with
 *              G < 16, fp8 with G < 4)
 * Bitwise deterministic for fixed arguments (fixed partitioning, no atomics).
 */
int kvattn_attn_decode(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads,
                       const void* q, int32_t q_dtype,
                       const int32_t* seq_lens, int32_t max_seq_len,
                       const int32_t* block_table, int32_t max_blocks,
                       const uint8_t* key_mask, int64_t key_mask_stride,
                       float scale, float* out,
                       void* workspace, size_t workspace_bytes, int32_t part_tokens,
                       void* stream);

/* kvattn_attn_decode_append - one decode step in one call: append the new
 * token's K/V, then attend it (append-then-attend, "Transformer Attention
 * Masks and KV-Cache Inference", section "Prefill and decode stages";
 * "KV Cache", section "TO-BE").
 *
 * Same result as kvattn_kv_append(positions = seq_lens - 1, n_new = 1)
 * followed by kvattn_attn_decode with the same arguments, bit for bit (the
 * cache bytes and the output), for every sequence with
 * 1 <= seq_lens[b] <= min(max_seq_len, capacity); a sequence outside that
 * range has nothing written.  The workgroup that attends key seq_lens[b] - 1
 * encodes the new rows and stores them in that cache slot before it reads
 * the cache (no other workgroup reads the slot), so no separate write pass
 * is launched.
 *
 *  k_new, v_new device [batch, num_kv_heads, head_dim] of in_dtype, 16-byte
 *               aligned: the new token of each sequence
 *  in_dtype     KVATTN_F32 or KVATTN_BF16; equal to cache->dtype unless the
 *               cache is fp8 (conversion as in kvattn_kv_append)
 *  every other argument as in kvattn_attn_decode.
 * The cache slot of position seq_lens[b] - 1 must belong to sequence b
 * alone (no other sequence's block table may map it) - as for any append
 * that runs beside a read of the same layer.
 */
int kvattn_attn_decode_append(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads,
                              const void* q, int32_t q_dtype,
                              const void* k_new, const void* v_new, int32_t in_dtype,
                              const int32_t* seq_lens, int32_t max_seq_len,
                              const int32_t* block_table, int32_t max_blocks,
                              const uint8_t* key_mask, int64_t key_mask_stride,
                              float scale, float* out,
                              void* workspace, size_t workspace_bytes, int32_t part_tokens,
                              void* stream);

/* kvattn_attn_decode_append_noalloc - kvattn_attn_decode_append for callers
 * that cannot allocate device memory: code under HIP graph capture, serving
 * loops that forbid allocation, harnesses without an allocator.  It takes no
 * workspace; the split-K partials go to a static device array of the library
 * (KVATTN_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the first call on
 * that GPU until the process ends).  The call allocates and frees nothing.
 *
 * Same arguments, same kernels and the same result as
 * kvattn_attn_decode_append without its workspace arguments, bit for bit.
 * Sizes whose partials (kvattn_decode_workspace_bytes for the same
 * arguments) exceed KVATTN_NOALLOC_SCRATCH_BYTES are refused with
 * KVATTN_EWORKSPACE before anything is enqueued.  The stream must belong to
 * the current device.
 *
 * Every call on one GPU uses that GPU's one array, and the array keeps the
 * last call's contents (nothing in it needs to start at zero: every partial
 * the merge reads was written by the same call).  Two calls that overlap in
 * time on one GPU - on different streams, or from different threads - race
 * on the array: serialise them.
 */
#define KVATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int kvattn_attn_decode_append_noalloc(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads,
                                      const void* q, int32_t q_dtype,
                                      const void* k_new, const void* v_new, int32_t in_dtype,
                                      const int32_t* seq_lens, int32_t max_seq_len,
                                      const int32_t* block_table, int32_t max_blocks,
                                      const uint8_t* key_mask, int64_t key_mask_stride,
                                      float scale, float* out, int32_t part_tokens,
                                      void* stream);

/* kvattn_attn_decode_multi - n_q new query tokens per sequence against the
 * cache that already holds them: decoding several tokens at once, such as
 * checking drafted tokens (speculative decoding) - the cache-read-bound
 * counterpart of a chunked prefill ("KV Cache" (heepie.pages.dev), section
 * "Prefill and Decode": decode steps are bound by the key/value scan;
 * "Transformer Attention Masks and KV-Cache Inference", sections "Prefill
 * and decode stages" and "Causal mask and future positions").
 *
 * For sequence b, head h and query i < n_q (at position seq_lens[b] - n_q + i):
 *   keys s in [0, seq_lens[b] - (n_q - 1 - i)) with key_mask[b, s] != 0,
 *   out[b, h, i, :] = sum_s softmax(scale * q[b, h, i, :] . K[s, :])_s V[s, :]
 * (0 if no key is allowed), i.e. causal among the n_q new tokens, whose K/V
 * sit at positions seq_lens[b] - n_q .. seq_lens[b] - 1: given as k_new and
 * v_new, they are stored there by this call first (the workgroup that
 * attends a position stores it, encoded as kvattn_kv_append would); with
 * k_new = v_new = NULL they must have been appended already.  Same as
 * kvattn_attn_prefill with attend_prefix over those tokens, computed as a
 * split-K decode: query i of head h is treated as head h * n_q + i, so the
 * group becomes G * n_q query columns per KV head.
 *
 *  num_q_heads  query heads Hq; G * n_q must be 1, 2, 4, 8 or 16, 16 only
 *               with a bf16 or fp8 cache
 *  n_q          queries per sequence, 1 .. 16
 *  q            device [batch, num_q_heads, n_q, head_dim] (bf16; f32 for an
 *               f32 cache), 16-byte aligned
 *  k_new, v_new device [batch, num_kv_heads, n_q, head_dim] of in_dtype (f32
 *               or bf16, equal to the cache dtype unless the cache is fp8),
 *               16-byte aligned, or both NULL; the position of a sequence
 *               outside [1, min(max_seq_len, capacity)] has nothing written
 *  out          device fp32 [batch, num_q_heads, n_q, head_dim]
 *  workspace    >= kvattn_decode_workspace_bytes(dtype, batch,
 *               num_q_heads * n_q, num_kv_heads, head_dim, max_seq_len,
 *               part_tokens) bytes (the query columns count as heads)
 *  every other argument as in kvattn_attn_decode (part_tokens * G * n_q
 *  <= 8192 with a bf16 cache and G * n_q < 16).
 */
int kvattn_attn_decode_multi(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads, int32_t n_q,
                             const void* q, int32_t q_dtype,
                             const void* k_new, const void* v_new, int32_t in_dtype,
                             const int32_t* seq_lens, int32_t max_seq_len,
                             const int32_t* block_table, int32_t max_blocks,
                             const uint8_t* key_mask, int64_t key_mask_stride,
                             float scale, float* out,
                             void* workspace, size_t workspace_bytes, int32_t part_tokens,
                             void* stream);

/* kvattn_attn_prefill - attention of n_max new tokens per sequence, causal
 * and/or padding masked, tiled so that no n x n score matrix is ever
 * stored ("KV Cache, Flash Attention and Inference Optimization", section
 * "Flash Attention - tiling trick"); optionally writing their K/V into the
 * cache ("KV Cache", section "Prefill and Decode": the prefill creates the
 * cache).
 *
 * Sequence b has q_lens[b] real new tokens (rows t >= q_lens[b] output 0)
 * at absolute positions P + t, P = positions[b].  Query t attends key
 * position s iff
 *   (attend_prefix ? 0 : P) <= s < P + q_lens[b],
 *   causal == 0 or s <= P + t            ("Causal mask and future positions"),
 *   key_mask == NULL or key_mask[b * key_mask_stride + s] != 0
 *                                        ("Padding mask and batch length").
 * Keys s >= P come from k / v (row s - P); keys s < P (attend_prefix only)
 * are read from the cache.
 *
 *  cache       NULL: no cache access (positions may then be NULL = all 0;
 *              attend_prefix must be 0).  Else the layer's cache: the new
 *              K/V are stored at positions P .. P + q_lens[b] - 1 (as
 *              kvattn_kv_append would) by the end of the call.  With the
 *              same element type in and out the attention kernel stores them
 *              itself after its output (bf16: each matrix-core workgroup the
 *              rows of its own query tile); into an fp8 cache an append
 *              kernel quantises them before the attention kernel runs.  The
 *              attention never reads these rows from the cache (keys s >= P
 *              come from k / v), so the order does not change the result.
 *  num_kv_heads, head_dim: shapes of q/k/v (must equal the cache's if given)
 *  q           device [batch, num_q_heads, n_max, head_dim] of dtype
 *  k, v        device [batch, num_kv_heads, n_max, head_dim] of dtype
 *  dtype       KVATTN_F32 or KVATTN_BF16 (q, k and v alike)
 *  positions   device int32 [batch] or NULL (all 0)
 *  q_lens      device int32 [batch] or NULL (all n_max); clamped to [0, n_max]
 *  block_table device int32 [batch, max_blocks] for a paged cache, else NULL
 *  key_mask    device uint8 or NULL; key_mask_stride >= largest P + n_max
 *  out         device fp32 [batch, num_q_heads, n_max, head_dim]
 * bf16 inputs run on bf16 MFMA with fp32 accumulation; the softmax
 * weights are rounded to bf16 for the second product and the row sum is
 * taken over the rounded weights.
 */
int kvattn_attn_prefill(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t n_max,
                        const void* q, const void* k, const void* v, int32_t dtype,
                        const int32_t* positions, const int32_t* q_lens,
                        const int32_t* block_table, int32_t max_blocks,
                        const uint8_t* key_mask, int64_t key_mask_stride,
                        int32_t causal, int32_t attend_prefix, float scale,
                        float* out, void* stream);

/* kvattn_validate - device-side check of the cache metadata contract
 * ("Transformer Attention Masks and KV-Cache Inference", section "Position
 * IDs and the append contract": the append position must equal the stored
 * length; lengths and block ids must stay inside the cache).
 * For each sequence b: 0 <= seq_lens[b] <= max_seq_len and <= the capacity
 * (contiguous: cache->capacity; paged: max_blocks * 16); every block id the
 * first seq_lens[b] positions use lies in [0, num_blocks); and, if
 * positions is not NULL, positions[b] == seq_lens[b] (the stored length
 * before an append).  *err_word (device int32, caller zeroes it) receives
 * the OR of KVATTN_VALIDATE_* bits.  A debug call, not on the timed path. */
#define KVATTN_VALIDATE_LEN_RANGE   1
#define KVATTN_VALIDATE_BLOCK_RANGE 2
#define KVATTN_VALIDATE_POSITION    4
int kvattn_validate(const kvattn_cache* cache, int32_t batch,
                    const int32_t* seq_lens, int32_t max_seq_len,
                    const int32_t* positions,
                    const int32_t* block_table, int32_t max_blocks,
                    int32_t* err_word, void* stream);

/* ---------------------------------------------------------------------------
 * Cache reorder and sharing.
 *
 * A paged cache moves and shares whole 16-token blocks by editing block
 * tables; only a write into a shared block needs a byte copy first
 * (copy-on-write).  "KV Cache, Flash Attention and Inference Optimization",
 * section "PagedAttention": the page table maps logical positions to
 * physical blocks, which lets beam-search and parallel-sampling branches
 * share KV and frees the cache from fragmentation; "KV Cache Fully
 * Explained", section "(4) PagedAttention": requests with a common prefix
 * point at the same physical blocks (copy-on-write).
 * ------------------------------------------------------------------------- */

/* kvattn_reorder_rows - batch/beam reorder of a paged cache.
 *
 * When the batch or beam order changes, every cache row must follow the
 * same permutation ("Transformer Attention Masks and KV-Cache Inference",
 * section "Batch and beam reorder": [A0, A1, B0] sorted to [B0, A1, A0] is
 * the permutation [2, 1, 0]).  With a block table a row is its table row
 * and its length, so only ids move:
 *   dst_table[i * max_blocks + j] = src_table[perm[i] * max_blocks + j]
 *   dst_lens[i]                   = src_lens[perm[i]]
 * A perm entry outside [0, src_rows) gives an empty row (all -1, length 0).
 * A perm with repeats leaves rows naming the same blocks: they are then
 * shared, and the host pool's references must follow (kvattn_pool_reorder
 * computes the same rows on the host and moves the references).
 *
 *  n_rows     rows of the result (0 <= n_rows <= 65535; 0 is a no-op)
 *  perm       device int32 [n_rows]
 *  src_rows   rows of src_table / src_lens (>= 0)
 *  src_table  device int32 [src_rows, max_blocks]
 *  src_lens   device int32 [src_rows], or NULL together with dst_lens
 *  max_blocks entries per table row, >= 1
 *  dst_table  device int32 [n_rows, max_blocks]; must not overlap src_table
 *  dst_lens   device int32 [n_rows] or NULL; must not overlap src_lens
 * Errors: KVATTN_EINVAL for a NULL required pointer or a size out of range. */
int kvattn_reorder_rows(int32_t n_rows, const int32_t* perm, int32_t src_rows,
                        const int32_t* src_table, const int32_t* src_lens,
                        int32_t max_blocks, int32_t* dst_table,
                        int32_t* dst_lens, void* stream);

/* kvattn_reorder_cache - batch/beam reorder of a contiguous cache: the rows
 * of `src` gathered into `dst` with the beam permutation ("Transformer
 * Attention Masks and KV-Cache Inference", section "Batch and beam
 * reorder"), for K and V and every KV head:
 *   dst[i, g, p, :] = src[perm[i], g, p, :]   for p < L,
 *   L = min(src_lens[perm[i]], capacity), or capacity when src_lens is NULL.
 * Positions >= L of dst row i keep their bytes.  A perm entry outside
 * [0, src->num_rows) leaves dst row i untouched.  dst_lens[i] =
 * src_lens[perm[i]] (0 for an out-of-range entry) when both are given.  The
 * bytes are copied as stored: fp8 codes stay codes, so dst is read with
 * src's scales (the scale pointers of both descriptors are not used here).
 *
 *  src, dst   contiguous caches with equal dtype, num_kv_heads, head_dim and
 *             capacity; dst->num_rows >= n_rows; their k/v memory must not
 *             overlap (the reorder is out of place)
 *  n_rows     0 <= n_rows <= 65535
 *  perm       device int32 [n_rows]
 *  src_lens   device int32 [src->num_rows] or NULL
 *  dst_lens   device int32 [n_rows] or NULL (needs src_lens); must not
 *             overlap src_lens
 * Errors: KVATTN_EINVAL (NULL pointer, mismatched caches, paged layout,
 * sizes). */
int kvattn_reorder_cache(const kvattn_cache* src, const kvattn_cache* dst,
                         int32_t n_rows, const int32_t* perm,
                         const int32_t* src_lens, int32_t* dst_lens,
                         void* stream);

/* kvattn_copy_blocks - copy whole physical blocks of a paged cache, the
 * copy half of copy-on-write ("KV Cache Fully Explained", section
 * "(4) PagedAttention": shared prefix blocks are copied before a holder
 * writes into them).  For every pair i, in the K pool and in the V pool:
 *   pool[dst_blocks[i], :, :, :] = pool[src_blocks[i], :, :, :]
 * (all KV heads, all 16 positions).  A pair with an id outside
 * [0, cache->num_blocks) is skipped.  The destinations must be distinct and
 * none may also be a source in the same call, so that the order of the
 * copies cannot matter; the pairs kvattn_pool_prepare_append returns meet
 * this.
 *
 *  cache                   paged cache (any dtype; bytes are copied)
 *  n                       pairs, 0 <= n <= 2^24 (0 is a no-op)
 *  src_blocks, dst_blocks  device int32 [n]
 * Errors: KVATTN_EINVAL (NULL pointer, contiguous layout, n out of range). */
int kvattn_copy_blocks(const kvattn_cache* cache, int32_t n,
                       const int32_t* src_blocks, const int32_t* dst_blocks,
                       void* stream);

/* kvattn_stream_read - measurement helper, not part of the attention path:
 * one plain pass over device memory, the context figure for the HBM-bound
 * calls above (decode reads the whole cache every step, "KV Cache", section
 * "Prefill and Decode").  Reads [src, src + bytes) once with 16-byte
 * non-temporal loads (each wave 1 KB contiguous per instruction; 4
 * workgroups of 256 threads per compute unit, each reading one contiguous
 * range) and XORs the XOR of all its 32-bit words into *sink, so the result
 * can be checked exactly.
 *
 *  src    device, 16-byte aligned
 *  bytes  a multiple of 16 (0 is a no-op)
 *  sink   device uint32, 4-byte aligned; the caller sets it (e.g. to 0)
 * Errors: KVATTN_EINVAL (NULL pointer, alignment, bytes). */
int kvattn_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* ---------------------------------------------------------------------------
 * Host block pool.
 *
 * The free list of a paged cache's physical blocks with a reference count
 * per block: "KV Cache, Flash Attention and Inference Optimization",
 * section "Exercises" (a toy PagedAttention with fixed 16-token blocks and
 * a free list; a finished sequence returns its blocks to the pool), with the
 * sharing of section "PagedAttention" and the copy-on-write prefix sharing
 * of "KV Cache Fully Explained", section "(4) PagedAttention".
 *
 * Host memory only: the block tables passed to these calls are host int32
 * arrays [rows, max_blocks] (-1 = no block) that the caller uploads for
 * the device calls.  A row of length L uses its first ceil(L / 16) entries.
 * A block's reference count is the number of table rows that name it; the
 * block is free at 0, and the free list hands out the lowest free id first.
 * Every call is all-or-nothing: on error neither the pool nor the caller's
 * arrays change.  Calls on one pool are serialised by a lock inside it.
 * ------------------------------------------------------------------------- */
typedef struct kvattn_pool kvattn_pool;

/* A pool of num_blocks free blocks (1 <= num_blocks <= 2^31 - 1), or NULL
 * with kvattn_last_error() set.  The caller destroys it. */
kvattn_pool* kvattn_pool_create(int64_t num_blocks);
void kvattn_pool_destroy(kvattn_pool* pool);
int64_t kvattn_pool_num_blocks(const kvattn_pool* pool);
int64_t kvattn_pool_num_free(const kvattn_pool* pool);
/* Reference count of one block; -1 for an id outside the pool. */
int32_t kvattn_pool_refcount(const kvattn_pool* pool, int32_t block);

/* Take n free blocks (count 1 each) into ids[n], lowest ids first.
 * KVATTN_ENOSPACE if fewer than n are free. */
int kvattn_pool_alloc(kvattn_pool* pool, int32_t n, int32_t* ids);
/* Add one reference to each listed block (all must be allocated). */
int kvattn_pool_retain(kvattn_pool* pool, int32_t n, const int32_t* ids);
/* Drop one reference per listing; a block reaching 0 returns to the free
 * list.  KVATTN_EINVAL if a block is listed more often than it is held. */
int kvattn_pool_release(kvattn_pool* pool, int32_t n, const int32_t* ids);

/* Share a prefix: dst_row names the first ceil(length / 16) blocks of
 * src_row (one more reference each) and -1 after them.  For a new beam or
 * sample branch, or a request that reuses a cached prefix. */
int kvattn_pool_fork(kvattn_pool* pool, const int32_t* src_row,
                     int32_t* dst_row, int32_t max_blocks, int32_t length);

/* A sequence of `length` positions ends: its blocks lose one reference each
 * and its row becomes -1. */
int kvattn_pool_free_seq(kvattn_pool* pool, int32_t* row, int32_t max_blocks,
                         int32_t length);

/* Make positions cur_lens[b] .. new_lens[b] - 1 of every row writable,
 * rows in order, before kvattn_kv_append / kvattn_attn_decode_append write
 * them:
 *  - if cur_lens[b] % 16 != 0 and new_lens[b] > cur_lens[b], the partly
 *    filled block at entry cur_lens[b] / 16 is written; if another row also
 *    holds it, the row gets a fresh block instead, the pair (old, fresh) is
 *    appended to copy_src / copy_dst, and the old block loses this row's
 *    reference (copy-on-write: run kvattn_copy_blocks on the pairs before
 *    the write);
 *  - entries ceil(cur_lens[b] / 16) .. ceil(new_lens[b] / 16) - 1 get fresh
 *    blocks.
 *  tables      host int32 [rows, max_blocks], updated in place
 *  cur_lens    host int32 [rows]: positions already stored
 *  new_lens    host int32 [rows]: positions stored after the write,
 *              cur_lens[b] <= new_lens[b] <= 16 * max_blocks
 *  copy_src, copy_dst  host int32 [rows] (at most one pair per row)
 *  n_copies    host: number of pairs written
 * KVATTN_ENOSPACE if the pool runs out (nothing changes). */
int kvattn_pool_prepare_append(kvattn_pool* pool, int32_t rows, int32_t* tables,
                               int32_t max_blocks, const int32_t* cur_lens,
                               const int32_t* new_lens, int32_t* copy_src,
                               int32_t* copy_dst, int32_t* n_copies);

/* Host side of kvattn_reorder_rows: the same dst rows and lengths, with the
 * references moved along (each dst row adds one reference to the blocks it
 * names, then every src row drops its own; rows no longer named return
 * their blocks to the free list, rows named twice share them).
 *  perm        host int32 [n_rows]
 *  src_tables  host int32 [src_rows, max_blocks]; src_lens host int32 [src_rows]
 *  dst_tables  host int32 [n_rows, max_blocks], must not overlap src_tables;
 *  dst_lens    host int32 [n_rows] */
int kvattn_pool_reorder(kvattn_pool* pool, int32_t n_rows, const int32_t* perm,
                        int32_t src_rows, const int32_t* src_tables,
                        const int32_t* src_lens, int32_t max_blocks,
                        int32_t* dst_tables, int32_t* dst_lens);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_H */
