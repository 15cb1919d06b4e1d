// Internal launch interface between the C ABI layer (kvattn_api.cpp) and the
// kernel translation units.  Host arguments are already validated when these
// are called; each returns KVATTN_OK or KVATTN_EUNSUPPORTED / KVATTN_ELAUNCH.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace kvattn {

struct AppendLaunch {
  CacheView c;
  int32_t cache_dtype;
  int32_t in_dtype;
  int32_t head_dim;
  int32_t batch, num_kv_heads, n_new;
  const uint8_t* k_new;
  const uint8_t* v_new;
  const float* k_scale;
  const float* v_scale;
  const int32_t* positions;  // may be NULL (all 0)
  const int32_t* n_valid;    // may be NULL (all n_new)
};
int launch_append(const AppendLaunch& a, hipStream_t stream);

struct DecodeLaunch {
  CacheView c;
  int32_t cache_dtype;
  int32_t head_dim;
  int32_t batch, num_q_heads, num_kv_heads;
  const uint8_t* q;
  const int32_t* seq_lens;
  int32_t ctx_limit;  // min(max_seq_len, capacity in tokens)
  const uint8_t* key_mask;
  int64_t key_mask_stride;
  float scale;
  const float* k_scale;
  const float* v_scale;
  float* out;
  float* ws_o;   // [batch, num_q_heads, num_parts, head_dim]
  float* ws_ml;  // [batch, num_q_heads, num_parts, 2]
  int32_t part_tokens;
  int32_t num_parts;
  // Fused append: the new tokens' K and V rows [batch, num_kv_heads,
  // n_tail, head_dim] of in_dtype, stored at positions seq_lens[b] - n_tail
  // .. seq_lens[b] - 1 by the workgroups that attend those keys.  Null for a
  // plain decode.
  const uint8_t* k_new;
  const uint8_t* v_new;
  int32_t in_dtype;
  // Queries per sequence (1 for a plain decode): num_q_heads counts
  // (head, query) pairs, query i of head h being virtual head h * n_tail + i;
  // it sees the keys below seq_lens[b] - (n_tail - 1 - i).
  int32_t n_tail;
};
int launch_decode(const DecodeLaunch& a, hipStream_t stream);
// Whether the decode partition pass for this cache type and group (query
// columns per KV head) keeps a running softmax per wave (no per-key scores
// in LDS, so no cap on part_tokens * group): the fp8 matrix-core pass
// (group >= 4) and the single-sweep bf16 matrix-core pass (16 columns).
#ifndef KVATTN_BF16_ONLINE_MIN_G
#define KVATTN_BF16_ONLINE_MIN_G 16
#endif
inline bool decode_single_pass(int32_t cache_dtype, int32_t group) {
  return (cache_dtype == KVATTN_FP8_E4M3 && group >= 4) ||
         (cache_dtype == KVATTN_BF16 && group >= KVATTN_BF16_ONLINE_MIN_G);
}
// Dynamic LDS bytes of the decode partition kernel.
int decode_lds_bytes(int part_tokens, int group, int head_dim);

struct PrefillLaunch {
  CacheView c;          // valid when has_cache
  int32_t has_cache;
  int32_t cache_dtype;
  const float* k_scale;
  const float* v_scale;
  int32_t dtype;        // of q, k, v
  int32_t head_dim;
  int32_t batch, num_q_heads, num_kv_heads, n_max;
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* positions;  // may be NULL
  const int32_t* q_lens;     // may be NULL
  const uint8_t* key_mask;
  int64_t key_mask_stride;
  int32_t causal, attend_prefix;
  float scale;
  float* out;
  // The attention kernel stores the new K/V rows into the cache itself
  // (same dtype in and out); otherwise the caller launches the append.
  int32_t write_cache;
};
int launch_prefill(const PrefillLaunch& a, hipStream_t stream);
// Whether launch_prefill runs the bf16 MFMA kernel for these arguments.
bool prefill_mfma_supports(const PrefillLaunch& a);

struct ValidateLaunch {
  CacheView c;
  int32_t batch;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int64_t cap_tokens;
  const int32_t* positions;
  int32_t* err_word;
};
int launch_validate(const ValidateLaunch& a, hipStream_t stream);

// Block-table row gather (batch/beam reorder of a paged cache).
struct RowReorderLaunch {
  int32_t n_rows, src_rows, max_blocks;
  const int32_t* perm;
  const int32_t* src_table;
  const int32_t* src_lens;  // may be NULL (then dst_lens is NULL)
  int32_t* dst_table;
  int32_t* dst_lens;
};
int launch_reorder_rows(const RowReorderLaunch& a, hipStream_t stream);

// Contiguous-cache row gather: for dst row i and KV head g, the first L
// positions of src row perm[i] (L from src_lens, else the capacity).
struct CacheReorderLaunch {
  const uint8_t* src_k;
  const uint8_t* src_v;
  uint8_t* dst_k;
  uint8_t* dst_v;
  int64_t pos_bytes;   // bytes per position of one head: head_dim * element bytes
  int32_t capacity;    // positions per head row
  int32_t num_kv_heads;
  int32_t n_rows, src_rows;
  const int32_t* perm;
  const int32_t* src_lens;  // may be NULL
  int32_t* dst_lens;        // may be NULL
};
int launch_reorder_cache(const CacheReorderLaunch& a, hipStream_t stream);

// Whole-block copies inside one paged cache (both pools).
struct BlockCopyLaunch {
  uint8_t* k;
  uint8_t* v;
  int64_t block_bytes;  // num_kv_heads * 16 * head_dim * element bytes
  int64_t num_blocks;
  int32_t n;
  const int32_t* src;
  const int32_t* dst;
};
int launch_copy_blocks(const BlockCopyLaunch& a, hipStream_t stream);

// Streaming read (a measurement helper): the XOR of every 32-bit word of
// [src, src + bytes) is XORed into *sink; bytes is a multiple of 16.
struct StreamReadLaunch {
  const uint8_t* src;
  int64_t bytes;
  int64_t chunks_per_wg;  // 16-byte chunks each workgroup reads, a multiple of 1024
  uint32_t* sink;
};
int launch_stream_read(const StreamReadLaunch& a, int32_t workgroups, hipStream_t stream);

}  // namespace kvattn
