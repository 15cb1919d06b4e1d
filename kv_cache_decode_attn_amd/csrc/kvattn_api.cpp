// C ABI of the kvattn library: host-side argument checks, launch geometry and
// workspace sizing.  No allocation, no synchronisation: every call enqueues
// on the caller's stream and returns.  See include/kvattn.h for the
// contract of each entry point.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "kvattn.h"
#include "block_pool.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return KVATTN_OK;
}

int elem_bytes(int dt) {
  switch (dt) {
    case KVATTN_F32: return 4;
    case KVATTN_BF16: return 2;
    case KVATTN_FP8_E4M3: return 1;
    default: return 0;
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int group_ok(int32_t hq, int32_t hkv) {
  if (hkv < 1 || hq < 1 || hq % hkv != 0) return 0;
  const int g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

// Decode groups: also 16 query columns per KV head on the matrix-core
// passes (bf16 and fp8 caches).
int decode_group_ok(int32_t dtype, int32_t hq, int32_t hkv) {
  if (group_ok(hq, hkv)) return 1;
  return hkv >= 1 && hq == 16 * hkv && dtype != KVATTN_F32;
}

// Fills the kernels' view of a cache descriptor; also returns the number of
// positions a sequence can hold.
int make_view(const char* who, const kvattn_cache* c, int32_t batch, const int32_t* block_table,
              int32_t max_blocks, kvattn::CacheView* v, int64_t* cap_tokens) {
  if (!c) return fail(KVATTN_EINVAL, "%s: cache descriptor is NULL", who);
  const int eb = elem_bytes(c->dtype);
  if (!eb) return fail(KVATTN_EINVAL, "%s: unknown cache dtype %d", who, c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVATTN_EUNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", who, c->head_dim);
  if (c->num_kv_heads < 1 || c->num_kv_heads > 65535)
    return fail(KVATTN_EINVAL, "%s: num_kv_heads %d out of range", who, c->num_kv_heads);
  if (!c->k || !c->v) return fail(KVATTN_EINVAL, "%s: cache k/v pointer is NULL", who);
  if (!aligned16(c->k) || !aligned16(c->v)) return fail(KVATTN_EINVAL, "%s: cache k/v not 16-byte aligned", who);
  if (c->dtype == KVATTN_FP8_E4M3 && (!c->k_scale || !c->v_scale))
    return fail(KVATTN_EINVAL, "%s: fp8 cache needs k_scale and v_scale", who);
  const int64_t row = (int64_t)c->head_dim * eb;
  *v = kvattn::CacheView{};
  v->k = static_cast<uint8_t*>(c->k);
  v->v = static_cast<uint8_t*>(c->v);
  v->row_stride = row;
  if (c->layout == KVATTN_CONTIGUOUS) {
    if (c->capacity <= 0 || c->capacity % KVATTN_BLOCK_TOKENS != 0 || c->capacity > (int64_t)1 << 30)
      return fail(KVATTN_EINVAL, "%s: contiguous capacity %lld must be a positive multiple of 16 (<= 2^30)",
                  who, (long long)c->capacity);
    if (c->num_rows < batch)
      return fail(KVATTN_EINVAL, "%s: contiguous cache has %lld rows < batch %d", who, (long long)c->num_rows, batch);
    v->head_stride = c->capacity * row;
    v->seq_stride = c->num_kv_heads * v->head_stride;
    v->capacity = c->capacity;
    v->paged = 0;
    *cap_tokens = c->capacity;
  } else if (c->layout == KVATTN_PAGED) {
    if (c->num_blocks <= 0 || c->num_blocks > INT32_MAX)
      return fail(KVATTN_EINVAL, "%s: paged cache num_blocks %lld out of range", who, (long long)c->num_blocks);
    if (!block_table) return fail(KVATTN_EINVAL, "%s: paged cache needs a block_table", who);
    if (max_blocks <= 0 || max_blocks > (1 << 26))
      return fail(KVATTN_EINVAL, "%s: max_blocks %d out of range", who, max_blocks);
    v->head_stride = (int64_t)KVATTN_BLOCK_TOKENS * row;
    v->block_stride = c->num_kv_heads * v->head_stride;
    v->num_blocks = c->num_blocks;
    v->block_table = block_table;
    v->max_blocks = max_blocks;
    v->paged = 1;
    *cap_tokens = (int64_t)max_blocks * KVATTN_BLOCK_TOKENS;
  } else {
    return fail(KVATTN_EINVAL, "%s: unknown layout %d", who, c->layout);
  }
  return KVATTN_OK;
}

constexpr int32_t kMaxPartTokens = 8192;
constexpr int kMaxDevices = 64;

// Compute units of the current device, read once per device.  A host with
// no visible device (sizing queries made on a CPU-only machine) gets 256, the
// count of a whole MI355X; a partitioned MI355X (CPX mode) reports its
// partition's share and the default partitioning follows it.
int64_t compute_units() {
  static std::mutex mu;
  static int cus[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next HIP call
    return 256;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cus[dev] = n;
  }
  return cus[dev];
}
constexpr int32_t kMaxPartScores = 8192;  // part_tokens * group, bounds the LDS

// Default keys per partition, per partition kernel (measured on MI355X):
//  - up to 512 keys: one partition (no merge launch);
//  - fp8 cache with G >= 4 (matrix-core pass): long partitions amortise the
//    per-workgroup combine and shrink the merge, and the pass runs best at
//    one workgroup per compute unit (a unit given two workgroups finishes
//    last).  Take as many partitions per (sequence, KV head) as the device's
//    compute units hold, with the keys split as evenly as 64-key steps allow
//    (4160 keys at 131,073 keys x 8 KV heads: exactly 256 workgroups).
//  - bf16 cache with 16 query columns per KV head (the single-sweep pass, in
//    eight-wave workgroups): 1,280 keys, halved in 64-key steps while the
//    grid has fewer than 768 workgroups.  On the check of 4 drafted tokens
//    (lengths U[1, 8192]) this gives 640 keys at batch 8 and 1,280 at
//    batches 16-64, the best of 256-1,536 at each.
//  - the three-phase passes: 512 keys for G >= 4, 256 for G <= 2, shrunk
//    until the grid offers >= 2048 workgroups.
bool fp8_mfma_pass(int32_t dtype, int32_t group) { return dtype == KVATTN_FP8_E4M3 && group >= 4; }

int32_t default_part_tokens(int32_t dtype, int32_t batch, int32_t hq, int32_t hkv, int32_t max_seq_len) {
  const int32_t group = hq / hkv;
  auto wgs = [&](int32_t t) { return (int64_t)batch * hkv * (((int64_t)max_seq_len + t - 1) / t); };
  // Up to 512 keys: one partition per sequence.  The whole decode is then a
  // single launch (no merge pass), which is what a latency-bound short
  // context wants; 512 keys x 16 columns still fit the per-key score buffer.
  if (max_seq_len <= 512) return max_seq_len <= 64 ? 64 : (max_seq_len + 63) / 64 * 64;
  if (fp8_mfma_pass(dtype, group)) {
    const int64_t heads = (int64_t)batch * hkv;
    const int64_t units = compute_units();
    const int64_t per = heads >= units ? 1 : units / heads;
    const int64_t t = ((max_seq_len + per - 1) / per + 63) / 64 * 64;
    return (int32_t)(t < 256 ? 256 : t > kMaxPartTokens ? kMaxPartTokens : t);
  }
  if (kvattn::decode_single_pass(dtype, group)) {
    // the single-sweep bf16 pass (eight-wave workgroups, no scores in LDS):
    // 1,280 keys, halved in 64-key steps while the grid has fewer than 768
    // workgroups
    int32_t t = 1280;
    while (t > 64 && wgs(t) < 768) t = std::max<int32_t>(64, t / 2 / 64 * 64);
    return t;
  }
  int32_t t = group >= 4 ? 512 : 256;
  while (t * group > kMaxPartScores) t /= 2;
  while (t > 64 && wgs(t) < 2048) t /= 2;
  return t;
}

// Shared body of kvattn_attn_decode and kvattn_attn_decode_append (k_new
// NULL for the former).
int attn_decode_impl(const char* who, const kvattn_cache* cache, int32_t batch, int32_t num_q_heads, const void* q,
                     int32_t q_dtype, const void* k_new, const void* v_new, int32_t in_dtype,
                     const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table, int32_t max_blocks,
                     const uint8_t* key_mask, int64_t key_mask_stride, float scale, float* out, void* workspace,
                     size_t workspace_bytes, int32_t part_tokens, void* stream, int32_t n_tail = 1) {
  if (batch < 0 || batch > 65535) return fail(KVATTN_EINVAL, "%s: batch %d out of range", who, batch);
  kvattn::CacheView view;
  int64_t cap = 0;
  int rc = make_view(who, cache, batch, block_table, max_blocks, &view, &cap);
  if (rc) return rc;
  if (!decode_group_ok(cache->dtype, num_q_heads, cache->num_kv_heads))
    return fail(KVATTN_EUNSUPPORTED,
                "%s: %d query columns over %d KV heads: group must be 1, 2, 4, 8 (or 16 with a bf16/fp8 cache)", who,
                num_q_heads, cache->num_kv_heads);
  const int32_t want_q = (cache->dtype == KVATTN_F32) ? KVATTN_F32 : KVATTN_BF16;
  if (q_dtype != want_q)
    return fail(KVATTN_EUNSUPPORTED, "%s: q dtype %d; this cache needs %s queries", who, q_dtype,
                want_q == KVATTN_F32 ? "f32" : "bf16");
  if (max_seq_len < 0) return fail(KVATTN_EINVAL, "%s: max_seq_len < 0", who);
  const bool append = k_new || v_new || in_dtype >= 0;
  if (append) {
    if (in_dtype != KVATTN_F32 && in_dtype != KVATTN_BF16)
      return fail(KVATTN_EINVAL, "%s: input dtype must be f32 or bf16", who);
    if (in_dtype != cache->dtype && cache->dtype != KVATTN_FP8_E4M3)
      return fail(KVATTN_EUNSUPPORTED, "%s: input dtype %d does not match cache dtype %d", who, in_dtype,
                  cache->dtype);
  }
  if (batch == 0) return ok();
  if (append) {
    if (!k_new || !v_new) return fail(KVATTN_EINVAL, "%s: k_new and v_new are required", who);
    if (!aligned16(k_new) || !aligned16(v_new))
      return fail(KVATTN_EINVAL, "%s: k_new/v_new not 16-byte aligned", who);
  }
  if (!q || !seq_lens || !out) return fail(KVATTN_EINVAL, "%s: q, seq_lens and out are required", who);
  if (!aligned16(q) || !aligned16(out)) return fail(KVATTN_EINVAL, "%s: q/out not 16-byte aligned", who);
  if (key_mask && key_mask_stride < max_seq_len)
    return fail(KVATTN_EINVAL, "%s: key_mask_stride %lld < max_seq_len %d", who, (long long)key_mask_stride,
                max_seq_len);
  const int32_t group = num_q_heads / cache->num_kv_heads;
  int32_t t = part_tokens;
  if (t == 0) t = default_part_tokens(cache->dtype, batch, num_q_heads, cache->num_kv_heads, max_seq_len);
  // the single-sweep passes keep no per-key scores in LDS
  const bool scores_in_lds = !kvattn::decode_single_pass(cache->dtype, group);
  if (t < 64 || t > kMaxPartTokens || t % 64 != 0 || (scores_in_lds && t * group > kMaxPartScores))
    return fail(KVATTN_EINVAL, "%s: part_tokens %d: need a multiple of 64 in [64, %d] with part_tokens*group <= %d",
                who, t, kMaxPartTokens, kMaxPartScores);
  const int64_t parts = ((int64_t)max_seq_len + t - 1) / t;
  if (parts > 65535) return fail(KVATTN_EINVAL, "%s: too many partitions (%lld)", who, (long long)parts);
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (parts > 1) {
    const size_t need = kvattn_decode_workspace_bytes(cache->dtype, batch, num_q_heads, cache->num_kv_heads,
                                                      cache->head_dim, max_seq_len, t);
    if (!workspace || workspace_bytes < need)
      return fail(KVATTN_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", who, workspace ? workspace_bytes : 0,
                  need);
    if (!aligned16(workspace)) return fail(KVATTN_EINVAL, "%s: workspace not 16-byte aligned", who);
    ws_o = static_cast<float*>(workspace);
    ws_ml = ws_o + (size_t)batch * num_q_heads * parts * cache->head_dim;
  }
  kvattn::DecodeLaunch a{};
  a.c = view;
  a.cache_dtype = cache->dtype;
  a.head_dim = cache->head_dim;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.q = static_cast<const uint8_t*>(q);
  a.seq_lens = seq_lens;
  a.ctx_limit = (int32_t)(cap < max_seq_len ? cap : max_seq_len);
  a.key_mask = key_mask;
  a.key_mask_stride = key_mask_stride;
  a.scale = scale;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.out = out;
  a.ws_o = ws_o;
  a.ws_ml = ws_ml;
  a.part_tokens = t;
  a.num_parts = (int32_t)(parts < 1 ? 1 : parts);
  a.n_tail = n_tail;
  if (append) {
    a.k_new = static_cast<const uint8_t*>(k_new);
    a.v_new = static_cast<const uint8_t*>(v_new);
    a.in_dtype = in_dtype;
  }
  rc = kvattn::launch_decode(a, static_cast<hipStream_t>(stream));
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

}  // namespace

extern "C" {

const char* kvattn_version(void) { return "kvattn 0.1.0 gfx950"; }

const char* kvattn_status_string(int status) {
  switch (status) {
    case KVATTN_OK: return "ok";
    case KVATTN_EINVAL: return "invalid argument";
    case KVATTN_EUNSUPPORTED: return "unsupported configuration";
    case KVATTN_EWORKSPACE: return "workspace missing or too small";
    case KVATTN_ELAUNCH: return "kernel launch failed";
    case KVATTN_ENOSPACE: return "block pool exhausted";
    default: return "unknown status";
  }
}

const char* kvattn_last_error(void) { return g_last_error.c_str(); }

uint64_t kvattn_cache_bytes(uint64_t layers, uint64_t batch, uint64_t kv_heads, uint64_t seq,
                            uint64_t head_dim, uint64_t elem_bytes) {
  uint64_t r = 2;
  const uint64_t f[6] = {layers, batch, kv_heads, seq, head_dim, elem_bytes};
  for (uint64_t x : f)
    if (__builtin_mul_overflow(r, x, &r)) return 0;
  return r;
}

int kvattn_kv_append(const kvattn_cache* cache, int32_t batch, int32_t n_new, const void* k_new,
                     const void* v_new, int32_t in_dtype, const int32_t* positions, const int32_t* n_valid,
                     const int32_t* block_table, int32_t max_blocks, void* stream) {
  const char* who = "kvattn_kv_append";
  if (batch < 0 || n_new < 0) return fail(KVATTN_EINVAL, "%s: negative batch or n_new", who);
  if (batch > 65535) return fail(KVATTN_EINVAL, "%s: batch %d too large", who, batch);
  kvattn::CacheView view;
  int64_t cap = 0;
  int rc = make_view(who, cache, batch, block_table, max_blocks, &view, &cap);
  if (rc) return rc;
  if (in_dtype != KVATTN_F32 && in_dtype != KVATTN_BF16)
    return fail(KVATTN_EINVAL, "%s: input dtype must be f32 or bf16", who);
  if (in_dtype != cache->dtype && cache->dtype != KVATTN_FP8_E4M3)
    return fail(KVATTN_EUNSUPPORTED, "%s: input dtype %d does not match cache dtype %d", who, in_dtype,
                cache->dtype);
  if ((int64_t)batch * n_new == 0) return ok();
  if (!k_new || !v_new || !positions) return fail(KVATTN_EINVAL, "%s: k_new, v_new and positions are required", who);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(KVATTN_EINVAL, "%s: k_new/v_new not 16-byte aligned", who);
  kvattn::AppendLaunch a{};
  a.c = view;
  a.cache_dtype = cache->dtype;
  a.in_dtype = in_dtype;
  a.head_dim = cache->head_dim;
  a.batch = batch;
  a.num_kv_heads = cache->num_kv_heads;
  a.n_new = n_new;
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.positions = positions;
  a.n_valid = n_valid;
  rc = kvattn::launch_append(a, static_cast<hipStream_t>(stream));
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

int32_t kvattn_decode_default_part_tokens(int32_t cache_dtype, int32_t batch, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t max_seq_len) {
  if (batch < 0 || max_seq_len < 0 || !elem_bytes(cache_dtype) ||
      !decode_group_ok(cache_dtype, num_q_heads, num_kv_heads))
    return 0;
  return default_part_tokens(cache_dtype, batch, num_q_heads, num_kv_heads, max_seq_len);
}

size_t kvattn_decode_workspace_bytes(int32_t cache_dtype, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_seq_len, int32_t part_tokens) {
  if (batch < 0 || max_seq_len < 0 || head_dim <= 0 || !elem_bytes(cache_dtype) ||
      !decode_group_ok(cache_dtype, num_q_heads, num_kv_heads))
    return 0;
  const int32_t t =
      part_tokens ? part_tokens : default_part_tokens(cache_dtype, batch, num_q_heads, num_kv_heads, max_seq_len);
  if (t <= 0) return 0;
  const int64_t parts = ((int64_t)max_seq_len + t - 1) / t;
  if (parts <= 1) return 0;
  return (size_t)batch * num_q_heads * parts * (head_dim + 2) * sizeof(float);
}

int kvattn_attn_decode(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads, const void* q,
                       int32_t q_dtype, const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                       int32_t max_blocks, const uint8_t* key_mask, int64_t key_mask_stride, float scale,
                       float* out, void* workspace, size_t workspace_bytes, int32_t part_tokens, void* stream) {
  return attn_decode_impl("kvattn_attn_decode", cache, batch, num_q_heads, q, q_dtype, nullptr, nullptr, -1,
                          seq_lens, max_seq_len, block_table, max_blocks, key_mask, key_mask_stride, scale, out,
                          workspace, workspace_bytes, part_tokens, stream);
}

int kvattn_attn_decode_append(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads, const void* q,
                              int32_t q_dtype, const void* k_new, const void* v_new, int32_t in_dtype,
                              const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                              int32_t max_blocks, const uint8_t* key_mask, int64_t key_mask_stride, float scale,
                              float* out, void* workspace, size_t workspace_bytes, int32_t part_tokens,
                              void* stream) {
  if (in_dtype < 0)
    return fail(KVATTN_EINVAL, "kvattn_attn_decode_append: input dtype must be f32 or bf16");
  return attn_decode_impl("kvattn_attn_decode_append", cache, batch, num_q_heads, q, q_dtype, k_new, v_new,
                          in_dtype, seq_lens, max_seq_len, block_table, max_blocks, key_mask, key_mask_stride, scale,
                          out, workspace, workspace_bytes, part_tokens, stream);
}

}  // extern "C"

namespace {

// Device memory of kvattn_attn_decode_append_noalloc: the split-K partials
// live in this array instead of a caller workspace.  Every device the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` is only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[KVATTN_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (NULL with the error recorded).
void* scratch_address(const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    fail(KVATTN_ELAUNCH, "%s: no current HIP device (%s)", who, hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      fail(KVATTN_ELAUNCH, "%s: hipGetSymbolAddress of the scratch array failed on device %d (%s)", who, dev,
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int kvattn_attn_decode_append_noalloc(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads, const void* q,
                                      int32_t q_dtype, const void* k_new, const void* v_new, int32_t in_dtype,
                                      const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                                      int32_t max_blocks, const uint8_t* key_mask, int64_t key_mask_stride,
                                      float scale, float* out, int32_t part_tokens, void* stream) {
  const char* who = "kvattn_attn_decode_append_noalloc";
  if (!cache) return fail(KVATTN_EINVAL, "%s: cache descriptor is NULL", who);
  if (in_dtype < 0) return fail(KVATTN_EINVAL, "%s: input dtype must be f32 or bf16", who);
  // the partials this call needs must fit the static array
  const size_t need = kvattn_decode_workspace_bytes(cache->dtype, batch, num_q_heads, cache->num_kv_heads,
                                                    cache->head_dim, max_seq_len, part_tokens);
  if (need > (size_t)KVATTN_NOALLOC_SCRATCH_BYTES)
    return fail(KVATTN_EWORKSPACE,
                "%s: these sizes need %zu bytes of split-K partials, more than the %zu-byte static scratch; "
                "use kvattn_attn_decode_append with a workspace",
                who, need, (size_t)KVATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address(who);
    if (!ws) return KVATTN_ELAUNCH;
  }
  return attn_decode_impl(who, cache, batch, num_q_heads, q, q_dtype, k_new, v_new, in_dtype, seq_lens, max_seq_len,
                          block_table, max_blocks, key_mask, key_mask_stride, scale, out, ws,
                          need > 0 ? (size_t)KVATTN_NOALLOC_SCRATCH_BYTES : 0, part_tokens, stream);
}

int kvattn_attn_decode_multi(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads, int32_t n_q,
                             const void* q, int32_t q_dtype, const void* k_new, const void* v_new, int32_t in_dtype,
                             const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                             int32_t max_blocks, const uint8_t* key_mask, int64_t key_mask_stride, float scale,
                             float* out, void* workspace, size_t workspace_bytes, int32_t part_tokens, void* stream) {
  const char* who = "kvattn_attn_decode_multi";
  if (n_q < 1 || n_q > 16) return fail(KVATTN_EINVAL, "%s: n_q %d out of range [1, 16]", who, n_q);
  if (num_q_heads < 1 || (int64_t)num_q_heads * n_q > 65535)
    return fail(KVATTN_EINVAL, "%s: %d query heads x %d queries out of range", who, num_q_heads, n_q);
  const bool append = k_new || v_new;
  if (append && in_dtype != KVATTN_F32 && in_dtype != KVATTN_BF16)
    return fail(KVATTN_EINVAL, "%s: input dtype must be f32 or bf16", who);
  // query i of head h is virtual head h * n_q + i: q and out [batch, heads, n_q, d]
  // are [batch, heads * n_q, d], and the group becomes G * n_q
  return attn_decode_impl(who, cache, batch, num_q_heads * n_q, q, q_dtype, k_new, v_new, append ? in_dtype : -1,
                          seq_lens, max_seq_len, block_table, max_blocks, key_mask, key_mask_stride, scale, out,
                          workspace, workspace_bytes, part_tokens, stream, n_q);
}

int kvattn_attn_prefill(const kvattn_cache* cache, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t n_max, const void* q, const void* k, const void* v, int32_t dtype,
                        const int32_t* positions, const int32_t* q_lens, const int32_t* block_table,
                        int32_t max_blocks, const uint8_t* key_mask, int64_t key_mask_stride, int32_t causal,
                        int32_t attend_prefix, float scale, float* out, void* stream) {
  const char* who = "kvattn_attn_prefill";
  if (batch < 0 || batch > 65535 || n_max < 0)
    return fail(KVATTN_EINVAL, "%s: batch %d / n_max %d out of range", who, batch, n_max);
  if (dtype != KVATTN_F32 && dtype != KVATTN_BF16) return fail(KVATTN_EINVAL, "%s: dtype must be f32 or bf16", who);
  if (head_dim != 64 && head_dim != 128)
    return fail(KVATTN_EUNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", who, head_dim);
  if (!group_ok(num_q_heads, num_kv_heads) || num_q_heads > 65535)
    return fail(KVATTN_EUNSUPPORTED, "%s: %d query heads over %d KV heads: group must be 1, 2, 4 or 8", who,
                num_q_heads, num_kv_heads);
  kvattn::PrefillLaunch a{};
  if (cache) {
    int64_t cap = 0;
    int rc = make_view(who, cache, batch, block_table, max_blocks, &a.c, &cap);
    if (rc) return rc;
    if (cache->num_kv_heads != num_kv_heads || cache->head_dim != head_dim)
      return fail(KVATTN_EINVAL, "%s: cache shape (%d heads, d %d) differs from k/v (%d, %d)", who,
                  cache->num_kv_heads, cache->head_dim, num_kv_heads, head_dim);
    if (cache->dtype != dtype && cache->dtype != KVATTN_FP8_E4M3)
      return fail(KVATTN_EUNSUPPORTED, "%s: dtype %d cannot be written to a cache of dtype %d", who, dtype,
                  cache->dtype);
    a.has_cache = 1;
    a.cache_dtype = cache->dtype;
    a.k_scale = cache->k_scale;
    a.v_scale = cache->v_scale;
  } else if (attend_prefix) {
    return fail(KVATTN_EINVAL, "%s: attend_prefix needs a cache", who);
  }
  if ((int64_t)batch * n_max == 0) return ok();
  if (!q || !k || !v || !out) return fail(KVATTN_EINVAL, "%s: q, k, v and out are required", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(KVATTN_EINVAL, "%s: q/k/v/out not 16-byte aligned", who);
  if (key_mask && key_mask_stride < n_max)
    return fail(KVATTN_EINVAL, "%s: key_mask_stride %lld < n_max %d", who, (long long)key_mask_stride, n_max);
  a.dtype = dtype;
  a.head_dim = head_dim;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.n_max = n_max;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.positions = positions;
  a.q_lens = q_lens;
  a.key_mask = key_mask;
  a.key_mask_stride = key_mask_stride;
  a.causal = causal ? 1 : 0;
  a.attend_prefix = attend_prefix ? 1 : 0;
  a.scale = scale;
  a.out = out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // With the same element type in and out, the attention kernel writes the
  // cache itself (the bf16 MFMA kernel: each workgroup the rows of the query
  // tile it owns; the general kernel: each query row's wave of the group's
  // first head).  An fp8 cache (quantised rows) gets the append kernel first.
  a.write_cache = cache && cache->dtype == dtype;
  if (cache && !a.write_cache) {
    kvattn::AppendLaunch w{};
    w.c = a.c;
    w.cache_dtype = cache->dtype;
    w.in_dtype = dtype;
    w.head_dim = head_dim;
    w.batch = batch;
    w.num_kv_heads = num_kv_heads;
    w.n_new = n_max;
    w.k_new = a.k;
    w.v_new = a.v;
    w.k_scale = cache->k_scale;
    w.v_scale = cache->v_scale;
    w.positions = positions;
    w.n_valid = q_lens;
    int rc = kvattn::launch_append(w, s);
    if (rc) return fail(rc, "%s: cache write: %s", who, kvattn_status_string(rc));
  }
  int rc = kvattn::launch_prefill(a, s);
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

int kvattn_validate(const kvattn_cache* cache, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                    const int32_t* positions, const int32_t* block_table, int32_t max_blocks, int32_t* err_word,
                    void* stream) {
  const char* who = "kvattn_validate";
  if (batch < 0) return fail(KVATTN_EINVAL, "%s: batch < 0", who);
  kvattn::ValidateLaunch a{};
  int64_t cap = 0;
  int rc = make_view(who, cache, batch, block_table, max_blocks, &a.c, &cap);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!seq_lens || !err_word) return fail(KVATTN_EINVAL, "%s: seq_lens and err_word are required", who);
  a.batch = batch;
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.cap_tokens = cap;
  a.positions = positions;
  a.err_word = err_word;
  rc = kvattn::launch_validate(a, static_cast<hipStream_t>(stream));
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

int kvattn_reorder_rows(int32_t n_rows, const int32_t* perm, int32_t src_rows, const int32_t* src_table,
                        const int32_t* src_lens, int32_t max_blocks, int32_t* dst_table, int32_t* dst_lens,
                        void* stream) {
  const char* who = "kvattn_reorder_rows";
  if (n_rows < 0 || n_rows > 65535) return fail(KVATTN_EINVAL, "%s: n_rows %d out of range", who, n_rows);
  if (src_rows < 0) return fail(KVATTN_EINVAL, "%s: src_rows %d < 0", who, src_rows);
  if (max_blocks < 1 || max_blocks > (1 << 26))
    return fail(KVATTN_EINVAL, "%s: max_blocks %d out of range", who, max_blocks);
  if (!src_lens != !dst_lens) return fail(KVATTN_EINVAL, "%s: give both src_lens and dst_lens or neither", who);
  if (n_rows == 0) return ok();
  if (!perm || !src_table || !dst_table) return fail(KVATTN_EINVAL, "%s: perm and both tables are required", who);
  const int32_t* s0 = src_table;
  const int32_t* s1 = src_table + (int64_t)src_rows * max_blocks;
  if (src_rows && (const int32_t*)dst_table < s1 && s0 < (const int32_t*)dst_table + (int64_t)n_rows * max_blocks)
    return fail(KVATTN_EINVAL, "%s: dst_table overlaps src_table", who);
  kvattn::RowReorderLaunch a{n_rows, src_rows, max_blocks, perm, src_table, src_lens, dst_table, dst_lens};
  const int rc = kvattn::launch_reorder_rows(a, static_cast<hipStream_t>(stream));
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

int kvattn_reorder_cache(const kvattn_cache* src, const kvattn_cache* dst, int32_t n_rows, const int32_t* perm,
                         const int32_t* src_lens, int32_t* dst_lens, void* stream) {
  const char* who = "kvattn_reorder_cache";
  if (n_rows < 0 || n_rows > 65535) return fail(KVATTN_EINVAL, "%s: n_rows %d out of range", who, n_rows);
  kvattn::CacheView sv, dv;
  int64_t cap = 0;
  if (!src || !dst) return fail(KVATTN_EINVAL, "%s: cache descriptors are required", who);
  if (src->layout != KVATTN_CONTIGUOUS || dst->layout != KVATTN_CONTIGUOUS)
    return fail(KVATTN_EINVAL, "%s: both caches must be contiguous (a paged cache reorders its block table)", who);
  int rc = make_view(who, src, 0, nullptr, 0, &sv, &cap);
  if (rc) return rc;
  rc = make_view(who, dst, n_rows, nullptr, 0, &dv, &cap);
  if (rc) return rc;
  if (src->dtype != dst->dtype || src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim ||
      src->capacity != dst->capacity)
    return fail(KVATTN_EINVAL, "%s: caches differ in dtype, num_kv_heads, head_dim or capacity", who);
  if (dst_lens && !src_lens) return fail(KVATTN_EINVAL, "%s: dst_lens needs src_lens", who);
  if (n_rows == 0) return ok();
  if (!perm) return fail(KVATTN_EINVAL, "%s: perm is required", who);
  const int64_t sbytes = src->num_rows * sv.seq_stride;
  const int64_t dbytes = dst->num_rows * dv.seq_stride;
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const uint8_t* x = static_cast<const uint8_t*>(a);
    const uint8_t* y = static_cast<const uint8_t*>(b);
    return x < y + nb && y < x + na;
  };
  if (overlap(src->k, sbytes, dst->k, dbytes) || overlap(src->k, sbytes, dst->v, dbytes) ||
      overlap(src->v, sbytes, dst->k, dbytes) || overlap(src->v, sbytes, dst->v, dbytes))
    return fail(KVATTN_EINVAL, "%s: src and dst cache memory overlap", who);
  kvattn::CacheReorderLaunch a{};
  a.src_k = sv.k;
  a.src_v = sv.v;
  a.dst_k = dv.k;
  a.dst_v = dv.v;
  a.pos_bytes = sv.row_stride;
  a.capacity = (int32_t)src->capacity;
  a.num_kv_heads = src->num_kv_heads;
  a.n_rows = n_rows;
  a.src_rows = (int32_t)(src->num_rows < INT32_MAX ? src->num_rows : INT32_MAX);
  a.perm = perm;
  a.src_lens = src_lens;
  a.dst_lens = dst_lens;
  rc = kvattn::launch_reorder_cache(a, static_cast<hipStream_t>(stream));
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

int kvattn_copy_blocks(const kvattn_cache* cache, int32_t n, const int32_t* src_blocks, const int32_t* dst_blocks,
                       void* stream) {
  const char* who = "kvattn_copy_blocks";
  if (n < 0 || n > (1 << 24)) return fail(KVATTN_EINVAL, "%s: n %d out of range", who, n);
  if (!cache) return fail(KVATTN_EINVAL, "%s: cache descriptor is NULL", who);
  if (cache->layout != KVATTN_PAGED) return fail(KVATTN_EINVAL, "%s: cache must be paged", who);
  if (n == 0) return ok();
  if (!src_blocks || !dst_blocks) return fail(KVATTN_EINVAL, "%s: src_blocks and dst_blocks are required", who);
  kvattn::CacheView v;
  int64_t cap = 0;
  static const int32_t kNoTable = -1;  // make_view wants a table; block copies use none
  int rc = make_view(who, cache, 0, &kNoTable, 1, &v, &cap);
  if (rc) return rc;
  kvattn::BlockCopyLaunch a{v.k, v.v, v.block_stride, v.num_blocks, n, src_blocks, dst_blocks};
  rc = kvattn::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

int kvattn_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  const char* who = "kvattn_stream_read";
  if (bytes < 0 || bytes % 16 != 0) return fail(KVATTN_EINVAL, "%s: bytes %lld must be a multiple of 16", who,
                                                (long long)bytes);
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(KVATTN_EINVAL, "%s: src and sink are required", who);
  if (!aligned16(src)) return fail(KVATTN_EINVAL, "%s: src not 16-byte aligned", who);
  if (reinterpret_cast<uintptr_t>(sink) % 4 != 0) return fail(KVATTN_EINVAL, "%s: sink not 4-byte aligned", who);
  // one contiguous range per workgroup, 4 workgroups per compute unit
  // (fewer for a small buffer); ranges are whole 16 KB steps (1024 chunks
  // of 16 bytes) so only the last one is ragged
  const int64_t chunks = bytes / 16;
  const int64_t target = 4 * compute_units();
  int64_t per = (chunks + target - 1) / target;
  per = (per + 1023) / 1024 * 1024;
  const int64_t wgs = (chunks + per - 1) / per;  // every range starts below the end
  kvattn::StreamReadLaunch a{static_cast<const uint8_t*>(src), bytes, per, sink};
  int rc = kvattn::launch_stream_read(a, (int32_t)wgs, static_cast<hipStream_t>(stream));
  if (rc) return fail(rc, "%s: %s", who, kvattn_status_string(rc));
  return ok();
}

struct kvattn_pool {
  explicit kvattn_pool(int32_t n) : p(n) {}
  kvattn::BlockPool p;
};

kvattn_pool* kvattn_pool_create(int64_t num_blocks) {
  if (num_blocks < 1 || num_blocks > INT32_MAX) {
    fail(KVATTN_EINVAL, "kvattn_pool_create: num_blocks %lld out of range", (long long)num_blocks);
    return nullptr;
  }
  try {
    kvattn_pool* p = new kvattn_pool((int32_t)num_blocks);
    ok();
    return p;
  } catch (...) {
    fail(KVATTN_EINVAL, "kvattn_pool_create: out of host memory for %lld blocks", (long long)num_blocks);
    return nullptr;
  }
}

void kvattn_pool_destroy(kvattn_pool* pool) { delete pool; }

int64_t kvattn_pool_num_blocks(const kvattn_pool* pool) { return pool ? pool->p.num_blocks() : 0; }

int64_t kvattn_pool_num_free(const kvattn_pool* pool) { return pool ? pool->p.num_free() : 0; }

int32_t kvattn_pool_refcount(const kvattn_pool* pool, int32_t block) { return pool ? pool->p.refcount(block) : -1; }

}  // extern "C"

namespace {
// Runs one pool operation: NULL checks, status and message.
template <typename F>
int pool_call(const char* who, kvattn_pool* pool, bool args_ok, F f) {
  if (!pool) return fail(KVATTN_EINVAL, "%s: pool is NULL", who);
  if (!args_ok) return fail(KVATTN_EINVAL, "%s: a required array is NULL", who);
  std::string err;
  const int rc = f(&err);
  if (rc) return fail(rc, "%s: %s", who, err.c_str());
  return ok();
}
}  // namespace

extern "C" {

int kvattn_pool_alloc(kvattn_pool* pool, int32_t n, int32_t* ids) {
  return pool_call("kvattn_pool_alloc", pool, ids || n == 0,
                   [&](std::string* e) { return pool->p.alloc(n, ids, e); });
}

int kvattn_pool_retain(kvattn_pool* pool, int32_t n, const int32_t* ids) {
  return pool_call("kvattn_pool_retain", pool, ids || n == 0,
                   [&](std::string* e) { return pool->p.retain(n, ids, e); });
}

int kvattn_pool_release(kvattn_pool* pool, int32_t n, const int32_t* ids) {
  return pool_call("kvattn_pool_release", pool, ids || n == 0,
                   [&](std::string* e) { return pool->p.release(n, ids, e); });
}

int kvattn_pool_fork(kvattn_pool* pool, const int32_t* src_row, int32_t* dst_row, int32_t max_blocks,
                     int32_t length) {
  return pool_call("kvattn_pool_fork", pool, src_row && dst_row,
                   [&](std::string* e) { return pool->p.fork(src_row, dst_row, max_blocks, length, e); });
}

int kvattn_pool_free_seq(kvattn_pool* pool, int32_t* row, int32_t max_blocks, int32_t length) {
  return pool_call("kvattn_pool_free_seq", pool, row != nullptr,
                   [&](std::string* e) { return pool->p.free_seq(row, max_blocks, length, e); });
}

int kvattn_pool_prepare_append(kvattn_pool* pool, int32_t rows, int32_t* tables, int32_t max_blocks,
                               const int32_t* cur_lens, const int32_t* new_lens, int32_t* copy_src,
                               int32_t* copy_dst, int32_t* n_copies) {
  const bool args = n_copies && (rows == 0 || (tables && cur_lens && new_lens && copy_src && copy_dst));
  return pool_call("kvattn_pool_prepare_append", pool, args, [&](std::string* e) {
    return pool->p.prepare_append(rows, tables, max_blocks, cur_lens, new_lens, copy_src, copy_dst, n_copies, e);
  });
}

int kvattn_pool_reorder(kvattn_pool* pool, int32_t n_rows, const int32_t* perm, int32_t src_rows,
                        const int32_t* src_tables, const int32_t* src_lens, int32_t max_blocks,
                        int32_t* dst_tables, int32_t* dst_lens) {
  const bool args = (n_rows == 0 || (perm && dst_tables && dst_lens)) && (src_rows == 0 || (src_tables && src_lens));
  return pool_call("kvattn_pool_reorder", pool, args, [&](std::string* e) {
    return pool->p.reorder(n_rows, perm, src_rows, src_tables, src_lens, max_blocks, dst_tables, dst_lens, e);
  });
}

}  // extern "C"
