// Cache reorder and sharing: block-table row gathers (batch/beam reorder of
// a paged cache), contiguous-cache row gathers, and whole-block copies for
// copy-on-write.  Integer and byte moves only.
//
// "Transformer Attention Masks and KV-Cache Inference" (c86j224s.github.io),
// section "Batch and beam reorder": the cache follows the beam permutation.
// "KV Cache Fully Explained" (techblog.paldyn.com), section
// "(4) PagedAttention": shared prefix blocks, copy-on-write.
//
// The byte moves are HBM streams with no reuse: each workgroup copies one
// 16 KiB chunk of a contiguous segment, every thread keeping four 16-byte
// loads in flight before its four stores, so each load and store
// instruction of a wave covers 1 KiB of consecutive bytes.  Loads and
// stores are non-temporal (each byte is moved once; the cache is far larger
// than L2).  On MI355X, against plain loads and stores: a 2 GiB contiguous
// copy 5.7 -> 6.2 TB/s (non-temporal loads alone 6.0); the 32 KiB block
// copies of a copy-on-write batch +4% and a beam reorder +8% for the
// stores; 8 KiB or one contiguous range per workgroup were slower.
#include "launch.h"

namespace kvattn {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyChunk = (int64_t)kCopyThreads * kCopyUnroll * 16;  // bytes per workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bytes [c * kCopyChunk, min((c + 1) * kCopyChunk, n)) of one segment; n is
// a multiple of 16 and both ends 16-byte aligned.
__device__ __forceinline__ void copy_chunk(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n,
                                           int64_t c) {
  const int64_t base = c * kCopyChunk + (int64_t)threadIdx.x * 16;
  u32x4 x[kCopyUnroll];
#pragma unroll
  for (int k = 0; k < kCopyUnroll; ++k) {
    const int64_t o = base + (int64_t)k * kCopyThreads * 16;
    if (o < n) x[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + o));
  }
#pragma unroll
  for (int k = 0; k < kCopyUnroll; ++k) {
    const int64_t o = base + (int64_t)k * kCopyThreads * 16;
    if (o < n) __builtin_nontemporal_store(x[k], reinterpret_cast<u32x4*>(dst + o));
  }
}

// One thread per table entry of destination row blockIdx.y; entry
// max_blocks stands for the row's length.
__global__ void __launch_bounds__(256) reorder_rows_kernel(const RowReorderLaunch a) {
  const int i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j > a.max_blocks) return;
  const int p = a.perm[i];
  const bool valid = p >= 0 && p < a.src_rows;
  if (j < a.max_blocks) {
    a.dst_table[(int64_t)i * a.max_blocks + j] = valid ? a.src_table[(int64_t)p * a.max_blocks + j] : -1;
  } else if (a.dst_lens) {
    a.dst_lens[i] = valid ? a.src_lens[p] : 0;
  }
}

// grid: x = KV head * chunks_per_head + chunk, y = destination row, z = K/V.
__global__ void __launch_bounds__(kCopyThreads) reorder_cache_kernel(const CacheReorderLaunch a,
                                                                     int64_t chunks_per_head) {
  const int i = blockIdx.y;
  const int g = (int)(blockIdx.x / chunks_per_head);
  const int64_t c = blockIdx.x % chunks_per_head;
  const int p = a.perm[i];
  const bool valid = p >= 0 && p < a.src_rows;
  if (a.dst_lens && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) a.dst_lens[i] = valid ? a.src_lens[p] : 0;
  if (!valid) return;
  const int32_t L = a.src_lens ? min(max(a.src_lens[p], 0), a.capacity) : a.capacity;
  const int64_t n = (int64_t)L * a.pos_bytes;
  if (c * kCopyChunk >= n) return;
  const int64_t head_bytes = (int64_t)a.capacity * a.pos_bytes;
  const uint8_t* s = (blockIdx.z ? a.src_v : a.src_k) + ((int64_t)p * a.num_kv_heads + g) * head_bytes;
  uint8_t* d = (blockIdx.z ? a.dst_v : a.dst_k) + ((int64_t)i * a.num_kv_heads + g) * head_bytes;
  copy_chunk(s, d, n, c);
}

// grid: x = pair * chunks_per_block + chunk, y = K/V.
__global__ void __launch_bounds__(kCopyThreads) copy_blocks_kernel(const BlockCopyLaunch a,
                                                                   int64_t chunks_per_block) {
  const int64_t pair = blockIdx.x / chunks_per_block;
  const int64_t c = blockIdx.x % chunks_per_block;
  const int64_t s = a.src[pair], d = a.dst[pair];
  if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks || s == d) return;
  uint8_t* pool = blockIdx.y ? a.v : a.k;
  copy_chunk(pool + s * a.block_bytes, pool + d * a.block_bytes, a.block_bytes, c);
}

int64_t chunks(int64_t bytes) { return (bytes + kCopyChunk - 1) / kCopyChunk; }

}  // namespace

int launch_reorder_rows(const RowReorderLaunch& a, hipStream_t s) {
  if (a.n_rows <= 0) return KVATTN_OK;
  hipLaunchKernelGGL(reorder_rows_kernel, dim3((a.max_blocks + 1 + 255) / 256, a.n_rows), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

int launch_reorder_cache(const CacheReorderLaunch& a, hipStream_t s) {
  if (a.n_rows <= 0) return KVATTN_OK;
  const int64_t cph = chunks((int64_t)a.capacity * a.pos_bytes);
  const int64_t gx = cph * a.num_kv_heads;
  if (gx > INT32_MAX) return KVATTN_EUNSUPPORTED;
  hipLaunchKernelGGL(reorder_cache_kernel, dim3((uint32_t)gx, a.n_rows, 2), dim3(kCopyThreads), 0, s, a, cph);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

int launch_copy_blocks(const BlockCopyLaunch& a, hipStream_t s) {
  if (a.n <= 0) return KVATTN_OK;
  const int64_t cpb = chunks(a.block_bytes);
  const int64_t gx = cpb * a.n;
  if (gx > INT32_MAX) return KVATTN_EUNSUPPORTED;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)gx, 2), dim3(kCopyThreads), 0, s, a, cpb);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

}  // namespace kvattn
