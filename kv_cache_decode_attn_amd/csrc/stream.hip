// A plain streaming read of device memory: the context figure for the
// HBM-bound kernels of the library (what one pass over contiguous bytes
// reaches on this GPU, against the 8 TB/s peak).  Decode is bound by
// reading the cache once per step ("KV Cache" (heepie.pages.dev), section
// "Prefill and Decode"), so this is the ceiling its kernels are compared
// with.
//
// Each workgroup reads one contiguous range of the buffer (a multiple of
// 16 KB; the last one takes the ragged tail): its threads read 16-byte
// chunks with non-temporal loads, four in flight, so a wave reads 1 KB
// contiguous per instruction and the workgroup walks its range in 16 KB
// steps.  Contiguous ranges per workgroup read faster on this GPU than a
// grid-stride walk of the whole buffer (about 7.0 against 6.1-6.4 TB/s
// measured on a 4 GiB buffer), so this is the faster of the two plain
// forms.  The chunks fold into one 32-bit XOR; each wave XORs its lanes'
// words into *sink with one atomic, so the loads cannot be dropped and the
// result is checkable bit for bit.
#include "launch.h"

namespace kvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(const u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ void __launch_bounds__(256) stream_read_kernel(const StreamReadLaunch a) {
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src);
  const int64_t n = a.bytes / 16;
  const int64_t lo = (int64_t)blockIdx.x * a.chunks_per_wg;
  const int64_t hi = lo + a.chunks_per_wg < n ? lo + a.chunks_per_wg : n;
  int64_t i = lo + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * 256 < hi; i += 4 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * 256);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * 256);
    x ^= fold(v0) ^ fold(v1) ^ fold(v2) ^ fold(v3);
  }
  for (; i < hi; i += 256) x ^= fold(__builtin_nontemporal_load(src + i));
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0 && x != 0) atomicXor(a.sink, x);
}

}  // namespace

int launch_stream_read(const StreamReadLaunch& a, int32_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

}  // namespace kvattn
