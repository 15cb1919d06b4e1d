// Shared device helpers of the kvattn HIP library (gfx950, wave64).
//
// Element formats, 64-lane reductions built on DPP row operations, and the
// OCP FP8 E4M3FN encoder used when the cache is stored at 8 bits ("KV Cache
// Fully Explained" (techblog.paldyn.com), section "(1) FP8 quantization").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvattn.h"

namespace kvattn {

constexpr int kWave = 64;
constexpr int kBlockTokens = KVATTN_BLOCK_TOKENS;

struct alignas(16) U4 {
  uint32_t x, y, z, w;
};
struct alignas(8) U2 {
  uint32_t x, y;
};

// ---------------------------------------------------------------- formats ---

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two OCP E4M3FN codes (byte 0/1 or byte 2/3 of w) -> two floats, exactly.
// gfx950's v_cvt_pk_f32_fp8 decodes the OCP format.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// Four OCP E4M3FN codes -> two words of two bf16 each (codes 0, 1 and codes
// 2, 3), exactly: every E4M3FN value is a bf16 value, and gfx950 converts a
// pair of codes to a bf16 pair in one instruction (scale 1).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
#else
  lo = hi = w;
#endif
}

// float -> OCP E4M3FN code: round to nearest, ties to even, saturate to
// +-448, NaN -> 0x7F, sign of x kept.  Written on the fp32 bit pattern:
// magnitudes below 2^-6 are subnormal codes in steps of 2^-9; above that the
// fp32 mantissa is rounded to 3 bits and the exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;           // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;   // |x| >= 448, inf: saturate
  if (a < 0x3c800000u) {                       // |x| < 2^-6: subnormal range
    const float y = __uint_as_float(a) * 512.0f;  // exact: |x| / 2^-9
    return sign | (uint32_t)__builtin_rintf(y);   // 0..8, ties to even
  }
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // RNE to 3 mantissa bits
  return sign | (r - (120u << 3));                             // exponent bias 127 -> 7
}

// ------------------------------------------------------------ reductions ---

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1] exchange lanes at
// distance 1 and 2 inside a quad; row_half_mirror pairs each quad of an
// 8-lane half-row with the other quad; row_mirror pairs the two halves of a
// 16-lane row.  Applied in that order, every lane of an N-lane group
// (N <= 16) ends with the group total.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over aligned groups of N consecutive lanes; result in every lane.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
  if constexpr (N >= 2) x += dpp_f<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_f<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_f<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_f<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f<kDppMirror>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Sum over the lanes that share (lane % STRIDE), i.e. across the 64/STRIDE
// groups of STRIDE lanes; result in every lane.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
  if constexpr (STRIDE <= 1) return group_sum<64>(x);
  if constexpr (STRIDE <= 2) x += __shfl_xor(x, 2);
  if constexpr (STRIDE <= 4) x += __shfl_xor(x, 4);
  if constexpr (STRIDE <= 8) x += __shfl_xor(x, 8);
  if constexpr (STRIDE <= 16) x += __shfl_xor(x, 16);
  if constexpr (STRIDE <= 32) x += __shfl_xor(x, 32);
  return x;
}

// ------------------------------------------------------------- addressing ---

// View of one layer's cache as the kernels see it.
struct CacheView {
  uint8_t* k;
  uint8_t* v;
  int64_t row_stride;     // bytes between consecutive positions (head_dim * elem)
  int64_t head_stride;    // contiguous: capacity * row; paged: 16 * row
  int64_t seq_stride;     // contiguous: Hkv * capacity * row (per sequence row)
  int64_t block_stride;   // paged: Hkv * 16 * row (per physical block)
  int64_t capacity;       // contiguous positions per row
  int64_t num_blocks;     // paged pool size
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t paged;
};

// Byte offset of the first position of the 16-token block `j` of sequence b,
// KV head g, or -1 if the block lies outside the cache.
__device__ __forceinline__ int64_t block_offset(const CacheView& c, int b, int g, int j) {
  if (c.paged) {
    if (j < 0 || j >= c.max_blocks) return -1;
    const int32_t blk = c.block_table[(int64_t)b * c.max_blocks + j];
    if (blk < 0 || (int64_t)blk >= c.num_blocks) return -1;
    return (int64_t)blk * c.block_stride + (int64_t)g * c.head_stride;
  }
  // contiguous capacity is a multiple of 16 (checked on the host)
  if (j < 0 || (int64_t)(j + 1) * kBlockTokens > c.capacity) return -1;
  return (int64_t)b * c.seq_stride + (int64_t)g * c.head_stride + (int64_t)j * kBlockTokens * c.row_stride;
}

// Byte offset of position p of sequence b, KV head g, or -1 if outside.
__device__ __forceinline__ int64_t position_offset(const CacheView& c, int b, int g, int64_t p) {
  if (p < 0) return -1;
  if (c.paged) {
    const int64_t j = p / kBlockTokens;
    if (j >= c.max_blocks) return -1;
    const int32_t blk = c.block_table[(int64_t)b * c.max_blocks + j];
    if (blk < 0 || (int64_t)blk >= c.num_blocks) return -1;
    return (int64_t)blk * c.block_stride + (int64_t)g * c.head_stride + (p % kBlockTokens) * c.row_stride;
  }
  if (p >= c.capacity) return -1;
  return (int64_t)b * c.seq_stride + (int64_t)g * c.head_stride + p * c.row_stride;
}

}  // namespace kvattn
