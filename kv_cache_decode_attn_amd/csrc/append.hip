// Cache writes (kv_append) and the metadata contract check (validate).
//
// kv_append implements the "append" half of append-then-attend: the new
// tokens' K and V join the layer's cache at their absolute positions
// ("Transformer Attention Masks and KV-Cache Inference" (c86j224s.github.io),
// sections "Prefill and decode stages" and "Position IDs and the append
// contract"), through the 16-token block table when the cache is paged
// ("KV Cache, Flash Attention and Inference Optimization"
// (factory.pai-world.com), section "PagedAttention").  Integer address work
// only, plus the E4M3FN encoder for an 8-bit cache ("KV Cache Fully
// Explained" (techblog.paldyn.com), section "(1) FP8 quantization").
//
// One thread moves one 16-byte chunk of an input row (8 bf16 or 4 fp32
// elements), so a wave writes whole rows with coalesced stores.
#include "launch.h"

namespace kvattn {
namespace {

template <int IN, int OUT>
__global__ void __launch_bounds__(256) kv_append_kernel(const AppendLaunch a, int64_t total) {
  constexpr int IES = (IN == KVATTN_F32) ? 4 : 2;  // input element bytes
  constexpr int CE = 16 / IES;                     // elements per chunk
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int D = a.head_dim;
  const int cpr = D / CE;  // chunks per row
  // idx -> (b, g, i, kv, chunk), chunk fastest
  int64_t r = idx;
  const int chunk = (int)(r % cpr);
  r /= cpr;
  const int kv = (int)(r % 2);
  r /= 2;
  const int i = (int)(r % a.n_new);
  r /= a.n_new;
  const int g = (int)(r % a.num_kv_heads);
  const int b = (int)(r / a.num_kv_heads);

  int nb = a.n_new;
  if (a.n_valid) nb = min(max(a.n_valid[b], 0), a.n_new);
  if (i >= nb) return;
  const int64_t p = (int64_t)(a.positions ? a.positions[b] : 0) + i;
  const int64_t off = position_offset(a.c, b, g, p);
  if (off < 0) return;  // outside the cache: skipped (reported by validate)

  const uint8_t* src = (kv ? a.v_new : a.k_new) +
                       ((((int64_t)b * a.num_kv_heads + g) * a.n_new + i) * D + (int64_t)chunk * CE) * IES;
  uint8_t* dst = (kv ? a.c.v : a.c.k) + off;
  const U4 x = *reinterpret_cast<const U4*>(src);
  if constexpr (OUT == IN) {
    *reinterpret_cast<U4*>(dst + (int64_t)chunk * 16) = x;
  } else {
    static_assert(OUT == KVATTN_FP8_E4M3, "conversion");
    const float s = (kv ? a.v_scale : a.k_scale)[g];
    if constexpr (IN == KVATTN_BF16) {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      U2 out;
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[2 * e] = f32_to_e4m3(bf16_lo(w[e]) / s);
        c[2 * e + 1] = f32_to_e4m3(bf16_hi(w[e]) / s);
      }
      out.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      out.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      *reinterpret_cast<U2*>(dst + (int64_t)chunk * 8) = out;
    } else {
      const uint32_t c0 = f32_to_e4m3(__uint_as_float(x.x) / s);
      const uint32_t c1 = f32_to_e4m3(__uint_as_float(x.y) / s);
      const uint32_t c2 = f32_to_e4m3(__uint_as_float(x.z) / s);
      const uint32_t c3 = f32_to_e4m3(__uint_as_float(x.w) / s);
      *reinterpret_cast<uint32_t*>(dst + (int64_t)chunk * 4) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  }
}

template <int IN, int OUT>
int launch_typed(const AppendLaunch& a, hipStream_t s) {
  const int ce = (IN == KVATTN_F32) ? 4 : 8;
  const int64_t total = (int64_t)a.batch * a.num_kv_heads * a.n_new * 2 * (a.head_dim / ce);
  if (total == 0) return KVATTN_OK;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL((kv_append_kernel<IN, OUT>), dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

// Checks of the metadata contract; one thread per sequence.
__global__ void validate_kernel(const ValidateLaunch a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  int err = 0;
  const int len = a.seq_lens[b];
  if (len < 0 || len > a.max_seq_len || (int64_t)len > a.cap_tokens) err |= KVATTN_VALIDATE_LEN_RANGE;
  if (a.c.paged) {
    const int64_t used = ((int64_t)max(len, 0) + kBlockTokens - 1) / kBlockTokens;
    const int64_t nchk = used < a.c.max_blocks ? used : a.c.max_blocks;
    for (int64_t j = 0; j < nchk; ++j) {
      const int32_t blk = a.c.block_table[(int64_t)b * a.c.max_blocks + j];
      if (blk < 0 || (int64_t)blk >= a.c.num_blocks) err |= KVATTN_VALIDATE_BLOCK_RANGE;
    }
  }
  if (a.positions && a.positions[b] != len) err |= KVATTN_VALIDATE_POSITION;
  if (err) atomicOr(a.err_word, err);
}

}  // namespace

int launch_append(const AppendLaunch& a, hipStream_t s) {
  if (a.in_dtype == a.cache_dtype) {
    if (a.in_dtype == KVATTN_F32) return launch_typed<KVATTN_F32, KVATTN_F32>(a, s);
    if (a.in_dtype == KVATTN_BF16) return launch_typed<KVATTN_BF16, KVATTN_BF16>(a, s);
    return KVATTN_EUNSUPPORTED;
  }
  if (a.cache_dtype == KVATTN_FP8_E4M3) {
    if (a.in_dtype == KVATTN_BF16) return launch_typed<KVATTN_BF16, KVATTN_FP8_E4M3>(a, s);
    if (a.in_dtype == KVATTN_F32) return launch_typed<KVATTN_F32, KVATTN_FP8_E4M3>(a, s);
  }
  return KVATTN_EUNSUPPORTED;
}

int launch_validate(const ValidateLaunch& a, hipStream_t s) {
  if (a.batch <= 0) return KVATTN_OK;
  hipLaunchKernelGGL(validate_kernel, dim3((a.batch + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

}  // namespace kvattn
