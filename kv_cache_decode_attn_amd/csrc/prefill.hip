// Prefill attention: many new tokens per sequence, causal and/or padding
// masked, optionally also attending a cached prefix.
//
// What is computed ("Transformer Attention Masks and KV-Cache Inference"
// (c86j224s.github.io), sections "State of scaled dot-product attention",
// "Padding mask and batch length", "Causal mask and future positions" and
// "Prefill and decode stages"): query t of sequence b, at absolute position
// P + t, attends key positions s with lo <= s < P + q_len, s <= P + t when
// causal, and key_mask[b, s] != 0; lo = 0 when the cached prefix is attended,
// else P.  Keys s >= P are the new tokens, s < P are read from the cache.
//
// This file holds the general kernel: any supported dtype and head_dim,
// fp32 arithmetic throughout, one wave per (query row, head, sequence),
// keys visited 64 at a time with the running (max, sum) update of "KV Cache,
// Flash Attention and Inference Optimization" (factory.pai-world.com),
// section "Build it", step 2.  It serves fp32 inputs, prefix-attending
// calls and shapes the MFMA kernel does not cover.  The bf16 MFMA kernel is
// in prefill_mfma.hip.
#include <math.h>

#include "launch.h"

namespace kvattn {

int launch_prefill_mfma(const PrefillLaunch& a, hipStream_t s);  // prefill_mfma.hip

namespace {

template <int DT>
__device__ __forceinline__ float load_elem(const uint8_t* row, int d) {
  if constexpr (DT == KVATTN_F32) {
    return reinterpret_cast<const float*>(row)[d];
  } else if constexpr (DT == KVATTN_BF16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(row)[d];
    return __uint_as_float((uint32_t)h << 16);
  } else {
    float f[4];
    fp8x4_to_f32((uint32_t)row[d], f);
    return f[0];
  }
}

constexpr int kDtypeBytes[3] = {4, 2, 1};

// Row pointer of key position s for (b, g): new tokens (s >= P) or the
// cache (s < P).  Returns nullptr for a cache position outside the cache.
struct KeySource {
  const uint8_t* newk;
  const uint8_t* newv;
  int64_t new_row_bytes;
  const PrefillLaunch* a;
  int P;
  int b, g;
  __device__ const uint8_t* row(bool value, int64_t s, bool& from_cache) const {
    if (s >= P) {
      from_cache = false;
      return (value ? newv : newk) + (s - P) * new_row_bytes;
    }
    from_cache = true;
    const int64_t off = position_offset(a->c, b, g, s);
    if (off < 0) return nullptr;
    return (value ? a->c.v : a->c.k) + off;
  }
};

template <int DT, int CDT, int D>
__global__ void __launch_bounds__(64) prefill_generic(const PrefillLaunch a) {
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int g = h / G;
  const int qlen = a.q_lens ? min(max(a.q_lens[b], 0), a.n_max) : a.n_max;
  float* orow = a.out + (((int64_t)b * a.num_q_heads + h) * a.n_max + t) * D;
  if (t >= qlen) {
    for (int d = lane; d < D; d += 64) orow[d] = 0.f;
    return;
  }
  const int P = a.positions ? max(a.positions[b], 0) : 0;
  const int64_t lo = a.attend_prefix ? 0 : P;
  const int64_t hi = a.causal ? (int64_t)P + t + 1 : (int64_t)P + qlen;

  __shared__ float qs[D];
  __shared__ float ps[64];
  constexpr int ES = kDtypeBytes[DT];
  const uint8_t* qrow = a.q + (((int64_t)b * a.num_q_heads + h) * a.n_max + t) * D * ES;
  for (int d = lane; d < D; d += 64) qs[d] = load_elem<DT>(qrow, d);
  __syncthreads();

  KeySource src;
  src.newk = a.k + ((int64_t)b * a.num_kv_heads + g) * a.n_max * D * ES;
  src.newv = a.v + ((int64_t)b * a.num_kv_heads + g) * a.n_max * D * ES;
  src.new_row_bytes = (int64_t)D * ES;
  src.a = &a;
  src.P = P;
  src.b = b;
  src.g = g;
  float kscale = 1.f, vscale = 1.f;
  if constexpr (CDT == KVATTN_FP8_E4M3) {
    kscale = a.k_scale[g];
    vscale = a.v_scale[g];
  }
  const uint8_t* mask_row = a.key_mask ? a.key_mask + (int64_t)b * a.key_mask_stride : nullptr;

  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int64_t s0 = lo; s0 < hi; s0 += 64) {
    const int64_t s = s0 + lane;
    float z = -INFINITY;
    // a key beyond the mask row (stride) counts as blocked
    if (s < hi && (!mask_row || (s < a.key_mask_stride && mask_row[s] != 0))) {
      bool cached;
      const uint8_t* kr = src.row(false, s, cached);
      if (kr) {
        float acc = 0.f;
        if (cached) {
          for (int d = 0; d < D; ++d) acc = fmaf(qs[d], load_elem<CDT>(kr, d) * kscale, acc);
        } else {
          for (int d = 0; d < D; ++d) acc = fmaf(qs[d], load_elem<DT>(kr, d), acc);
        }
        z = acc * a.scale;
      }
    }
    const float cm = group_max<64>(z);
    const float nm = fmaxf(m, cm);
    if (nm == -INFINITY) continue;  // nothing allowed yet (uniform across the wave)
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - nm);
    const float pz = (z == -INFINITY) ? 0.f : expf(z - nm);
    l = l * alpha + group_sum<64>(pz);
    ps[lane] = pz;
    __syncthreads();
    o0 *= alpha;
    o1 *= alpha;
    const int nk = (int)min((int64_t)64, hi - s0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = ps[jj];
      if (pj == 0.f) continue;  // masked keys never touch V
      bool cached;
      const uint8_t* vr = src.row(true, s0 + jj, cached);
      if (!vr) continue;
      if (cached) {
        o0 = fmaf(pj, load_elem<CDT>(vr, lane) * vscale, o0);
        if (D > 64) o1 = fmaf(pj, load_elem<CDT>(vr, lane + 64) * vscale, o1);
      } else {
        o0 = fmaf(pj, load_elem<DT>(vr, lane), o0);
        if (D > 64) o1 = fmaf(pj, load_elem<DT>(vr, lane + 64), o1);
      }
    }
    m = nm;
    __syncthreads();
  }
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  orow[lane] = o0 * inv;
  if (D > 64) orow[lane + 64] = o1 * inv;

  // Cache write (same element type in and out: the bits are copied): the
  // wave of the group's first query head stores new row t of its KV head at
  // position P + t, as kv_append would; skipped outside the cache.  The
  // attention above never reads these positions from the cache.
  if (a.write_cache && h % G == 0) {
    const int64_t off = position_offset(a.c, b, g, (int64_t)P + t);
    if (off >= 0) {
      constexpr int W = D * ES / 4;  // 32-bit words per row
      const uint32_t* ks = reinterpret_cast<const uint32_t*>(src.newk + (int64_t)t * D * ES);
      const uint32_t* vs = reinterpret_cast<const uint32_t*>(src.newv + (int64_t)t * D * ES);
      uint32_t* kd = reinterpret_cast<uint32_t*>(a.c.k + off);
      uint32_t* vd = reinterpret_cast<uint32_t*>(a.c.v + off);
      for (int w = lane; w < W; w += 64) {
        kd[w] = ks[w];
        vd[w] = vs[w];
      }
    }
  }
}

template <int DT, int CDT, int D>
int launch_generic(const PrefillLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_generic<DT, CDT, D>), dim3(a.n_max, a.num_q_heads, a.batch), dim3(64), 0, s, a);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

template <int DT, int CDT>
int launch_generic_dim(const PrefillLaunch& a, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return launch_generic<DT, CDT, 64>(a, s);
    case 128: return launch_generic<DT, CDT, 128>(a, s);
    default: return KVATTN_EUNSUPPORTED;
  }
}

template <int DT>
int launch_generic_cache(const PrefillLaunch& a, hipStream_t s) {
  // The cache element type only matters when the prefix is read from it.
  const int cdt = (a.has_cache && a.attend_prefix) ? a.cache_dtype : DT;
  switch (cdt) {
    case KVATTN_F32: return launch_generic_dim<DT, KVATTN_F32>(a, s);
    case KVATTN_BF16: return launch_generic_dim<DT, KVATTN_BF16>(a, s);
    case KVATTN_FP8_E4M3: return launch_generic_dim<DT, KVATTN_FP8_E4M3>(a, s);
    default: return KVATTN_EUNSUPPORTED;
  }
}

}  // namespace

int launch_prefill(const PrefillLaunch& a, hipStream_t s) {
  if (a.n_max == 0 || a.batch == 0) return KVATTN_OK;
  if (prefill_mfma_supports(a)) return launch_prefill_mfma(a, s);
  switch (a.dtype) {
    case KVATTN_F32: return launch_generic_cache<KVATTN_F32>(a, s);
    case KVATTN_BF16: return launch_generic_cache<KVATTN_BF16>(a, s);
    default: return KVATTN_EUNSUPPORTED;
  }
}

}  // namespace kvattn
