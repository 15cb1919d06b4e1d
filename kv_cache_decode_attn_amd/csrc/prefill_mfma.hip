// bf16 prefill attention on MFMA (gfx950 v_mfma_f32_16x16x32_bf16).
//
// What is computed is the masked scaled dot-product attention of the new
// tokens ("Transformer Attention Masks and KV-Cache Inference"
// (c86j224s.github.io), sections "State of scaled dot-product attention",
// "Padding mask and batch length" and "Causal mask and future positions"),
// tiled so that no n x n score matrix is stored and every K/V tile makes one
// trip from HBM ("KV Cache, Flash Attention and Inference Optimization"
// (factory.pai-world.com), section "Flash Attention - tiling trick"), with
// the exact running (max, sum) rescaling of its numerical-trick paragraph.
// Prefill is compute bound ("KV Cache" (heepie.pages.dev), section "Prefill
// and Decode"), so both products run on the matrix cores.
//
// Work split.  A workgroup of 4 waves owns HW = min(G, 4) query heads of one
// KV head and a tile of 32 * 4 / HW query rows; each wave owns one head and
// 32 query rows.  The heads of a GQA group share the K/V tiles staged in LDS.
// Causal tiles are issued heaviest first.
//
// Per 32-key tile, per wave:
//   S^T[key][q] = K Q^T      A = K rows from LDS, B = Q (registers), fp32 acc.
//                            The accumulator layout (lane l holds rows
//                            4*(l/16)+r, column l%16) puts each query in one
//                            lane column, so the row max needs only two
//                            cross-lane steps and P^T is already the B
//                            operand of the second product.
//   P = exp2(S*c - m)        c = scale*log2(e); m is a per-query running
//                            maximum that is only raised (with rescaling of
//                            the accumulators) when the tile maximum exceeds
//                            it by more than 8, so P <= 2^8; P rounded to bf16.
//   O^T[d][q] += V^T P^T     A = V^T from LDS.  V is transposed while it is
//                            staged into LDS; its key order inside an LDS row
//                            follows the key order of P^T's operand slots.
//   l[q] += 1 . P^T          an MFMA against a ones operand, so the row sum
//                            is the sum of the same bf16 weights used for O.
// Masked keys (causal, beyond q_len, key_mask) get P = 0 and their V rows are
// staged as zeros, so non-finite padding never reaches O.
#include <math.h>

#include "launch.h"

namespace kvattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKeys = 32;      // keys per tile
constexpr int kWaveQ = 32;     // query rows per wave
constexpr int kThreads = 256;  // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;  // log2 headroom before the running max moves

__device__ __forceinline__ f32x4 mfma(const U4& a, const U4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;  // round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// LDS geometry (bytes).  K rows are padded to 68 dwords and V^T rows to 20
// dwords so that 16 lanes reading 16 consecutive rows at one column touch 16
// disjoint groups of 4 banks.
template <int D>
struct Geo {
  static constexpr int KROW = D * 2 + 16;
  static constexpr int VROW = kKeys * 2 + 16;
  static constexpr int KBYTES = kKeys * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
};

// Slot of key k (0..31) inside a V^T row: the PV operand of lane group lg
// holds keys 4lg..4lg+3 (from the first 16-key score tile) then
// 16+4lg..16+4lg+3 (second tile), as 8 consecutive bf16.
__device__ __forceinline__ int vslot(int k) { return 8 * ((k & 15) >> 2) + (k & 3) + 4 * (k >> 4); }

template <int D, bool CAUSAL, bool MASK>
__global__ void __launch_bounds__(kThreads, 2) prefill_mfma_kernel(const PrefillLaunch a, int hw) {
  using GE = Geo<D>;
  constexpr int DC = D / 32;  // d chunks of the QK^T contraction
  constexpr int DT = D / 16;  // d tiles of the output
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int b = blockIdx.z;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int qw_per_head = 4 / hw;                  // 32-row sub-tiles per head
  const int wg_rows = kWaveQ * qw_per_head;
  const int qtile = gridDim.x - 1 - blockIdx.x;    // heaviest (causal) first
  const int h = blockIdx.y * hw + (wave % hw);
  const int g = (blockIdx.y * hw) / G;
  const int q_wg = qtile * wg_rows;
  const int q0 = q_wg + kWaveQ * (wave / hw);      // this wave's first row
  const int n_max = a.n_max;
  const int qlen = a.q_lens ? min(max(a.q_lens[b], 0), n_max) : n_max;
  const int P = a.positions ? max(a.positions[b], 0) : 0;

  float* out_h = a.out + ((int64_t)b * a.num_q_heads + h) * n_max * D;
  if (q_wg >= qlen) {  // the whole tile is padding rows: zeros
    for (int r = 0; r < kWaveQ; ++r) {
      const int t = q0 + r;
      if (t < n_max)
        for (int d = lane; d < D; d += 64) out_h[(int64_t)t * D + d] = 0.f;
    }
    return;
  }
  const int key_end = CAUSAL ? min(qlen, q_wg + wg_rows) : qlen;  // workgroup bound
  const int wave_end = CAUSAL ? min(qlen, q0 + kWaveQ) : qlen;     // this wave's bound
  const int ntiles = (key_end + kKeys - 1) / kKeys;

  const uint8_t* kg = a.k + ((int64_t)b * a.num_kv_heads + g) * n_max * D * 2;
  const uint8_t* vg = a.v + ((int64_t)b * a.num_kv_heads + g) * n_max * D * 2;
  const uint8_t* qg = a.q + ((int64_t)b * a.num_q_heads + h) * n_max * D * 2;
  const uint8_t* mrow = MASK ? a.key_mask + (int64_t)b * a.key_mask_stride : nullptr;

  // ---- Q fragments (B operand of S^T = K Q^T): rows q0 + 16 qt + lc ----
  U4 qf[2][DC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int t = q0 + 16 * qt + lc;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (t < n_max)
        qf[qt][dc] = *reinterpret_cast<const U4*>(qg + ((int64_t)t * D + 32 * dc + 8 * lg) * 2);
      else
        qf[qt][dc] = U4{0, 0, 0, 0};
    }
  }

  // ---- staging of one K/V tile: global -> registers -> LDS ----
  // K: 32 rows x D*2 bytes = 32*D/8 chunks of 16 B; thread handles chunks
  // tid, tid + 256 (D = 128) or tid (D = 64).
  constexpr int KCH = kKeys * D / 8 / kThreads;  // 16-byte K chunks per thread
  // V: thread handles keys (2m, 2m+1) x 8 columns d in [8 dg, 8 dg + 8);
  // 16 key pairs x D/8 column groups = 2*D threads (D = 64: half the block).
  const int vm = tid & 15, vdg = tid >> 4;
  const bool v_active = vdg < D / 8;
  U4 kreg[KCH], vreg[2];

  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = tid + c * kThreads;
      const int key = kt0 + ch / (D / 8);
      const int col = ch % (D / 8);
      kreg[c] = (key < n_max) ? *reinterpret_cast<const U4*>(kg + ((int64_t)key * D + col * 8) * 2) : U4{0, 0, 0, 0};
    }
    if (v_active) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = kt0 + 2 * vm + e;
        bool live = key < qlen;
        if (MASK && live) live = (P + key < a.key_mask_stride) && mrow[P + key] != 0;
        vreg[e] = live ? *reinterpret_cast<const U4*>(vg + ((int64_t)key * D + 8 * vdg) * 2) : U4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* kl = smem + buf * GE::BUF;
    uint8_t* vl = kl + GE::KBYTES;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = tid + c * kThreads;
      *reinterpret_cast<U4*>(kl + (ch / (D / 8)) * GE::KROW + (ch % (D / 8)) * 16) = kreg[c];
    }
    if (v_active) {
      // transpose 2 keys x 8 columns into 8 dwords (key 2m low, 2m+1 high)
      const uint32_t x0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t x1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const int slot = vslot(2 * vm);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_amdgcn_perm(x1[i], x0[i], 0x05040100u);  // column 2i
        const uint32_t hi = __builtin_amdgcn_perm(x1[i], x0[i], 0x07060302u);  // column 2i+1
        *reinterpret_cast<uint32_t*>(vl + (8 * vdg + 2 * i) * GE::VROW + slot * 2) = lo;
        *reinterpret_cast<uint32_t*>(vl + (8 * vdg + 2 * i + 1) * GE::VROW + slot * 2) = hi;
      }
    }
  };

  // ---- accumulators ----
  f32x4 o[DT][2], lsum[2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  lsum[0] = lsum[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {-INFINITY, -INFINITY};
  const float c = a.scale * kLog2e;
  const uint32_t one2 = 0x3F803F80u;  // two bf16 1.0
  const U4 ones = U4{one2, one2, one2, one2};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int kt0 = it * kKeys;
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile(kt0 + kKeys);
    if (kt0 < wave_end) {
      const uint8_t* kl = smem + buf * GE::BUF;
      const uint8_t* vl = kl + GE::KBYTES;
      // S^T for keys kt0 + 16 kk + 4 lg + r, queries q0 + 16 qt + lc
      f32x4 s[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        s[kk][0] = s[kk][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const U4 kf = *reinterpret_cast<const U4*>(kl + (16 * kk + lc) * GE::KROW + (32 * dc + 8 * lg) * 2);
          s[kk][0] = mfma(kf, qf[0][dc], s[kk][0]);
          s[kk][1] = mfma(kf, qf[1][dc], s[kk][1]);
        }
      }
      // masking: causal edge, keys beyond q_len, key mask
      const bool edge = (kt0 + kKeys > qlen) || (CAUSAL && kt0 + kKeys - 1 > q0);
      if (MASK || edge) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kt0 + 16 * kk + 4 * lg + r;
            bool kv = key < qlen;
            if (MASK && kv) kv = (P + key < a.key_mask_stride) && mrow[P + key] != 0;
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
              const int t = q0 + 16 * qt + lc;
              const bool ok = kv && (!CAUSAL || key <= t);
              if (!ok) s[kk][qt][r] = -INFINITY;
            }
          }
      }
      // running maximum per query (log2 domain), raised lazily
      U4 pf[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float tm = fmaxf(fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), fmaxf(s[0][qt][2], s[0][qt][3])),
                         fmaxf(fmaxf(s[1][qt][0], s[1][qt][1]), fmaxf(s[1][qt][2], s[1][qt][3])));
        tm = fmaxf(tm, __shfl_xor(tm, 16));
        tm = fmaxf(tm, __shfl_xor(tm, 32));
        tm *= c;
        const bool need = tm > mrun[qt] + kRescale;
        if (__any(need)) {
          const float mnew = need ? tm : mrun[qt];
          const float alpha = need ? exp2f(mrun[qt] - mnew) : 1.f;  // 0 when mrun = -inf
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][qt] *= alpha;
          lsum[qt] *= alpha;
          mrun[qt] = mnew;
        }
        const float msub = (mrun[qt] == -INFINITY) ? 0.f : mrun[qt];
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(s[0][qt][r], c, -msub));
          p[4 + r] = __builtin_amdgcn_exp2f(fmaf(s[1][qt][r], c, -msub));
        }
        pf[qt] = U4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
      }
      // O^T += V^T P^T ; l += 1 . P^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const U4 vf = *reinterpret_cast<const U4*>(vl + (16 * dt + lc) * GE::VROW + 16 * lg);
        o[dt][0] = mfma(vf, pf[0], o[dt][0]);
        o[dt][1] = mfma(vf, pf[1], o[dt][1]);
      }
      lsum[0] = mfma(ones, pf[0], lsum[0]);
      lsum[1] = mfma(ones, pf[1], lsum[1]);
    }
    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O^T[d][q] / l[q] -> out[q][d]; rows >= q_len are 0 ----
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int t = q0 + 16 * qt + lc;
    if (t >= n_max) continue;
    const float l = lsum[qt][0];
    const float inv = (t < qlen && l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 v = o[dt][qt] * inv;
      float4 w;
      w.x = (t < qlen) ? v[0] : 0.f;
      w.y = (t < qlen) ? v[1] : 0.f;
      w.z = (t < qlen) ? v[2] : 0.f;
      w.w = (t < qlen) ? v[3] : 0.f;
      *reinterpret_cast<float4*>(out_h + (int64_t)t * D + 16 * dt + 4 * lg) = w;
    }
  }
}

template <int D, bool CAUSAL, bool MASK>
int launch_typed(const PrefillLaunch& a, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int hw = G < 4 ? G : 4;
  const int rows = kWaveQ * (4 / hw);
  const dim3 grid((a.n_max + rows - 1) / rows, a.num_q_heads / hw, a.batch);
  const size_t lds = 2 * Geo<D>::BUF;
  hipLaunchKernelGGL((prefill_mfma_kernel<D, CAUSAL, MASK>), grid, dim3(kThreads), lds, s, a, hw);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

template <int D>
int launch_flags(const PrefillLaunch& a, hipStream_t s) {
  if (a.causal) return a.key_mask ? launch_typed<D, true, true>(a, s) : launch_typed<D, true, false>(a, s);
  return a.key_mask ? launch_typed<D, false, true>(a, s) : launch_typed<D, false, false>(a, s);
}

}  // namespace

bool prefill_mfma_supports(const PrefillLaunch& a) {
  if (a.dtype != KVATTN_BF16) return false;
  if (a.head_dim != 64 && a.head_dim != 128) return false;
  if (a.has_cache && a.attend_prefix) return false;  // cached prefix: general kernel
  const int G = a.num_q_heads / a.num_kv_heads;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

int launch_prefill_mfma(const PrefillLaunch& a, hipStream_t s) {
  return a.head_dim == 64 ? launch_flags<64>(a, s) : launch_flags<128>(a, s);
}

}  // namespace kvattn
