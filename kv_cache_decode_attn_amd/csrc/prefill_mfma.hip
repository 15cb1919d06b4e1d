// bf16 prefill attention on MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
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
// and Decode"), so both products run on the matrix cores.  The 32x32x16
// bf16 shape is used because it is the one that issues at the full matrix
// rate on gfx950 (the 16x16x32 shape measured at about half of it).
//
// Work split.  A workgroup of 4 waves owns HW = min(G, 4) query heads of one
// KV head and a tile of 32 * 4 / HW query rows; each wave owns one head and
// 32 query rows.  The heads of a GQA group share the K/V tiles staged in LDS.
// Causal tiles are issued heaviest first.
//
// Per 32-key tile, per wave (h = lane / 32):
//   S^T[key][q] = K Q^T      A = K rows from LDS, B = Q (registers), fp32
//                            accumulate.  The 32x32 accumulator gives lane l
//                            query column l % 32 and keys 8*(r/4) + 4h + r%4
//                            (r = 0..15): a query's 32 scores sit in two
//                            lanes, so the row max is a local max plus one
//                            cross-half swap, and P^T is already the B
//                            operand of the second product.
//   P = exp2(S*c - m)        c = scale*log2(e); m is a per-query running
//                            maximum that is only raised (with rescaling of
//                            the accumulators) when the tile maximum exceeds
//                            it by more than 8, so P <= 2^8; P rounded to bf16.
//   O^T[d][q] += V^T P^T     A = V^T from LDS.  V is transposed while it is
//                            staged into LDS; inside a V^T row the keys are
//                            ordered like P^T's operand slots.
//   l[q] += 1 . P^T          an MFMA against a ones operand, so the row sum
//                            is the sum of the same bf16 weights used for O.
// Masked keys (causal, beyond q_len, key_mask) get P = 0 and their V rows are
// staged as zeros, so non-finite padding never reaches O.
#include <math.h>

#include "launch.h"

namespace kvattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKeys = 64;      // keys per tile (two 32-key score sub-tiles)
constexpr int kSub = kKeys / 32;
constexpr int kWaveQ = 32;     // query rows per wave
constexpr int kThreads = 256;  // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;  // log2 headroom before the running max moves

__device__ __forceinline__ f32x16 mfma(const U4& a, const U4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;  // round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// LDS geometry (bytes), two buffers.  K rows are padded to D/2 + 4 dwords
// and V^T rows to kKeys/2 + 4 dwords, so that 16 lanes reading 16
// consecutive rows at one column touch 16 disjoint groups of 4 banks.
template <int D>
struct Geo {
  static constexpr int KROW = D * 2 + 16;
  static constexpr int VROW = kKeys * 2 + 16;
  static constexpr int KBYTES = kKeys * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int MBYTES = kKeys;  // per-key valid flags of the tile
  static constexpr int BUF = KBYTES + VBYTES + MBYTES;
};

// Position of key k (0..kKeys-1) inside a V^T row.  The PV product for keys
// 16m .. 16m+15 of a 32-key sub-tile takes, in lane half h, operand slot j =
// key 16m + 8*(j/4) + 4h + j%4 (the key order of the score accumulator), so
// keys are stored at 16m + 8h + j to make each slot group one 16-byte read.
__device__ __forceinline__ int vpos(int k) {
  return 32 * (k >> 5) + 16 * ((k >> 4) & 1) + 8 * ((k >> 2) & 1) + 4 * ((k >> 3) & 1) + (k & 3);
}

template <int D, bool CAUSAL, bool MASK>
__global__ void __launch_bounds__(kThreads, 2) prefill_mfma_kernel(const PrefillLaunch a, int hw) {
  using GE = Geo<D>;
  constexpr int DK = D / 16;  // 16-wide d chunks of the QK^T contraction
  constexpr int DT = D / 32;  // 32-row d tiles of the output
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, lc = lane & 31;
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

  // ---- Q fragments (B operand of S^T = K Q^T): row q0 + lc, d 16c + 8hh ----
  const int tq = q0 + lc;
  U4 qf[DK];
#pragma unroll
  for (int c = 0; c < DK; ++c)
    qf[c] = (tq < n_max) ? *reinterpret_cast<const U4*>(qg + ((int64_t)tq * D + 16 * c + 8 * hh) * 2) : U4{0, 0, 0, 0};

  // ---- staging of one K/V tile: global -> registers -> LDS ----
  // K: kKeys rows x D*2 bytes in 16-byte chunks, KCH per thread.
  constexpr int KCH = kKeys * D / 8 / kThreads;
  // V: a thread handles key pairs (2m, 2m+1) x 8 columns d in [8 dg, 8 dg+8);
  // kKeys/2 pairs x D/8 column groups = VCH items per thread.
  constexpr int VITEMS = (kKeys / 2) * (D / 8);
  constexpr int VCH = VITEMS / kThreads;
  static_assert(VCH * kThreads == VITEMS && KCH * kThreads == kKeys * D / 8, "staging split");
  U4 kreg[KCH], vreg[VCH][2];
  uint32_t mflag = 0;  // threads 0..kKeys-1: valid flag of key kt0 + tid

  // A key is valid if it is a real token (< q_len) and, with a key mask,
  // its mask byte (at absolute position P + key) is nonzero.
  auto key_valid = [&](int key) -> bool {
    bool ok = key < qlen;
    if (MASK && ok) ok = (P + key < a.key_mask_stride) && mrow[P + key] != 0;
    return ok;
  };
  auto load_tile = [&](int kt0) {
    if (tid < kKeys) mflag = key_valid(kt0 + tid) ? 1u : 0u;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = tid + c * kThreads;
      const int key = kt0 + ch / (D / 8);
      const int col = ch % (D / 8);
      kreg[c] = (key < n_max) ? *reinterpret_cast<const U4*>(kg + ((int64_t)key * D + col * 8) * 2) : U4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int item = tid + c * kThreads;
      const int vm = item % (kKeys / 2), vdg = item / (kKeys / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = kt0 + 2 * vm + e;
        vreg[c][e] = key_valid(key) ? *reinterpret_cast<const U4*>(vg + ((int64_t)key * D + 8 * vdg) * 2)
                                    : U4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* kl = smem + buf * GE::BUF;
    uint8_t* vl = kl + GE::KBYTES;
    if (tid < kKeys) vl[GE::VBYTES + tid] = (uint8_t)mflag;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = tid + c * kThreads;
      *reinterpret_cast<U4*>(kl + (ch / (D / 8)) * GE::KROW + (ch % (D / 8)) * 16) = kreg[c];
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int item = tid + c * kThreads;
      const int vm = item % (kKeys / 2), vdg = item / (kKeys / 2);
      // transpose 2 keys x 8 columns into 8 dwords (key 2m low, 2m+1 high)
      const uint32_t x0[4] = {vreg[c][0].x, vreg[c][0].y, vreg[c][0].z, vreg[c][0].w};
      const uint32_t x1[4] = {vreg[c][1].x, vreg[c][1].y, vreg[c][1].z, vreg[c][1].w};
      const int pos = vpos(2 * vm);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_amdgcn_perm(x1[i], x0[i], 0x05040100u);  // column 2i
        const uint32_t hi = __builtin_amdgcn_perm(x1[i], x0[i], 0x07060302u);  // column 2i+1
        *reinterpret_cast<uint32_t*>(vl + (8 * vdg + 2 * i) * GE::VROW + pos * 2) = lo;
        *reinterpret_cast<uint32_t*>(vl + (8 * vdg + 2 * i + 1) * GE::VROW + pos * 2) = hi;
      }
    }
  };

  // ---- accumulators ----
  f32x16 o[DT], lsum;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    lsum[r] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][r] = 0.f;
  }
  float mrun = -INFINITY;
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
      // S^T of the two 32-key sub-tiles: keys kt0 + 32 st + 8*(r/4) + 4hh +
      // r%4, query q0 + lc; the two accumulation chains interleave.
      f32x16 s[kSub];
#pragma unroll
      for (int st = 0; st < kSub; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
#pragma unroll
      for (int cc = 0; cc < DK; ++cc) {
#pragma unroll
        for (int st = 0; st < kSub; ++st) {
          const U4 kf = *reinterpret_cast<const U4*>(kl + (32 * st + lc) * GE::KROW + (16 * cc + 8 * hh) * 2);
          s[st] = mfma(kf, qf[cc], s[st]);
        }
      }
      // masking: causal edge, keys beyond q_len, key mask.  The tile's key
      // flags come from LDS as words of 4 keys (keys 32st + 8g + 4hh + 0..3).
      const bool edge = (kt0 + kKeys > qlen) || (CAUSAL && kt0 + kKeys - 1 > q0);
      if (MASK || edge) {
        const uint32_t* mw = reinterpret_cast<const uint32_t*>(vl + GE::VBYTES);
#pragma unroll
        for (int st = 0; st < kSub; ++st)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const uint32_t w = mw[8 * st + 2 * gq + hh];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * gq + e;
              const int key = kt0 + 32 * st + 8 * gq + 4 * hh + e;
              const bool ok = ((w >> (8 * e)) & 0xffu) != 0 && (!CAUSAL || key <= tq);
              s[st][r] = ok ? s[st][r] : -INFINITY;
            }
          }
      }
      // running maximum of this query (log2 domain), raised lazily
      float tm = s[0][0];
#pragma unroll
      for (int st = 0; st < kSub; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, s[st][r]);
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
        tm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
      }
      const bool need = tm > mrun + kRescale;
      if (__any(need)) {
        const float mnew = need ? tm : mrun;
        const float alpha = need ? exp2f(mrun - mnew) : 1.f;  // 0 when mrun = -inf
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        lsum *= alpha;
        mrun = mnew;
      }
      const float msub = (mrun == -INFINITY) ? 0.f : mrun;
      U4 pf[kSub][2];
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[st][r], c, -msub));
#pragma unroll
        for (int m = 0; m < 2; ++m)
          pf[st][m] = U4{pack_bf16(p[8 * m], p[8 * m + 1]), pack_bf16(p[8 * m + 2], p[8 * m + 3]),
                         pack_bf16(p[8 * m + 4], p[8 * m + 5]), pack_bf16(p[8 * m + 6], p[8 * m + 7])};
      }
      // O^T += V^T P^T ; l += 1 . P^T   (consecutive MFMAs hit different
      // accumulators)
#pragma unroll
      for (int st = 0; st < kSub; ++st)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const U4 vf =
                *reinterpret_cast<const U4*>(vl + (32 * dt + lc) * GE::VROW + (32 * st + 16 * m + 8 * hh) * 2);
            o[dt] = mfma(vf, pf[st][m], o[dt]);
          }
          lsum = mfma(ones, pf[st][m], lsum);
        }
    }
    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O^T[d][q] / l[q] -> out[q][d]; rows >= q_len are 0 ----
  if (tq < n_max) {
    const float l = lsum[0];
    const bool live = tq < qlen;
    const float inv = (live && l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float4 w;
        w.x = live ? o[dt][4 * rg] * inv : 0.f;
        w.y = live ? o[dt][4 * rg + 1] * inv : 0.f;
        w.z = live ? o[dt][4 * rg + 2] * inv : 0.f;
        w.w = live ? o[dt][4 * rg + 3] * inv : 0.f;
        *reinterpret_cast<float4*>(out_h + (int64_t)tq * D + 32 * dt + 8 * rg + 4 * hh) = w;
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
