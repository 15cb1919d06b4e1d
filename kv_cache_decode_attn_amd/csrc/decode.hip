// Single-token decode attention against one layer's KV cache (gfx950).
//
// What is computed: for each sequence b and query head h, the softmax over
// the cached keys (including the token just appended) of scale * q.k,
// applied to the cached values ("Transformer Attention Masks and KV-Cache
// Inference" (c86j224s.github.io), sections "State of scaled dot-product
// attention" and "Prefill and decode stages"; "KV Cache" (heepie.pages.dev),
// section "TO-BE").  Decode is bound by reading the cache from HBM
// ("KV Cache", section "Prefill and Decode": decode is memory-bandwidth
// bound), so the kernels are organised around streaming K and V once.
//
// Pass 1 (decode_partition): one workgroup of 4 waves per (partition of
// part_tokens keys, KV head, sequence).  All G query heads of the KV head's
// group are served by the same workgroup, so each K/V byte is read once per
// group ("KV Cache Fully Explained", section "(2) GQA").
//   phase 1  every wave streams 16-token blocks of K with 16-byte (8-byte for
//            fp8) coalesced non-temporal loads: lane (row, col) holds EPL elements of one
//            token row; dot products with the G queries are reduced over the
//            LPT lanes of a row with DPP row operations; scores go to LDS.
//   phase 2  per query head, the partition's max and sum of exp2(z - max)
//            (the score scale carries log2 e); weights replace the scores.
//   phase 3  the waves stream the same blocks of V and accumulate
//            o[h] += w * v in fp32 registers, then reduce across rows (lane
//            shuffles) and waves (LDS).
//   The partition's (max, sum, unnormalised o) is its split-K partial; a
//   sequence that fits in one partition is normalised and written directly.
// Pass 2 (decode_merge): per (sequence, query head), the partials are merged
// with the exact running max/sum renormalisation of "KV Cache, Flash
// Attention and Inference Optimization" (factory.pai-world.com), section
// "Flash Attention", numerical trick.  It is not launched when every
// sequence fits one partition.
//
// Pass 1 comes in four forms, chosen by cache type and query columns per KV
// head (each has its own header below): decode_partition (the three phases
// above, vector ALU: f32 caches and groups of 1 or 2), decode_partition_bf16_mfma
// (bf16, 4 or 8 columns: the three phases with both contractions on the
// matrix cores), decode_partition_bf16_online (bf16, 16 columns: one sweep
// with a running softmax, 8 waves per workgroup) and decode_partition_fp8_mfma
// (fp8, 4 or more columns: one sweep with a running softmax).
#include <math.h>

#include "launch.h"

namespace kvattn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int KVT>
struct Traits;

// fp32 cache: 16-byte loads of 4 elements; q kept as fp32.
template <>
struct Traits<KVATTN_F32> {
  static constexpr int EPL = 4;
  typedef U4 Raw;
  __device__ static void to_f32(const Raw& r, float* f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
};

// bf16 cache: 16-byte loads of 8 elements; q kept as packed bf16 pairs so
// the dot product runs on v_dot2_f32_bf16 (fp32 accumulate) without
// unpacking K.
template <>
struct Traits<KVATTN_BF16> {
  static constexpr int EPL = 8;
  typedef U4 Raw;
  __device__ static void to_f32(const Raw& r, float* f) {
    f[0] = bf16_lo(r.x);
    f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y);
    f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z);
    f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w);
    f[7] = bf16_hi(r.w);
  }
};

// fp8 cache: 8-byte loads of 8 codes, decoded exactly to fp32.
template <>
struct Traits<KVATTN_FP8_E4M3> {
  static constexpr int EPL = 8;
  typedef U2 Raw;
  __device__ static void to_f32(const Raw& r, float* f) {
    fp8x4_to_f32(r.x, f);
    fp8x4_to_f32(r.y, f + 4);
  }
};

// Query fragment of one lane: the EPL elements [col*EPL, col*EPL+EPL) of
// each of the G query heads of the group.
template <int KVT, int G>
struct QFrag {
  float f[G][Traits<KVT>::EPL];
  __device__ void load(const uint8_t* q, int64_t row0, int D, int col) {
    // q is fp32 for an fp32 cache, bf16 otherwise
    constexpr int EPL = Traits<KVT>::EPL;
    for (int h = 0; h < G; ++h) {
      if constexpr (KVT == KVATTN_F32) {
        const U4 r = *reinterpret_cast<const U4*>(q + ((row0 + h) * D + col * EPL) * 4);
        Traits<KVATTN_F32>::to_f32(r, f[h]);
      } else {
        const U4 r = *reinterpret_cast<const U4*>(q + ((row0 + h) * D + col * EPL) * 2);
        Traits<KVATTN_BF16>::to_f32(r, f[h]);
      }
    }
  }
  __device__ float dot(int h, const float* k) const {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < Traits<KVT>::EPL; ++e) acc = fmaf(f[h][e], k[e], acc);
    return acc;
  }
};

template <int G>
struct QFrag<KVATTN_BF16, G> {
  uint32_t w[G][4];
  __device__ void load(const uint8_t* q, int64_t row0, int D, int col) {
    for (int h = 0; h < G; ++h) {
      const U4 r = *reinterpret_cast<const U4*>(q + ((row0 + h) * D + col * 8) * 2);
      w[h][0] = r.x;
      w[h][1] = r.y;
      w[h][2] = r.z;
      w[h][3] = r.w;
    }
  }
  __device__ float dot_raw(int h, const U4& k) const {
    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[h][0]),
                                                __builtin_bit_cast(bf16x2_t, k.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[h][1]),
                                          __builtin_bit_cast(bf16x2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[h][2]),
                                          __builtin_bit_cast(bf16x2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[h][3]),
                                          __builtin_bit_cast(bf16x2_t, k.w), acc, false);
    return acc;
  }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
// Register sets in each wave's block ring (blocks in flight + 1), per
// partition kernel.
#ifndef KVATTN_RING_VEC
#define KVATTN_RING_VEC 2
#endif
#ifndef KVATTN_RING_BF16
#define KVATTN_RING_BF16 3
#endif
#ifndef KVATTN_RING_FP8
#define KVATTN_RING_FP8 3
#endif
constexpr int kRingVec = KVATTN_RING_VEC;
constexpr int kRingBf16 = KVATTN_RING_BF16;
constexpr int kRingFp8 = KVATTN_RING_FP8;
// DPP control: rotate each row of 16 lanes right by 8 (lane i reads lane i ^ 8)
constexpr int kDppRowRor8 = 0x128;

// LDS layout of the partition kernel, in floats: block offsets (int64, one
// per 16-token block of the partition), then scores/weights [T][G] (reused
// for the cross-wave output reduction [kWaves][G][D]), then (max, sum) per
// head.
__host__ __device__ constexpr int decode_off_floats(int T) { return 2 * (T / kBlockTokens); }
// Row stride (floats) of the cross-wave reduction [wave][head][d]: D + 4, so
// the 16-byte writes of 8 consecutive heads' rows fall on distinct LDS banks.
__host__ __device__ constexpr int red_stride(int D) { return D + 4; }
__host__ __device__ constexpr int decode_lds_floats(int T, int G, int D) {
  return decode_off_floats(T) + ((T * G > kWaves * G * red_stride(D)) ? T * G : kWaves * G * red_stride(D)) + 2 * G;
}
// Fused append: the new tokens' K and V rows (k_new/v_new [batch,
// num_kv_heads, n_tail, head_dim]) go to positions seq_lens[b] - n_tail ..
// seq_lens[b] - 1.  Each partition's workgroup stores the rows whose
// positions fall in its own key range, encoded as kv_append encodes them (a
// copy for an fp32 or bf16 cache, E4M3(x / scale) for an fp8 cache), then
// reads the cache as usual: the barrier that follows makes the stores
// visible to every wave of the workgroup (a workgroup-scope release and
// acquire on global memory).  A position is read only by the workgroup of
// its partition, so the step needs no separate write pass.
template <int KVT, int D>
__device__ void store_new_row(const DecodeLaunch& p, int b, int g, int tn, int row) {
  constexpr int ES = (KVT == KVATTN_F32) ? 4 : (KVT == KVATTN_BF16) ? 2 : 1;
  constexpr int EPW = 4 / ES;     // elements per 32-bit word
  constexpr int W = D * ES / 4;   // words per row
  const int64_t off = position_offset(p.c, b, g, tn);
  if (off < 0) return;  // outside the cache: nothing is stored (and the key is masked)
  for (int i = threadIdx.x; i < 2 * W; i += blockDim.x) {
    const int kv = i / W, w = i - kv * W;
    const int64_t src = (((int64_t)b * p.num_kv_heads + g) * p.n_tail + row) * D + (int64_t)w * EPW;
    const uint8_t* in = kv ? p.v_new : p.k_new;
    uint32_t word;
    if constexpr (KVT == KVATTN_F32) {
      word = reinterpret_cast<const uint32_t*>(in)[src];
    } else if constexpr (KVT == KVATTN_BF16) {
      word = *reinterpret_cast<const uint32_t*>(in + src * 2);
    } else {
      const float s = (kv ? p.v_scale : p.k_scale)[g];
      float x[4];
      if (p.in_dtype == KVATTN_F32) {
        const U4 r = *reinterpret_cast<const U4*>(in + src * 4);
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
      } else {
        const U2 r = *reinterpret_cast<const U2*>(in + src * 2);
        x[0] = bf16_lo(r.x);
        x[1] = bf16_hi(r.x);
        x[2] = bf16_lo(r.y);
        x[3] = bf16_hi(r.y);
      }
      word = f32_to_e4m3(x[0] / s) | (f32_to_e4m3(x[1] / s) << 8) | (f32_to_e4m3(x[2] / s) << 16) |
             (f32_to_e4m3(x[3] / s) << 24);
    }
    *reinterpret_cast<uint32_t*>((kv ? p.c.v : p.c.k) + off + 4 * w) = word;
  }
}

// Values the compiler cannot prove wave-uniform (LDS reads at one address,
// the wave index) moved to scalar registers, so branches on them are scalar
// and the load addresses are scalar base + lane offset.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Streams the blocks jb, jb + kWaves, ... (< nblk) of one wave through a
// ring of NB register sets: while one block is consumed the next NB - 1
// blocks' loads are in flight.  ring_fill loads the first NB - 1 blocks
// (before anything else needs the wave, so the first loads overlap other
// work); stream_ring then consumes every block, refilling the set it has
// just freed with the block NB - 1 places ahead.  Every load is a real block
// and every steady-state iteration issues the same loads, so the compiler's
// load-count waits release exactly the block about to be consumed; the
// scheduling barriers keep each prefetch ahead of the wait for the block
// before it.  The last 2 NB - 2 blocks form an explicit tail.
template <int NB, typename Buf, typename LoadF, int STEP = kWaves>
__device__ __forceinline__ void ring_fill(int jb, int nblk, Buf (&r)[NB], const LoadF& load) {
#pragma unroll
  for (int i = 0; i < NB - 1; ++i)
    if (jb + i * STEP < nblk) load(jb + i * STEP, r[i]);
}

template <int NB, typename Buf, typename LoadF, typename BodyF, int STEP = kWaves>
__device__ __forceinline__ void stream_ring(int jb, int nblk, Buf (&r)[NB], const LoadF& load, const BodyF& body) {
  static_assert(NB >= 2, "ring");
  for (; jb + (2 * NB - 2) * STEP < nblk; jb += NB * STEP) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      load(jb + (i + NB - 1) * STEP, r[(i + NB - 1) % NB]);
      __builtin_amdgcn_sched_barrier(0);
      body(jb + i * STEP, r[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * NB - 2; ++i) {
    if (i <= NB - 2 && jb + (i + NB - 1) * STEP < nblk) load(jb + (i + NB - 1) * STEP, r[(i + NB - 1) % NB]);
    __builtin_amdgcn_sched_barrier(0);
    if (jb + i * STEP < nblk) body(jb + i * STEP, r[i % NB]);
  }
}

// K and V bytes are read exactly once per call: load them non-temporally so
// the stream does not displace reusable lines (q, block table, partials)
// from the caches.
template <typename Raw>
__device__ __forceinline__ Raw stream_load(const Raw* p) {
  if constexpr (sizeof(Raw) == 16) {
    typedef unsigned v4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(Raw, __builtin_nontemporal_load(reinterpret_cast<const v4*>(p)));
  } else {
    typedef unsigned v2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(Raw, __builtin_nontemporal_load(reinterpret_cast<const v2*>(p)));
  }
}

// K blocks of the MFMA partition passes are staged through LDS.  The matrix
// core wants lane l to hold key l % 16, so loading K straight into registers
// reads 64 bytes of each of 16 rows per instruction: half cache lines, which
// cap a plain read of such blocks at about 5.8 TB/s on MI355X against
// 6.8 TB/s for whole rows.  Instead each wave copies its block into an LDS
// slot of its own with 16-byte-per-lane global-to-LDS transfers in which 16
// lanes read one row completely, and then reads the slot in the MFMA layout.
// In the slot, 16-byte chunk c of row r sits at position c ^ swz(r), so the
// 16 rows of one MFMA-layout read fall on distinct LDS banks.
template <int ROWB>
struct KStage {
  static constexpr int BYTES = kBlockTokens * ROWB;  // one 16-token block of one head
  static constexpr int XFERS = BYTES / 1024;          // 1 KB transfers per block
  static constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  static constexpr int RP = 256 / ROWB;               // rows per 256 bytes (one pass over the banks)
  static_assert(XFERS >= 1 && CPR >= 4 && RP >= 1, "row size");
  __device__ static int swz(int r) { return (r / RP) % CPR; }
  // byte of the block that lane `lane` of transfer x copies
  __device__ static int src(int x, int lane) {
    const int e = x * 1024 + 16 * lane;  // its slot byte
    const int r = e / ROWB;
    return r * ROWB + 16 * (((e % ROWB) / 16) ^ swz(r));
  }
  // slot byte of chunk c of row r
  __device__ static int at(int r, int c) { return r * ROWB + 16 * (c ^ swz(r)); }
};
// s_waitcnt immediates (gfx9 encoding): all vector memory operations done;
// all LDS operations done.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;
// s_waitcnt immediate: at most n vector memory operations outstanding.
__host__ __device__ constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// Cache policy of the K transfers: non-temporal (each byte is read once).
[[maybe_unused]] constexpr int kPolicyNT = 2;  // used in the device pass only

// 16 bytes per lane from `src` into LDS at dst + 16 * lane (dst uniform over
// the wave), non-temporally.  The body exists in the device pass only: the
// host pass compiles each kernel just for its launch stub.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* src, uint8_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, kPolicyNT);
#endif
}

// The same transfer issued as inline assembly: the compiler then does not
// count it among the loads in flight, so it does not wait for it before every
// LDS read or before the use of any older load; completion is awaited
// explicitly.
__device__ __forceinline__ void copy16_to_lds_async(const uint8_t* src, uint8_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)dst;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, off nt"
      :
      : "s"(m0), "v"(src)
      : "memory", "m0");
#endif
}

// Byte offset of the K slots in the dynamic LDS of an MFMA partition pass
// whose other arrays take `floats` floats (rounded up to 16 bytes).
__host__ __device__ constexpr int kslot_offset(int floats) { return ((floats * 4 + 15) / 16) * 16; }

template <int KVT, int D, int G, bool MASK, bool TAIL>
__global__ void __launch_bounds__(256) decode_partition(const DecodeLaunch p) {
  using TR = Traits<KVT>;
  using Raw = typename TR::Raw;
  constexpr int EPL = TR::EPL;
  constexpr int LPT = D / EPL;        // lanes per token row
  constexpr int TPI = kWave / LPT;    // token rows per wave-wide load
  constexpr int NI = kBlockTokens / TPI;  // loads per 16-token block
  static_assert(TPI * NI == kBlockTokens && NI >= 1, "row split");
  constexpr int ROWB = D * (int)sizeof(Raw) / EPL;  // bytes per token row

  extern __shared__ float lds[];
  // KV head fastest in the grid: neighbouring workgroups read the heads of
  // the same 16-token blocks, which sit side by side in the paged pool.
  // grid (KV head, sequence, partition): partition-major, so every
  // sequence's first partitions are dispatched before any later one
  const int g = blockIdx.x, b = blockIdx.y, part = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int col = lane % LPT, row = lane / LPT;
  const int T = p.part_tokens;
  const int ctx = min(max(p.seq_lens[b], 0), p.ctx_limit);
  const int hq0 = g * G;
  const int t0 = part * T;
  if (t0 >= ctx) {
    // An empty sequence still has a defined output: zeros.
    if (part == 0) {
      for (int i = tid; i < G * D; i += 256)
        p.out[((int64_t)b * p.num_q_heads + hq0) * D + i] = 0.f;
    }
    return;
  }
  const int t1 = min(t0 + T, ctx);
  const int n = t1 - t0;
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const int j0 = t0 / kBlockTokens;
  // Several queries per sequence (TAIL): column h of the group is query
  // h % n_tail of its head, which sees the keys below
  // ctx - (n_tail - 1 - h % n_tail); ncol is that bound relative to t0.
  auto ncol = [&](int h) { return ctx - (p.n_tail - 1 - h % p.n_tail) - t0; };

  int64_t* offs = reinterpret_cast<int64_t*>(lds);        // [T/16] block byte offsets (-1: outside)
  float* s_lds = lds + decode_off_floats(T);              // [T][G] scores -> weights
  float* stat = lds + decode_lds_floats(T, G, D) - 2 * G;  // [G][2] (max, sum)
  uint8_t* mflag = reinterpret_cast<uint8_t*>(lds + decode_lds_floats(T, G, D));  // [T] mask (MASK only)
  for (int i = tid; i < nblk; i += 256) offs[i] = block_offset(p.c, b, g, j0 + i);
  if constexpr (MASK) {
    const uint8_t* mask_row = p.key_mask + (int64_t)b * p.key_mask_stride + t0;
    for (int t = tid; t < n; t += 256) mflag[t] = mask_row[t];
  }
  // fused append: each partition stores the new rows in its key range
  if (p.k_new != nullptr && p.seq_lens[b] == ctx) {
    for (int i = 0; i < p.n_tail; ++i) {
      const int tn = ctx - p.n_tail + i;
      if (tn >= t0 && tn < t1) store_new_row<KVT, D>(p, b, g, tn, i);
    }
  }

  QFrag<KVT, G> q;
  q.load(p.q, (int64_t)b * p.num_q_heads + hq0, D, col);
  float zscale = p.scale * kLog2e;
  if constexpr (KVT == KVATTN_FP8_E4M3) zscale *= p.k_scale[g];
  const uint8_t* kbase = p.c.k + row * ROWB + col * (int)sizeof(Raw);
  const uint8_t* vbase = p.c.v + row * ROWB + col * (int)sizeof(Raw);
  __syncthreads();  // also publishes the fused append's stores to every wave

  // Block jb's rows (jb < nblk); a block outside the cache is read at offset
  // 0, a valid address whose bytes are never used (its keys are masked).
  auto load_block = [&](int jb, const uint8_t* base, Raw* r) {
    const int64_t o = offs[jb];
    const int64_t off = uniform64(o >= 0 ? o : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) r[i] = stream_load(reinterpret_cast<const Raw*>(base + off + i * TPI * ROWB));
  };

  // ---- phase 1: scores of every key of the partition ----
  // Wave w handles blocks w, w + 4, ... (stream_ring).
  auto scores = [&](int jb, const Raw* cur) {
    const bool in_cache = uniform64(offs[jb]) >= 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = kBlockTokens * jb + i * TPI + row;  // partition-relative key
      float acc[G];
      if constexpr (KVT == KVATTN_BF16) {
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = q.dot_raw(h, cur[i]);
      } else {
        float kf[EPL];
        TR::to_f32(cur[i], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = q.dot(h, kf);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = group_sum<LPT>(acc[h]);
      if (t < n) {
        bool valid = in_cache;
        if constexpr (MASK) valid = valid && mflag[t] != 0;
        if (col == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const bool ok = valid && (!TAIL || t < ncol(h));
            s_lds[t * G + h] = ok ? acc[h] * zscale : -INFINITY;
          }
        }
      }
    }
  };
  {
    Raw kr[kRingVec][NI];
    auto load_k = [&](int jb, Raw* r) { load_block(jb, kbase, r); };
    ring_fill(wave, nblk, kr, load_k);
    stream_ring(wave, nblk, kr, load_k, scores);
  }
  // The first V blocks are fetched while the softmax statistics are formed.
  Raw vr[kRingVec][NI];
  auto load_v = [&](int jb, Raw* r) { load_block(jb, vbase, r); };
  ring_fill(wave, nblk, vr, load_v);
  __syncthreads();

  // ---- phase 2: per-head max and sum; scores -> weights exp2(z - max) ----
  for (int h = wave; h < G; h += kWaves) {
    float m = -INFINITY;
    for (int t = lane; t < n; t += kWave) m = fmaxf(m, s_lds[t * G + h]);
    m = group_max<64>(m);
    const float mref = (m == -INFINITY) ? 0.f : m;
    float l = 0.f;
    for (int t = lane; t < n; t += kWave) {
      const float e = __builtin_amdgcn_exp2f(s_lds[t * G + h] - mref);  // argument <= 0
      s_lds[t * G + h] = e;
      l += e;
    }
    l = group_sum<64>(l);
    if (lane == 0) {
      stat[2 * h] = m;
      stat[2 * h + 1] = l;
    }
  }
  __syncthreads();

  // ---- phase 3: o[h] += w * v over the same blocks ----
  float o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;

  auto accumulate = [&](int jb, const Raw* cur) {
    // A block wholly inside the partition with no key mask has only live
    // keys; otherwise a key with zero weight for every head is dropped so
    // that non-finite bytes in padding or stale slots cannot reach o.  A
    // block outside the cache was fully masked (all weights 0).
    if (uniform64(offs[jb]) < 0) return;
    const bool full = !MASK && kBlockTokens * (jb + 1) <= n;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = kBlockTokens * jb + i * TPI + row;
      float w[G];
      bool live = true;
      if (full) {
#pragma unroll
        for (int h = 0; h < G; ++h) w[h] = s_lds[t * G + h];
      } else {
        live = false;
        const bool in = t < n;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          w[h] = in ? s_lds[t * G + h] : 0.f;
          live = live || (w[h] != 0.f);
        }
      }
      float vf[EPL];
      TR::to_f32(cur[i], vf);
      if (!live) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(w[h], vf[e], o[h][e]);
    }
  };
  stream_ring(wave, nblk, vr, load_v, accumulate);

  // reduce over the TPI rows of the wave (lanes sharing col)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = strided_sum<LPT>(o[h][e]);

  __syncthreads();  // every wave is done reading weights; reuse LDS
  float* red = s_lds;  // [kWaves][G][D]
  static_assert(EPL % 4 == 0, "16-byte reduction writes");
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(red + (wave * G + h) * D + col * EPL + e) =
            make_float4(o[h][e], o[h][e + 1], o[h][e + 2], o[h][e + 3]);
  }
  __syncthreads();

  const int nparts_b = (ctx + T - 1) / T;
  float vscale = 1.f;
  if constexpr (KVT == KVATTN_FP8_E4M3) vscale = p.v_scale[g];
  for (int idx = tid; idx < G * D / 4; idx += 256) {
    const int h = idx / (D / 4), d = 4 * (idx - h * (D / 4));
    float4 acc = *reinterpret_cast<const float4*>(red + h * D + d);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(red + (w * G + h) * D + d);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    acc.x *= vscale;
    acc.y *= vscale;
    acc.z *= vscale;
    acc.w *= vscale;
    const int hq = hq0 + h;
    const float l = stat[2 * h + 1];
    if (nparts_b == 1) {
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      *reinterpret_cast<float4*>(p.out + ((int64_t)b * p.num_q_heads + hq) * D + d) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
      const int64_t slot = ((int64_t)b * p.num_q_heads + hq) * p.num_parts + part;
      *reinterpret_cast<float4*>(p.ws_o + slot * D + d) = acc;
      if (d == 0) {
        p.ws_ml[slot * 2] = stat[2 * h];
        p.ws_ml[slot * 2 + 1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 cache with G >= 4 query heads per KV head: the partition pass with
// both contractions on v_mfma_f32_16x16x16_bf16 and the same three phases.
//   phase 1  S^T[key][h] = K Q^T per 16-token block.  A = K, staged
//            through the wave's LDS slot (KStage) and read from it so that
//            lane l holds key l%16, 16-byte chunks c at row bytes
//            64c + 16(l/16) (k-step 2c + u takes half u of chunk c);
//            B = q of head l%16 in the same d order (zero for heads >= G).
//            Lane l gets keys 4(l/16) + r of head l%16, stored head-major.
//   phase 2  as in decode_partition: per head max, exp2 weights and sum.
//   phase 3  O^T += V^T P^T.  A = V^T: lane l loads 8 bytes (d 4(l%16)..+3
//            of a 64-wide half) of keys 4(l/16)..+3 and transposes the 4x4
//            block of 16-bit values with v_perm_b32, so output tile (half,
//            j) row l%16 holds d = 64*half + 4*(l%16) + j.  B = the lane's
//            own 4 weights (keys 4(l/16) + r of head l%16, contiguous in
//            LDS), split into bf16 hi + lo parts (two MFMAs) so P keeps
//            about 16 bits.
// Per 16-token block a wave issues 8 (D = 128) MFMAs for the scores and 16
// for the output instead of the vector pass's per-element dot products,
// lane reductions and multiply-adds.
template <int D, int G, bool MASK, bool TAIL>
__global__ void __launch_bounds__(256) decode_partition_bf16_mfma(const DecodeLaunch p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  constexpr int ROWB = 2 * D;       // bytes per token row
  constexpr int KC = ROWB / 64;     // 16-byte K chunks per lane and block
  constexpr int KS = 2 * KC;        // k-steps of 4 bf16
  constexpr int HALVES = D / 64;    // 64-wide d halves of the V^T tiles
  constexpr int NT = 4 * HALVES;    // output tiles of 16 d rows
  static_assert(G >= 1 && G <= 16 && KC >= 1, "shape");

  extern __shared__ float lds[];
  const int g = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  const int T = p.part_tokens;
  const int ctx = min(max(p.seq_lens[b], 0), p.ctx_limit);
  const int hq0 = g * G;
  const int t0 = part * T;
  if (t0 >= ctx) {
    if (part == 0)
      for (int i = tid; i < G * D; i += 256) p.out[((int64_t)b * p.num_q_heads + hq0) * D + i] = 0.f;
    return;
  }
  const int t1 = min(t0 + T, ctx);
  const int n = t1 - t0;
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const int j0 = t0 / kBlockTokens;

  int64_t* offs = reinterpret_cast<int64_t*>(lds);
  float* s_lds = lds + decode_off_floats(T);               // [G][T] scores -> weights
  float* stat = lds + decode_lds_floats(T, G, D) - 2 * G;  // [G][2] (max, sum)
  uint8_t* mflag = reinterpret_cast<uint8_t*>(lds + decode_lds_floats(T, G, D));  // [T] mask (MASK only)
  for (int i = tid; i < nblk; i += 256) offs[i] = block_offset(p.c, b, g, j0 + i);
  if constexpr (MASK) {
    const uint8_t* mask_row = p.key_mask + (int64_t)b * p.key_mask_stride + t0;
    for (int t = tid; t < n; t += 256) mflag[t] = mask_row[t];
  }
  // fused append (as in decode_partition)
  if (p.k_new != nullptr && p.seq_lens[b] == ctx) {
    for (int i = 0; i < p.n_tail; ++i) {
      const int tn = ctx - p.n_tail + i;
      if (tn >= t0 && tn < t1) store_new_row<KVATTN_BF16, D>(p, b, g, tn, i);
    }
  }

  // q of head r16 in the k order of the K chunks: k-step s = 2c + u uses
  // d 32c + 8*lg + 4u + 0..3 (zero for heads >= G)
  uint32_t qb[KS][2];
  {
    const int hr = r16 < G ? r16 : 0;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)b * p.num_q_heads + hq0 + hr) * D;
#pragma unroll
    for (int sd = 0; sd < KS; ++sd) {
      const uint2 w = *reinterpret_cast<const uint2*>(qrow + 32 * (sd / 2) + 8 * lg + 4 * (sd % 2));
      qb[sd][0] = r16 < G ? w.x : 0u;
      qb[sd][1] = r16 < G ? w.y : 0u;
    }
  }
  const float zscale = p.scale * kLog2e;
  __syncthreads();  // also publishes the fused append's stores to every wave

  // Key t of the partition is attended (inside it and not masked).
  auto key_ok = [&](int t) -> bool {
    if (t >= n) return false;
    if constexpr (MASK) return mflag[t] != 0;
    return true;
  };
  // Byte offset of block jb (jb < nblk); a block outside the cache is read at
  // offset 0, a valid address whose bytes are never used (its keys are masked).
  auto load_off = [&](int jb) -> int64_t {
    const int64_t o = offs[jb];
    return uniform64(o >= 0 ? o : 0);
  };

  // ---- phase 1: scores; wave w takes blocks w, w + 4, ... ----
  // Chunk c of lane (r16, lg) is bytes 64c + 16*lg of key r16's row (read from
  // the wave's K slot; the next block's transfer is in flight meanwhile).
  using KST = KStage<ROWB>;
  uint8_t* kslot = reinterpret_cast<uint8_t*>(lds) +
                   kslot_offset(decode_lds_floats(T, G, D) + (MASK ? T / 4 : 0)) + wave * KST::BYTES;
  int ksrc[KST::XFERS], kat[KC];
#pragma unroll
  for (int x = 0; x < KST::XFERS; ++x) ksrc[x] = KST::src(x, lane);
#pragma unroll
  for (int c = 0; c < KC; ++c) kat[c] = KST::at(r16, 4 * c + lg);
  auto issue_k = [&](int jb, uint8_t* slot) {
    const uint8_t* blk = p.c.k + load_off(jb);
#pragma unroll
    for (int x = 0; x < KST::XFERS; ++x) copy16_to_lds(blk + ksrc[x], slot + x * 1024);
  };
  auto scores = [&](int jb, const U4* kr) {
    const bool in_cache = uniform64(offs[jb]) >= 0;
    v4f sacc = v4f{0.f, 0.f, 0.f, 0.f}, sacc2 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const v4s a0 = __builtin_bit_cast(v4s, v2u{kr[c].x, kr[c].y});
      const v4s a1 = __builtin_bit_cast(v4s, v2u{kr[c].z, kr[c].w});
      const v4s b0 = __builtin_bit_cast(v4s, v2u{qb[2 * c][0], qb[2 * c][1]});
      const v4s b1 = __builtin_bit_cast(v4s, v2u{qb[2 * c + 1][0], qb[2 * c + 1][1]});
      sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, b0, sacc, 0, 0, 0);
      sacc2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, b1, sacc2, 0, 0, 0);
    }
    sacc += sacc2;
    if (r16 < G) {
      const int tk = kBlockTokens * jb + 4 * lg;  // partition-relative key of r = 0
      // several queries per sequence (TAIL): column r16 is query r16 % n_tail,
      // which sees keys below ctx - (n_tail - 1 - r16 % n_tail)
      const int ncol = TAIL ? ctx - (p.n_tail - 1 - r16 % p.n_tail) - t0 : n;
      float4 z;
      z.x = (in_cache && key_ok(tk + 0) && tk + 0 < ncol) ? sacc[0] * zscale : -INFINITY;
      z.y = (in_cache && key_ok(tk + 1) && tk + 1 < ncol) ? sacc[1] * zscale : -INFINITY;
      z.z = (in_cache && key_ok(tk + 2) && tk + 2 < ncol) ? sacc[2] * zscale : -INFINITY;
      z.w = (in_cache && key_ok(tk + 3) && tk + 3 < ncol) ? sacc[3] * zscale : -INFINITY;
      *reinterpret_cast<float4*>(s_lds + r16 * T + tk) = z;
    }
  };
  // One slot per wave (a second slot, letting the next transfer start before
  // the current block is read, measured slower: the LDS it takes costs a
  // workgroup per CU).  Only K transfers are in flight in this phase, so
  // waiting for all of them means block jb has landed; the slot is read out
  // before the next transfer refills it.
  if (wave < nblk) issue_k(wave, kslot);
  for (int jb = wave; jb < nblk; jb += kWaves) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    U4 kr[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) kr[c] = *reinterpret_cast<const U4*>(kslot + kat[c]);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (jb + kWaves < nblk) issue_k(jb + kWaves, kslot);
    scores(jb, kr);
  }
  // V: 8 bytes (d 64*hf + 4*r16 ..+3) of each of keys 4*lg + i
  const uint8_t* vbase = p.c.v + (4 * lg) * ROWB + 8 * r16;
  auto load_v = [&](int jb, uint2 (*vr)[4]) {
    const int64_t off = load_off(jb);
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[hf][i] = __builtin_bit_cast(
            uint2, __builtin_nontemporal_load(reinterpret_cast<const v2u*>(vbase + off + i * ROWB + 128 * hf)));
  };
  // The first V block is fetched while the softmax statistics are formed.
  uint2 vring[kRingBf16][HALVES][4];
  ring_fill(wave, nblk, vring, load_v);
  __syncthreads();

  // ---- phase 2: per-head max and sum; scores -> weights exp2(z - max) ----
  for (int h = wave; h < G; h += kWaves) {
    float* sh = s_lds + h * T;
    float m = -INFINITY;
    for (int t = lane; t < n; t += kWave) m = fmaxf(m, sh[t]);
    m = group_max<64>(m);
    const float mref = (m == -INFINITY) ? 0.f : m;
    float l = 0.f;
    for (int t = lane; t < n; t += kWave) {
      const float e = __builtin_amdgcn_exp2f(sh[t] - mref);  // argument <= 0
      sh[t] = e;
      l += e;
    }
    l = group_sum<64>(l);
    if (lane == 0) {
      stat[2 * h] = m;
      stat[2 * h + 1] = l;
    }
  }
  __syncthreads();

  // ---- phase 3: O^T += V^T P^T ----
  v4f o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  auto accumulate = [&](int jb, const uint2 (*vr)[4]) {
    if (uniform64(offs[jb]) < 0) return;  // block outside the cache: every weight is 0
    const int tk = kBlockTokens * jb + 4 * lg;
    bool live[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) live[r] = key_ok(tk + r);
    float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r16 < G) w = *reinterpret_cast<const float4*>(s_lds + r16 * T + tk);
    const float pw[4] = {live[0] ? w.x : 0.f, live[1] ? w.y : 0.f, live[2] ? w.z : 0.f, live[3] ? w.w : 0.f};
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 h01, h23, l01, l23;
    h01[0] = (__bf16)pw[0];
    h01[1] = (__bf16)pw[1];
    h23[0] = (__bf16)pw[2];
    h23[1] = (__bf16)pw[3];
    l01[0] = (__bf16)(pw[0] - (float)h01[0]);
    l01[1] = (__bf16)(pw[1] - (float)h01[1]);
    l23[0] = (__bf16)(pw[2] - (float)h23[0]);
    l23[1] = (__bf16)(pw[3] - (float)h23[1]);
    const v4s phi = __builtin_bit_cast(v4s, v2u{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)});
    const v4s plo = __builtin_bit_cast(v4s, v2u{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf) {
      uint2 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = live[i] ? vr[hf][i] : uint2{0u, 0u};  // dead keys never reach O
      // 4 keys x 4 d (16-bit) -> per d j the 4 keys' values
      const uint32_t x01l = __builtin_amdgcn_perm(a[1].x, a[0].x, 0x05040100u);
      const uint32_t x23l = __builtin_amdgcn_perm(a[3].x, a[2].x, 0x05040100u);
      const uint32_t x01h = __builtin_amdgcn_perm(a[1].x, a[0].x, 0x07060302u);
      const uint32_t x23h = __builtin_amdgcn_perm(a[3].x, a[2].x, 0x07060302u);
      const uint32_t y01l = __builtin_amdgcn_perm(a[1].y, a[0].y, 0x05040100u);
      const uint32_t y23l = __builtin_amdgcn_perm(a[3].y, a[2].y, 0x05040100u);
      const uint32_t y01h = __builtin_amdgcn_perm(a[1].y, a[0].y, 0x07060302u);
      const uint32_t y23h = __builtin_amdgcn_perm(a[3].y, a[2].y, 0x07060302u);
      const v4s av[4] = {__builtin_bit_cast(v4s, v2u{x01l, x23l}), __builtin_bit_cast(v4s, v2u{x01h, x23h}),
                         __builtin_bit_cast(v4s, v2u{y01l, y23l}), __builtin_bit_cast(v4s, v2u{y01h, y23h})};
      // hi parts of the four tiles, then the lo parts: no back-to-back
      // MFMAs on one accumulator
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[4 * hf + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], phi, o[4 * hf + j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[4 * hf + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], plo, o[4 * hf + j], 0, 0, 0);
    }
  };
  stream_ring(wave, nblk, vring, load_v, accumulate);

  __syncthreads();  // every wave is done reading weights; reuse LDS
  constexpr int RS = red_stride(D);
  float* red = s_lds;  // [kWaves][G][RS]
  // lane (r16, lg) holds d = 64 hf + 4 (4 lg + rr) + j of head r16 in o[4 hf + j][rr]
  if (r16 < G) {
    float* row = red + (wave * G + r16) * RS;
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<float4*>(row + 64 * hf + 4 * (4 * lg + rr)) =
            make_float4(o[4 * hf][rr], o[4 * hf + 1][rr], o[4 * hf + 2][rr], o[4 * hf + 3][rr]);
  }
  __syncthreads();

  const int nparts_b = (ctx + T - 1) / T;
  for (int idx = tid; idx < G * D / 4; idx += 256) {
    const int h = idx / (D / 4), d = 4 * (idx - h * (D / 4));
    float4 acc = *reinterpret_cast<const float4*>(red + h * RS + d);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(red + (w * G + h) * RS + d);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    const int hq = hq0 + h;
    const float l = stat[2 * h + 1];
    if (nparts_b == 1) {
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      *reinterpret_cast<float4*>(p.out + ((int64_t)b * p.num_q_heads + hq) * D + d) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
      const int64_t slot = ((int64_t)b * p.num_q_heads + hq) * p.num_parts + part;
      *reinterpret_cast<float4*>(p.ws_o + slot * D + d) = acc;
      if (d == 0) {
        p.ws_ml[slot * 2] = stat[2 * h];
        p.ws_ml[slot * 2 + 1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 cache, many query columns per KV head (several queries per sequence):
// the bf16 matrix-core pass in one sweep over the blocks, with the running
// softmax of the fp8 pass instead of a per-partition score buffer.  With 16
// columns per KV head the three-phase pass above keeps 16 scores per key in
// LDS, which caps its partitions at 512 keys and its occupancy at three
// workgroups per compute unit; here the LDS holds only the K slots and the
// final cross-wave combine, so partitions can be long and the split-K
// partials few.
//   per 16-token block: S^T = K Q^T on MFMA (K staged through the wave's LDS
//   slot exactly as in decode_partition_bf16_mfma), mask, block max and the
//   lazily raised running max (as in decode_partition_fp8_mfma), weights
//   exp2(z - m) split into bf16 hi + lo, then O^T += V^T P^T with V^T built
//   by 16-bit v_perm_b32 transposes of the lane's own V loads.
// Each wave keeps its own (max, sum, O) over its blocks; the waves are
// combined through LDS.
// s_waitcnt vmcnt(n) for a count known only at run time (0 <= n <= 31).
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
#define KVATTN_WAIT_CASE(k) \
  case k: __builtin_amdgcn_s_waitcnt(wait_vm(k)); break;
    KVATTN_WAIT_CASE(1) KVATTN_WAIT_CASE(2) KVATTN_WAIT_CASE(3) KVATTN_WAIT_CASE(4) KVATTN_WAIT_CASE(5)
    KVATTN_WAIT_CASE(6) KVATTN_WAIT_CASE(7) KVATTN_WAIT_CASE(8) KVATTN_WAIT_CASE(9) KVATTN_WAIT_CASE(10)
    KVATTN_WAIT_CASE(11) KVATTN_WAIT_CASE(12) KVATTN_WAIT_CASE(13) KVATTN_WAIT_CASE(14) KVATTN_WAIT_CASE(15)
    KVATTN_WAIT_CASE(16) KVATTN_WAIT_CASE(17) KVATTN_WAIT_CASE(18) KVATTN_WAIT_CASE(19) KVATTN_WAIT_CASE(20)
    KVATTN_WAIT_CASE(21) KVATTN_WAIT_CASE(22) KVATTN_WAIT_CASE(23) KVATTN_WAIT_CASE(24) KVATTN_WAIT_CASE(25)
    KVATTN_WAIT_CASE(26) KVATTN_WAIT_CASE(27) KVATTN_WAIT_CASE(28) KVATTN_WAIT_CASE(29) KVATTN_WAIT_CASE(30)
    KVATTN_WAIT_CASE(31)
#undef KVATTN_WAIT_CASE
    default: __builtin_amdgcn_s_waitcnt(wait_vm(0)); break;
  }
}

// Waves per workgroup of decode_partition_bf16_online: eight, two per SIMD,
// so a workgroup gets through its partition in half the time of four waves
// and the grid's last workgroups finish sooner, for the same partials.
#ifndef KVATTN_ONLINE_WAVES
#define KVATTN_ONLINE_WAVES 8
#endif
constexpr int kOnlineWaves = KVATTN_ONLINE_WAVES;

// LDS of decode_partition_bf16_online: block offsets, (max, sum) per wave and
// head, the key mask flags (MASK), then one area that holds the waves' K
// slots (two per wave) during the sweep and the cross-wave reduction
// [kOnlineWaves][G][D] afterwards.
__host__ __device__ constexpr int bf16_online_area_offset(int T, int G, bool mask) {
  return kslot_offset(decode_off_floats(T) + kOnlineWaves * G * 2 + (mask ? T / 4 : 0));
}
__host__ __device__ constexpr int bf16_online_lds_bytes(int T, int G, int D, bool mask) {
  // two K slots per wave of one 16-token block of bf16 rows (2 D bytes each)
  return bf16_online_area_offset(T, G, mask) + (kOnlineWaves * G * red_stride(D) * 4 > kOnlineWaves * 2 * kBlockTokens * 2 * D
                                                    ? kOnlineWaves * G * red_stride(D) * 4
                                                    : kOnlineWaves * 2 * kBlockTokens * 2 * D);
}

template <int D, int G, bool MASK, bool TAIL>
__global__ void __launch_bounds__(kOnlineWaves * kWave) decode_partition_bf16_online(const DecodeLaunch p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  constexpr int ROWB = 2 * D;       // bytes per token row
  constexpr int KC = ROWB / 64;     // 16-byte K chunks per lane and block
  constexpr int HALVES = D / 64;    // 64-wide d halves of the V^T tiles
  constexpr int NT = 4 * HALVES;    // output tiles of 16 d rows
  constexpr float kRescale = 8.f;
  static_assert(G >= 4 && G <= 16 && KC >= 1, "shape");

  extern __shared__ float lds[];
  const int g = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  const int T = p.part_tokens;
  const int ctx = min(max(p.seq_lens[b], 0), p.ctx_limit);
  const int hq0 = g * G;
  const int t0 = part * T;
  if (t0 >= ctx) {
    if (part == 0)
      for (int i = tid; i < G * D; i += kOnlineWaves * kWave) p.out[((int64_t)b * p.num_q_heads + hq0) * D + i] = 0.f;
    return;
  }
  const int t1 = min(t0 + T, ctx);
  const int n = t1 - t0;
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const int j0 = t0 / kBlockTokens;

  int64_t* offs = reinterpret_cast<int64_t*>(lds);
  float* wstat = lds + decode_off_floats(T);                            // [kOnlineWaves][G][2]
  uint8_t* mflag = reinterpret_cast<uint8_t*>(wstat + kOnlineWaves * G * 2);  // [T] mask (MASK only)
  // the K slots during the sweep, then the cross-wave reduction [kOnlineWaves][G][D]
  uint8_t* area = reinterpret_cast<uint8_t*>(lds) + bf16_online_area_offset(T, G, MASK);
  float* red = reinterpret_cast<float*>(area);
  for (int i = tid; i < nblk; i += kOnlineWaves * kWave) offs[i] = block_offset(p.c, b, g, j0 + i);
  if constexpr (MASK) {
    const uint8_t* mask_row = p.key_mask + (int64_t)b * p.key_mask_stride + t0;
    for (int t = tid; t < n; t += kOnlineWaves * kWave) mflag[t] = mask_row[t];
  }
  // fused append (as in decode_partition)
  if (p.k_new != nullptr && p.seq_lens[b] == ctx) {
    for (int i = 0; i < p.n_tail; ++i) {
      const int tn = ctx - p.n_tail + i;
      if (tn >= t0 && tn < t1) store_new_row<KVATTN_BF16, D>(p, b, g, tn, i);
    }
  }

  // q of head r16 in the k order of the K chunks: k-step s = 2c + u uses
  // d 32c + 8*lg + 4u + 0..3 (zero for heads >= G)
  uint32_t qb[2 * KC][2];
  {
    const int hr = r16 < G ? r16 : 0;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)b * p.num_q_heads + hq0 + hr) * D;
#pragma unroll
    for (int sd = 0; sd < 2 * KC; ++sd) {
      const uint2 w = *reinterpret_cast<const uint2*>(qrow + 32 * (sd / 2) + 8 * lg + 4 * (sd % 2));
      qb[sd][0] = r16 < G ? w.x : 0u;
      qb[sd][1] = r16 < G ? w.y : 0u;
    }
  }
  const float zscale = p.scale * kLog2e;
  __syncthreads();  // also publishes the fused append's stores to every wave

  auto key_ok = [&](int t) -> bool {
    if (t >= n) return false;
    if constexpr (MASK) return mflag[t] != 0;
    return true;
  };
  auto load_off = [&](int jb) -> int64_t {
    const int64_t o = offs[jb];
    return uniform64(o >= 0 ? o : 0);
  };
  // K through the wave's LDS slot (see KStage), V into registers: 8 bytes
  // (d 64*hf + 4*r16 ..+3) of each of keys 4*lg + i
  using KST = KStage<ROWB>;
  uint8_t* kslots = area + wave * 2 * KST::BYTES;  // this wave's two K slots
  int ksrc[KST::XFERS], kat[KC];
#pragma unroll
  for (int x = 0; x < KST::XFERS; ++x) ksrc[x] = KST::src(x, lane);
#pragma unroll
  for (int c = 0; c < KC; ++c) kat[c] = KST::at(r16, 4 * c + lg);
  // block jb goes to slot (jb / kOnlineWaves) % 2
  auto issue_k = [&](int jb) {
    const uint8_t* blk = p.c.k + load_off(jb);
    uint8_t* slot = kslots + ((jb / kOnlineWaves) & 1) * KST::BYTES;
#pragma unroll
    for (int x = 0; x < KST::XFERS; ++x) copy16_to_lds_async(blk + ksrc[x], slot + x * 1024);
  };
  const uint8_t* vbase = p.c.v + (4 * lg) * ROWB + 8 * r16;
  auto load_v = [&](int jb, uint2 (*vr)[4]) {
    const int64_t off = load_off(jb);
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[hf][i] = __builtin_bit_cast(
            uint2, __builtin_nontemporal_load(reinterpret_cast<const v2u*>(vbase + off + i * ROWB + 128 * hf)));
  };

  v4f o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;

  auto process = [&](int jb, const U4* kr, const uint2 (*vr)[4]) {
    if (uniform64(offs[jb]) < 0) return;  // block outside the cache: fully masked
    // ---- scores S^T (keys 4*lg + r, head r16), two accumulation chains ----
    v4f sacc = v4f{0.f, 0.f, 0.f, 0.f}, sacc2 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const v4s a0 = __builtin_bit_cast(v4s, v2u{kr[c].x, kr[c].y});
      const v4s a1 = __builtin_bit_cast(v4s, v2u{kr[c].z, kr[c].w});
      const v4s b0 = __builtin_bit_cast(v4s, v2u{qb[2 * c][0], qb[2 * c][1]});
      const v4s b1 = __builtin_bit_cast(v4s, v2u{qb[2 * c + 1][0], qb[2 * c + 1][1]});
      sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, b0, sacc, 0, 0, 0);
      sacc2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, b1, sacc2, 0, 0, 0);
    }
    sacc += sacc2;
    // ---- mask, block max, lazily raised running max ----
    const int tk = kBlockTokens * jb + 4 * lg;
    // several queries per sequence (TAIL): column r16 is query r16 % n_tail,
    // which sees keys below ctx - (n_tail - 1 - r16 % n_tail)
    const int ncol = TAIL ? ctx - (p.n_tail - 1 - r16 % p.n_tail) - t0 : n;
    float z[4];
    bool live[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      live[r] = key_ok(tk + r);
      z[r] = (live[r] && tk + r < ncol) ? sacc[r] * zscale : -INFINITY;
    }
    float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    {
      auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
      auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
    }
    const bool need = bm > mrun + kRescale;
    if (__any(need)) {
      const float mnew = need ? bm : mrun;
      const float alpha = need ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.f;  // 0 when mrun = -inf
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] *= alpha;
      lsum *= alpha;
      mrun = mnew;
    }
    const float msub = (mrun == -INFINITY) ? 0.f : mrun;
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = __builtin_amdgcn_exp2f(z[r] - msub);
      lsum += pw[r];
    }
    // weights as bf16 hi + lo (B operand: keys 4*lg + i)
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 h01, h23, l01, l23;
    h01[0] = (__bf16)pw[0];
    h01[1] = (__bf16)pw[1];
    h23[0] = (__bf16)pw[2];
    h23[1] = (__bf16)pw[3];
    l01[0] = (__bf16)(pw[0] - (float)h01[0]);
    l01[1] = (__bf16)(pw[1] - (float)h01[1]);
    l23[0] = (__bf16)(pw[2] - (float)h23[0]);
    l23[1] = (__bf16)(pw[3] - (float)h23[1]);
    const v4s phi = __builtin_bit_cast(v4s, v2u{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)});
    const v4s plo = __builtin_bit_cast(v4s, v2u{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
    // ---- O^T += V^T P^T: 4 keys x 4 d (16-bit) transposed per half ----
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf) {
      uint2 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = live[i] ? vr[hf][i] : uint2{0u, 0u};  // dead keys never reach O
      const uint32_t x01l = __builtin_amdgcn_perm(a[1].x, a[0].x, 0x05040100u);
      const uint32_t x23l = __builtin_amdgcn_perm(a[3].x, a[2].x, 0x05040100u);
      const uint32_t x01h = __builtin_amdgcn_perm(a[1].x, a[0].x, 0x07060302u);
      const uint32_t x23h = __builtin_amdgcn_perm(a[3].x, a[2].x, 0x07060302u);
      const uint32_t y01l = __builtin_amdgcn_perm(a[1].y, a[0].y, 0x05040100u);
      const uint32_t y23l = __builtin_amdgcn_perm(a[3].y, a[2].y, 0x05040100u);
      const uint32_t y01h = __builtin_amdgcn_perm(a[1].y, a[0].y, 0x07060302u);
      const uint32_t y23h = __builtin_amdgcn_perm(a[3].y, a[2].y, 0x07060302u);
      const v4s av[4] = {__builtin_bit_cast(v4s, v2u{x01l, x23l}), __builtin_bit_cast(v4s, v2u{x01h, x23h}),
                         __builtin_bit_cast(v4s, v2u{y01l, y23l}), __builtin_bit_cast(v4s, v2u{y01h, y23h})};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[4 * hf + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], phi, o[4 * hf + j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[4 * hf + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], plo, o[4 * hf + j], 0, 0, 0);
    }
  };

  // The wave's blocks jb = wave + kOnlineWaves i stream one block ahead: V through
  // a two-set register ring (stream_ring), K through the wave's two LDS
  // slots with transfers the compiler does not count (the waits below are
  // the only ones on them).  V of block i + 1 is issued before block i's
  // body, K of block i + 1 (into the other slot, read out in the previous
  // body) at the start of the body, so the loads issued after K of block i
  // are V and K of block i + 1, if it exists, and the load-count wait
  // releases exactly block i.  With the whole device streaming, more blocks
  // in flight per wave only lengthen every load's wait: each workgroup takes
  // longer to start and to finish for the same bandwidth, and the grid's
  // last workgroups, which run with the device half idle, finish later.
  constexpr int VL = 4 * HALVES;     // V loads per block
  constexpr int KL = KST::XFERS;     // K transfers per block
  uint2 vring[2][HALVES][4];
  auto body = [&](int jb, const uint2 (*vr)[4]) {
    const bool b1 = jb + kOnlineWaves < nblk;
    if (b1) issue_k(jb + kOnlineWaves);
    wait_vm_dyn(b1 ? VL + KL : 0);
    const uint8_t* slot = kslots + ((jb / kOnlineWaves) & 1) * KST::BYTES;
    U4 kr[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) kr[c] = *reinterpret_cast<const U4*>(slot + kat[c]);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the slot is read out before its next transfer
    process(jb, kr, vr);
  };
  ring_fill<2, uint2[HALVES][4], decltype(load_v), kOnlineWaves>(wave, nblk, vring, load_v);
  if (wave < nblk) issue_k(wave);
  stream_ring<2, uint2[HALVES][4], decltype(load_v), decltype(body), kOnlineWaves>(wave, nblk, vring, load_v, body);
  __syncthreads();  // every wave is done with its K slots: the area becomes the reduction

  // ---- combine the waves (as in decode_partition_fp8_mfma) ----
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (lg == 0 && r16 < G) {
    wstat[(wave * G + r16) * 2] = mrun;
    wstat[(wave * G + r16) * 2 + 1] = lsum;
  }
  constexpr int RS = red_stride(D);
  // lane (r16, lg) holds d = 64 hf + 4 (4 lg + rr) + j of head r16 in
  // o[4 hf + j][rr] (each wave's own scale is applied when combining)
  if (r16 < G) {
    float* row = red + (wave * G + r16) * RS;
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<float4*>(row + 64 * hf + 4 * (4 * lg + rr)) =
            make_float4(o[4 * hf][rr], o[4 * hf + 1][rr], o[4 * hf + 2][rr], o[4 * hf + 3][rr]);
  }
  __syncthreads();
  const int nparts_b = (ctx + T - 1) / T;
  for (int idx = tid; idx < G * D / 4; idx += kOnlineWaves * kWave) {
    const int h = idx / (D / 4), d = 4 * (idx - h * (D / 4));
    float Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < kOnlineWaves; ++w) Mh = fmaxf(Mh, wstat[(w * G + h) * 2]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kOnlineWaves; ++w) {
      const float mw = wstat[(w * G + h) * 2];
      const float sw = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mh);
      L = fmaf(sw, wstat[(w * G + h) * 2 + 1], L);
      const float4 x = *reinterpret_cast<const float4*>(red + (w * G + h) * RS + d);
      acc.x = fmaf(sw, x.x, acc.x);
      acc.y = fmaf(sw, x.y, acc.y);
      acc.z = fmaf(sw, x.z, acc.z);
      acc.w = fmaf(sw, x.w, acc.w);
    }
    const int hq = hq0 + h;
    if (nparts_b == 1) {
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      *reinterpret_cast<float4*>(p.out + ((int64_t)b * p.num_q_heads + hq) * D + d) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
      const int64_t slot = ((int64_t)b * p.num_q_heads + hq) * p.num_parts + part;
      *reinterpret_cast<float4*>(p.ws_o + slot * D + d) = acc;
      if (d == 0) {
        p.ws_ml[slot * 2] = Mh;
        p.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 cache with G >= 4 query heads per KV head: the partition pass on MFMA.
//
// With 8 heads per KV head an fp8 byte costs 8 multiply-adds on each of K and
// V, more than the vector ALUs can issue at HBM speed, so both contractions
// of a 16-token block go to v_mfma_f32_16x16x16_bf16 (fp8 -> bf16 is exact):
//   S^T[key][h] = K Q^T   A = K rows: lane l holds key l%16, 16-byte chunks
//                         c at row bytes 64c + 16(l/16) (one load reads 64
//                         contiguous bytes of 16 rows); k-step 4c + u takes
//                         word u of chunk c.  B = q of head l%16 in the same
//                         d order (zero for heads >= G).  The accumulator
//                         gives lane l keys 4(l/16) + r of head l%16.
//   O^T += V^T P^T        B = the lane's own 4 weights (keys 4(l/16) + r), so
//                         no data moves between lanes; A = V^T: lane l loads
//                         bytes D/16 * (l%16) .. + D/16 of keys 4(l/16)..+3
//                         (16 lanes read a whole row) and byte-transposes
//                         them with v_perm_b32, so output tile t row l%16
//                         holds d = D/16 * (l%16) + t.
// The weights are split into bf16 hi + lo parts (two MFMAs), so P keeps about
// 16 bits.  Each wave keeps its own running (max, sum, O) over its blocks with
// a lazily raised maximum; the four waves are combined through LDS.
template <int D, int G, bool MASK, bool TAIL>
__global__ void __launch_bounds__(256) decode_partition_fp8_mfma(const DecodeLaunch p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  constexpr int KC = D / 64;        // 16-byte K chunks per lane and block
  constexpr int KS = 4 * KC;        // k-steps of 4 codes
  constexpr int VW = D / 64;        // 4-byte V words per lane and key
  constexpr int VB = 4 * VW;        // V bytes per lane and key
  constexpr int NT = VB;            // output tiles of 16 d rows
  constexpr float kRescale = 8.f;
  static_assert(G >= 4 && G <= 16 && KC >= 1, "shape");
  typedef uint32_t VRow[VW];

  extern __shared__ float lds[];
  const int g = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  const int T = p.part_tokens;
  const int ctx = min(max(p.seq_lens[b], 0), p.ctx_limit);
  const int hq0 = g * G;
  const int t0 = part * T;
  if (t0 >= ctx) {
    if (part == 0)
      for (int i = tid; i < G * D; i += 256) p.out[((int64_t)b * p.num_q_heads + hq0) * D + i] = 0.f;
    return;
  }
  const int t1 = min(t0 + T, ctx);
  const int n = t1 - t0;
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const int j0 = t0 / kBlockTokens;

  int64_t* offs = reinterpret_cast<int64_t*>(lds);
  float* red = lds + decode_off_floats(T);  // [kWaves][G][kRedStride] outputs, then [kWaves][G][2]
  constexpr int RS = red_stride(D);
  float* wstat = red + kWaves * G * RS;
  uint8_t* mflag = reinterpret_cast<uint8_t*>(wstat + kWaves * G * 2);  // [T] mask (MASK only)
  for (int i = tid; i < nblk; i += 256) offs[i] = block_offset(p.c, b, g, j0 + i);
  if constexpr (MASK) {
    const uint8_t* mask_row = p.key_mask + (int64_t)b * p.key_mask_stride + t0;
    for (int t = tid; t < n; t += 256) mflag[t] = mask_row[t];
  }
  // fused append (as in decode_partition)
  if (p.k_new != nullptr && p.seq_lens[b] == ctx) {
    for (int i = 0; i < p.n_tail; ++i) {
      const int tn = ctx - p.n_tail + i;
      if (tn >= t0 && tn < t1) store_new_row<KVATTN_FP8_E4M3, D>(p, b, g, tn, i);
    }
  }

  // q of head r16 as bf16 pairs: k-step s uses d 4*KS*lg + 4s + 0..3, the
  // bytes of the K row that lane group lg holds (see the K load below)
  uint32_t qb[KS][2];
  {
    const int hr = r16 < G ? r16 : 0;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)b * p.num_q_heads + hq0 + hr) * D;
#pragma unroll
    for (int sd = 0; sd < KS; ++sd) {
      const uint2 w = *reinterpret_cast<const uint2*>(qrow + 4 * KS * lg + 4 * sd);
      qb[sd][0] = r16 < G ? w.x : 0u;
      qb[sd][1] = r16 < G ? w.y : 0u;
    }
  }
  const float zscale = p.scale * kLog2e * p.k_scale[g];
  __syncthreads();  // also publishes the fused append's stores to every wave

  v4f o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;

  auto cvt4 = [](uint32_t w, uint32_t& lo, uint32_t& hi) { fp8x4_to_bf16x4(w, lo, hi); };
  auto key_ok = [&](int t) -> bool {
    if (t >= n) return false;
    if constexpr (MASK) return mflag[t] != 0;
    return true;
  };
  // Block jb's K chunks and V words (jb < nblk); a block outside the cache
  // is read at offset 0, a valid address whose bytes are never used.
  // K: every load instruction reads whole 64-byte (D = 64) or 128-byte
  // (D = 128) rows.  D = 64: lane (r16, lg) reads bytes 16lg.. of row r16.
  // D = 128: load c reads rows 8c..8c+7, lane (r16, lg) bytes 16((r16 >> 3)
  // + 2lg).. of row 8c + (r16 & 7); one swap with the lane 8 apart (DPP row
  // rotate) then leaves lane (r16, lg) with bytes 32lg..32lg+31 of row r16.
  const uint8_t* kbase = (KC == 1) ? p.c.k + r16 * D + 16 * lg : p.c.k + (r16 & 7) * D + 16 * ((r16 >> 3) + 2 * lg);
  static_assert(KC <= 2, "K row split");
  const uint8_t* vbase = p.c.v + (4 * lg) * D + VB * r16;
  struct Blk {
    U4 k[KC];
    VRow v[4];
  };
  auto load = [&](int jb, Blk& blk) {
    U4* kr = blk.k;
    VRow* vr = blk.v;
    const int64_t o0 = offs[jb];
    const int64_t off = uniform64(o0 >= 0 ? o0 : 0);
#pragma unroll
    for (int c = 0; c < KC; ++c) kr[c] = stream_load(reinterpret_cast<const U4*>(kbase + off + 8 * D * c));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (VW == 2) {
        const uint2 w = __builtin_bit_cast(
            uint2, __builtin_nontemporal_load(reinterpret_cast<const v2u*>(vbase + off + i * D)));
        vr[i][0] = w.x;
        vr[i][VW - 1] = w.y;
      } else {
        vr[i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vbase + off + i * D));
      }
    }
  };
  auto process = [&](int jb, const Blk& blk) {
    const U4* kr = blk.k;
    const VRow* vr = blk.v;
    if (uniform64(offs[jb]) < 0) return;  // block outside the cache: fully masked
    // ---- scores S^T (keys 4*lg + r, head r16), two accumulation chains ----
    v4f sacc = v4f{0.f, 0.f, 0.f, 0.f}, sacc2 = v4f{0.f, 0.f, 0.f, 0.f};
    U4 kx[KC];
    if constexpr (KC == 1) {
      kx[0] = kr[0];
    } else {
      // lane r16 < 8 holds row r16's chunk 2lg (load 0) and row r16 + 8's
      // chunk 2lg (load 1); lane r16 >= 8 holds row r16 - 8's chunk 2lg + 1
      // and row r16's chunk 2lg + 1: each gives the other its foreign chunk
      const bool lo = r16 < 8;
      const uint32_t* k0 = reinterpret_cast<const uint32_t*>(&kr[0]);
      const uint32_t* k1 = reinterpret_cast<const uint32_t*>(&kr[1]);
      uint32_t* x0 = reinterpret_cast<uint32_t*>(&kx[0]);
      uint32_t* x1 = reinterpret_cast<uint32_t*>(&kx[1]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t give = lo ? k1[w] : k0[w];
        const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)give, kDppRowRor8, 0xF, 0xF, false);
        x0[w] = lo ? k0[w] : got;
        x1[w] = lo ? got : k1[w];
      }
    }
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(kx);
#pragma unroll
    for (int sd = 0; sd < KS; ++sd) {
      uint32_t a0, a1;
      cvt4(kw[sd], a0, a1);
      const v4s av = __builtin_bit_cast(v4s, v2u{a0, a1});
      const v4s bv = __builtin_bit_cast(v4s, v2u{qb[sd][0], qb[sd][1]});
      if (sd & 1)
        sacc2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, sacc2, 0, 0, 0);
      else
        sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, sacc, 0, 0, 0);
    }
    sacc += sacc2;
    // ---- mask, block max, lazily raised running max ----
    const int tk = kBlockTokens * jb + 4 * lg;
    // several queries per sequence (TAIL): column r16 is query r16 % n_tail,
    // which sees keys below ctx - (n_tail - 1 - r16 % n_tail)
    const int ncol = TAIL ? ctx - (p.n_tail - 1 - r16 % p.n_tail) - t0 : n;
    float z[4];
    bool live[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      live[r] = key_ok(tk + r);
      z[r] = (live[r] && tk + r < ncol) ? sacc[r] * zscale : -INFINITY;
    }
    float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    {
      auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
      auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
    }
    const bool need = bm > mrun + kRescale;
    if (__any(need)) {
      const float mnew = need ? bm : mrun;
      const float alpha = need ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.f;  // 0 when mrun = -inf
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] *= alpha;
      lsum *= alpha;
      mrun = mnew;
    }
    const float msub = (mrun == -INFINITY) ? 0.f : mrun;
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = __builtin_amdgcn_exp2f(z[r] - msub);
      lsum += pw[r];
    }
    // weights as bf16 hi + lo (B operand: keys 4*lg + i)
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 h01, h23, l01, l23;
    h01[0] = (__bf16)pw[0];
    h01[1] = (__bf16)pw[1];
    h23[0] = (__bf16)pw[2];
    h23[1] = (__bf16)pw[3];
    l01[0] = (__bf16)(pw[0] - (float)h01[0]);
    l01[1] = (__bf16)(pw[1] - (float)h01[1]);
    l23[0] = (__bf16)(pw[2] - (float)h23[0]);
    l23[1] = (__bf16)(pw[3] - (float)h23[1]);
    const v4s phi = __builtin_bit_cast(v4s, v2u{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)});
    const v4s plo = __builtin_bit_cast(v4s, v2u{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
    // ---- V^T tiles: transpose 4 keys x 4 d per word, zero dead keys ----
#pragma unroll
    for (int w = 0; w < VW; ++w) {
      uint32_t a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = live[i] ? vr[i][w] : 0u;  // keys with no weight never reach O
      const uint32_t t01l = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);
      const uint32_t t01h = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);
      const uint32_t t23l = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
      const uint32_t t23h = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
      const uint32_t tj[4] = {__builtin_amdgcn_perm(t23l, t01l, 0x05040100u),
                              __builtin_amdgcn_perm(t23l, t01l, 0x07060302u),
                              __builtin_amdgcn_perm(t23h, t01h, 0x05040100u),
                              __builtin_amdgcn_perm(t23h, t01h, 0x07060302u)};
      v4s av[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t b0, b1;
        cvt4(tj[j], b0, b1);
        av[j] = __builtin_bit_cast(v4s, v2u{b0, b1});
      }
      // hi parts of the four tiles, then the lo parts: no back-to-back
      // MFMAs on one accumulator
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[4 * w + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], phi, o[4 * w + j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[4 * w + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], plo, o[4 * w + j], 0, 0, 0);
    }
  };
  {
    Blk ring[kRingFp8];
    ring_fill(wave, nblk, ring, load);
    stream_ring(wave, nblk, ring, load, process);
  }

  // ---- combine the waves: per head, M = max of the wave maxima ----
  // the wave's row sum of head r16 is spread over its four lane groups
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (lg == 0 && r16 < G) {
    wstat[(wave * G + r16) * 2] = mrun;
    wstat[(wave * G + r16) * 2 + 1] = lsum;
  }
  // lane (r16, lg) holds d = VB (4 lg + rr) + t of head r16: 16-byte writes
  // of t = 4c .. 4c + 3 (each wave's own scale is applied when combining)
  if (r16 < G) {
    float* row = red + (wave * G + r16) * RS;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int c = 0; c < NT / 4; ++c)
        *reinterpret_cast<float4*>(row + VB * (4 * lg + rr) + 4 * c) =
            make_float4(o[4 * c][rr], o[4 * c + 1][rr], o[4 * c + 2][rr], o[4 * c + 3][rr]);
  }
  __syncthreads();
  const int nparts_b = (ctx + T - 1) / T;
  const float vscale = p.v_scale[g];
  for (int idx = tid; idx < G * D / 4; idx += 256) {
    const int h = idx / (D / 4), d = 4 * (idx - h * (D / 4));
    float Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Mh = fmaxf(Mh, wstat[(w * G + h) * 2]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = wstat[(w * G + h) * 2];
      const float sw = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mh);
      L = fmaf(sw, wstat[(w * G + h) * 2 + 1], L);
      const float4 x = *reinterpret_cast<const float4*>(red + (w * G + h) * RS + d);
      acc.x = fmaf(sw, x.x, acc.x);
      acc.y = fmaf(sw, x.y, acc.y);
      acc.z = fmaf(sw, x.z, acc.z);
      acc.w = fmaf(sw, x.w, acc.w);
    }
    acc.x *= vscale;
    acc.y *= vscale;
    acc.z *= vscale;
    acc.w *= vscale;
    const int hq = hq0 + h;
    if (nparts_b == 1) {
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      *reinterpret_cast<float4*>(p.out + ((int64_t)b * p.num_q_heads + hq) * D + d) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
      const int64_t slot = ((int64_t)b * p.num_q_heads + hq) * p.num_parts + part;
      *reinterpret_cast<float4*>(p.ws_o + slot * D + d) = acc;
      if (d == 0) {
        p.ws_ml[slot * 2] = Mh;
        p.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// Merge the split-K partials of one (sequence, query head).  256 threads =
// D/4 float4 columns x phases; a phase thread takes partitions ph, ph + PH,
// ... and issues all their loads (the (max, sum) pair and its float4 of the
// output) before using any, keeping its own running max, sum and output
// (each partition's weight exp2(m_p - M) relative to the running M); the
// phases are then combined in order through LDS.  The first U partitions of
// each phase are loaded together with the sequence length (every slot below
// num_parts is inside the workspace; slots at or past the sequence's own
// partition count hold stale bytes and are dropped unread), so the usual
// merge takes one round trip to memory.  Fixed order throughout, so the
// result is bitwise reproducible.
template <int D>
__global__ void __launch_bounds__(256) decode_merge(const DecodeLaunch p) {
  constexpr int NC = D / 4;       // float4 columns
  constexpr int PH = 256 / NC;    // partition phases
  constexpr int U = 5;            // partitions per batch of loads
  __shared__ float4 pacc[PH][NC];
  __shared__ float pm[PH], pl[PH];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, c = tid % NC, ph = tid / NC;
  const int64_t slot0 = ((int64_t)b * p.num_q_heads + hq) * p.num_parts;
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + slot0;
  const float4* wo = reinterpret_cast<const float4*>(p.ws_o + slot0 * D) + c;
  float2 s0[U];
  float4 x0[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int i = ph + k * PH;
    if (i < p.num_parts) {
      s0[k] = ml[i];
      x0[k] = wo[(int64_t)i * NC];
    }
  }
  const int T = p.part_tokens;
  const int ctx = min(max(p.seq_lens[b], 0), p.ctx_limit);
  const int np = (ctx + T - 1) / T;
  if (np <= 1) return;  // written by the partition pass
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float2 s, float4 x) {
    if (s.x == -INFINITY) return;  // partition with no attended key
    if (s.x > m) {
      const float alpha = exp2f(m - s.x);  // 0 while m = -inf
      acc.x *= alpha;
      acc.y *= alpha;
      acc.z *= alpha;
      acc.w *= alpha;
      l *= alpha;
      m = s.x;
    }
    const float w = exp2f(s.x - m);
    acc.x = fmaf(w, x.x, acc.x);
    acc.y = fmaf(w, x.y, acc.y);
    acc.z = fmaf(w, x.z, acc.z);
    acc.w = fmaf(w, x.w, acc.w);
    l = fmaf(w, s.y, l);
  };
#pragma unroll
  for (int k = 0; k < U; ++k)
    if (ph + k * PH < np) add(s0[k], x0[k]);
  int i = ph + U * PH;
  for (; i + (U - 1) * PH < np; i += U * PH) {
    float2 s[U];
    float4 x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      s[k] = ml[i + k * PH];
      x[k] = wo[(int64_t)(i + k * PH) * NC];
    }
#pragma unroll
    for (int k = 0; k < U; ++k) add(s[k], x[k]);
  }
  for (; i < np; i += PH) add(ml[i], wo[(int64_t)i * NC]);
  pacc[ph][c] = acc;
  if (c == 0) {
    pm[ph] = m;
    pl[ph] = l;
  }
  __syncthreads();
  if (ph == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < PH; ++k) M = fmaxf(M, pm[k]);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < PH; ++k) {
      if (pm[k] == -INFINITY) continue;
      const float w = exp2f(pm[k] - M);
      const float4 y = pacc[k][c];
      o.x = fmaf(w, y.x, o.x);
      o.y = fmaf(w, y.y, o.y);
      o.z = fmaf(w, y.z, o.z);
      o.w = fmaf(w, y.w, o.w);
      L = fmaf(w, pl[k], L);
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    reinterpret_cast<float4*>(p.out + ((int64_t)b * p.num_q_heads + hq) * D)[c] =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

template <int KVT, int D, int G, bool MASK, bool TAIL>
int launch_typed(const DecodeLaunch& a, hipStream_t s) {
  const dim3 grid(a.num_kv_heads, a.num_parts, a.batch);
  if constexpr (KVT == KVATTN_FP8_E4M3 && G >= 4) {
    const size_t lds = (size_t)(decode_off_floats(a.part_tokens) + kWaves * G * red_stride(D) + kWaves * G * 2 +
                                (MASK ? a.part_tokens / 4 : 0)) * sizeof(float);
    hipLaunchKernelGGL((decode_partition_fp8_mfma<D, G, MASK, TAIL>), grid, dim3(256), lds, s, a);
  } else if constexpr (KVT == KVATTN_BF16 && G >= KVATTN_BF16_ONLINE_MIN_G) {
    const size_t lds = (size_t)bf16_online_lds_bytes(a.part_tokens, G, D, MASK);
    hipLaunchKernelGGL((decode_partition_bf16_online<D, G, MASK, TAIL>), grid, dim3(kOnlineWaves * kWave), lds, s, a);
  } else if constexpr (KVT == KVATTN_BF16 && G >= 4) {
    const size_t lds = (size_t)kslot_offset(decode_lds_floats(a.part_tokens, G, D) + (MASK ? a.part_tokens / 4 : 0)) +
                       (size_t)kWaves * KStage<2 * D>::BYTES;
    hipLaunchKernelGGL((decode_partition_bf16_mfma<D, G, MASK, TAIL>), grid, dim3(256), lds, s, a);
  } else {
    const size_t lds = (size_t)(decode_lds_floats(a.part_tokens, G, D) + (MASK ? a.part_tokens / 4 : 0)) * sizeof(float);
    const dim3 pgrid(a.num_kv_heads, a.batch, a.num_parts);
    hipLaunchKernelGGL((decode_partition<KVT, D, G, MASK, TAIL>), pgrid, dim3(256), lds, s, a);
  }
  if (hipGetLastError() != hipSuccess) return KVATTN_ELAUNCH;
  if (a.num_parts > 1) {
    hipLaunchKernelGGL((decode_merge<D>), dim3(a.num_q_heads, a.batch), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return KVATTN_ELAUNCH;
  }
  return KVATTN_OK;
}

template <int KVT, int D, int G, bool TAIL>
int launch_mask(const DecodeLaunch& a, hipStream_t s) {
  return a.key_mask ? launch_typed<KVT, D, G, true, TAIL>(a, s) : launch_typed<KVT, D, G, false, TAIL>(a, s);
}

template <int KVT, int D, int G>
int launch_tail(const DecodeLaunch& a, hipStream_t s) {
  return a.n_tail > 1 ? launch_mask<KVT, D, G, true>(a, s) : launch_mask<KVT, D, G, false>(a, s);
}

template <int KVT, int D>
int launch_group(const DecodeLaunch& a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_tail<KVT, D, 1>(a, s);
    case 2: return launch_tail<KVT, D, 2>(a, s);
    case 4: return launch_tail<KVT, D, 4>(a, s);
    case 8: return launch_tail<KVT, D, 8>(a, s);
    case 16:  // matrix-core passes only (16 columns per KV head)
      if constexpr (KVT == KVATTN_F32) return KVATTN_EUNSUPPORTED;
      else return launch_tail<KVT, D, 16>(a, s);
    default: return KVATTN_EUNSUPPORTED;
  }
}

template <int KVT>
int launch_dim(const DecodeLaunch& a, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return launch_group<KVT, 64>(a, s);
    case 128: return launch_group<KVT, 128>(a, s);
    default: return KVATTN_EUNSUPPORTED;
  }
}

}  // namespace

int decode_lds_bytes(int part_tokens, int group, int head_dim) {
  return decode_lds_floats(part_tokens, group, head_dim) * (int)sizeof(float);
}

int launch_decode(const DecodeLaunch& a, hipStream_t s) {
  switch (a.cache_dtype) {
    case KVATTN_F32: return launch_dim<KVATTN_F32>(a, s);
    case KVATTN_BF16: return launch_dim<KVATTN_BF16>(a, s);
    case KVATTN_FP8_E4M3: return launch_dim<KVATTN_FP8_E4M3>(a, s);
    default: return KVATTN_EUNSUPPORTED;
  }
}

}  // namespace kvattn
