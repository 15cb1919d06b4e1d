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
// and Decode"), so both products run on the matrix cores.
//
// Budget on gfx950 per compute unit (measured): the matrix cores reach
// ~1.9 PFLOP/s on back-to-back 32x32x16 bf16 MFMAs, the LDS serves ~256
// bytes per clock for 16-byte reads, and exp2 issues at a quarter of the
// vector rate.  Per 32-key tile a wave's softmax costs about as much vector
// ALU time as its 16 MFMAs take on the matrix core, so the kernel runs two
// waves per SIMD: while one wave works through its softmax, the other's
// MFMAs keep the matrix core busy.  That fixes the register budget at 256
// per wave (all in vector registers: no accumulation registers are used, so
// the compiler may give the wave the whole budget), which holds one 32-column
// query block per wave: Q, O^T, two steps of scores and the weights.
//
// Work split.  A workgroup of 8 waves owns HW = min(G, 8) query heads of one
// KV head and 256 / HW query rows, cut into eight 32-row column blocks, one
// per wave.  The heads of a GQA group share the K/V tiles staged in LDS.
// The KV head is the fastest grid dimension, so with 8 KV heads every XCD
// (and its L2) serves one KV head; causal query tiles are issued heaviest
// first.
//
// Staging.  32-key tiles of K and V go from global memory straight into an
// 8-tile LDS ring (7 with an fp8 prefix; buffer loads that write LDS), 5
// tiles ahead of the one being scored; each wave waits only for its own
// transfers of the tile it publishes, and one barrier per step publishes
// it.  V stays row-major in LDS and its MFMA operand is read with the
// transposing LDS read.
//
// Pipeline.  Step t runs the QK^T product of tile t+1, the softmax of tile
// t and the PV product of tile t-1: three independent parts that the
// compiler interleaves.  Tiles away from the causal diagonal and the
// sequence end take a step without mask tests.
//
// Per 32-key tile and column block (h = lane / 32):
//   S^T[key][q] = K Q^T      A = K rows from LDS, B = Q (registers), fp32
//                            accumulate.  The 32x32 accumulator gives lane l
//                            query column l % 32 and keys 8*(r/4) + 4h + r%4
//                            (r = 0..15): a query's scores sit in two lanes,
//                            so the row max is a local max plus one
//                            cross-half swap, and P^T is already the B
//                            operand of the second product.
//   P = exp2(S*c - m)        c = scale*log2(e); m is a per-query running
//                            maximum that is only raised (with rescaling of
//                            the accumulators) when the tile maximum exceeds
//                            it by more than 64, so P <= 2^64; P rounded to
//                            bf16.
//   O^T[d][q] += V^T P^T     A = V^T, read from row-major V in LDS so that
//                            its operand slots hold the keys in P^T's order.
//   l[q] += P . 1            bf16 dot products of the rounded weights, so the
//                            row sum is the sum of the same weights used for O.
// Masked keys (causal, beyond q_len, key_mask) get P = 0 and their V rows are
// staged as zeros, so non-finite padding never reaches O.
//
// Cached prefix (chunked prefill, verification of drafted tokens: query t at
// position P + t also attends the cached positions 0 .. P-1; "KV Cache"
// (heepie.pages.dev), section "Prefill and Decode", and "Transformer
// Attention Masks and KV-Cache Inference", section "Prefill and decode
// stages").  Keys are then indexed from position 0; tiles are gathered row
// by row, a prefix row through the block table (or the contiguous cache) and
// a new row from the new K/V, with per-lane global-to-LDS transfers.  The
// workgroup first checks that every prefix block id is valid; if one is not,
// its positions are masked keys and every tile takes the masked step.  The
// ids of a paged prefix are copied to LDS by that check, and a tile of whole
// cached blocks takes its rows' addresses from them without a branch.
//
// fp8 cache prefix.  An E4M3FN code is exactly a bf16 value, so a cached row
// is staged as its codes (not yet scaled).  The 32-key tile grid is shifted
// so that a tile starts at key P: a tile then holds only cached keys or only
// new ones.  The codes of a cached tile (half the bytes of its bf16 rows)
// take one 16-byte global-to-LDS transfer per lane into a staging ring, and
// when the tile is published each wave expands its piece into the bf16
// slots.  The dequantisation
// scales ("KV Cache Fully Explained", section "(1) FP8 quantization": values
// are stored at 8 bits with a scale) enter as factors: the K scale is folded
// into the score scale of the tiles of cached keys, and since every cached
// key precedes every new one, the output accumulates the cached keys' V
// codes unscaled and is multiplied by the V scale once, before the PV
// product of the tile that starts at P.  The row sums take the weights as
// they are.
#include <math.h>

#include <type_traits>

#include "launch.h"

namespace kvattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kKeys = 32;      // keys per tile
constexpr int kCB = 1;                 // 32-row query column blocks per wave
constexpr int kWaves = 8;              // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBlocks = kWaves * kCB;  // 32-row query column blocks per workgroup
constexpr int kBufs = 8;       // LDS tile buffers (a ring)
constexpr int kAhead = 5;      // tiles loaded ahead of the one being scored
constexpr float kLog2e = 1.4426950408889634f;
// log2 headroom before the running max moves: weights stay below 2^64, far
// inside the range of bf16 weights and fp32 sums, so a moved maximum (and
// the rescaling of the accumulators it needs) is rare.
constexpr float kRescale = 64.0f;

__device__ __forceinline__ f32x16 mfma(const U4& a, const U4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// An empty inline-assembly statement (it emits no instruction) that needs
// x: the loads that produce x complete before it.  Used so that no load the
// compiler tracks is still in flight inside the tile loop, whose waits would
// otherwise also wait for the tile transfers.
__device__ __forceinline__ void settle(const U4& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  asm volatile("" ::"v"(__builtin_bit_cast(u32x4, x)));
#endif
}

// Marks the scores as written at this point (an empty asm statement), so
// the softmax that reads them stays inside the step that issues it, between
// the matrix products it is meant to overlap, instead of being moved into a
// block of its own between steps.
__device__ __forceinline__ void pin(f32x16& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
}

// Marks a value as used at this point (an empty asm statement).
__device__ __forceinline__ void keep(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

// sum of the two bf16 weights of w, accumulated in fp32
__device__ __forceinline__ float dot2_ones(uint32_t w, float acc) {
  const uint32_t one2 = 0x3F803F80u;  // two bf16 1.0
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, one2), acc,
                                         false);
}

// LDS geometry (bytes) of one tile buffer: K and V rows of D*2 bytes in
// 16-byte chunks, unpadded.  The LDS
// serves 256 bytes per clock: 16 lanes of a 16-byte read, or 32 lanes of
// an 8-byte read, must touch 16 distinct 16-byte slots modulo 256 bytes.
// So the chunk index of row r is XOR-swizzled:
//   K (16-byte reads, 16 lanes = rows r .. r+15 at one chunk):
//     d = 128 (256-byte rows): c ^ (r % 16);
//     d = 64 (128-byte rows, two per 256 bytes): c ^ ((r / 2) % 8);
//   V (transposing 8-byte reads, 32 lanes = 4 rows x 2 d halves x 4 pieces):
//     d = 128: c ^ 4 (r % 4);  d = 64: c ^ 4 ((r / 2) % 2).
// VP: the V tile in placed-row form (d = 128), so that every transposing V
// read of a step is one per-lane address plus constant offsets.  Key k of
// the tile sits in piece k % 4 + 4 (k / 16), row (k / 4) % 4 of that 1 KB
// piece, its chunks in order, and each piece is followed by 64 bytes of
// padding: the four keys a 16-lane group reads together (k % 4 = 0..3) lie
// in four pieces whose rows start 64 bytes apart in the bank cycle, so the
// group's reads fall on distinct banks without an XOR swizzle of the chunks.
template <int D, bool VP = false>
struct Geo {
  static constexpr int RB = D * 2;  // row bytes
  static constexpr int NC = D / 8;  // 16-byte chunks per row
  static constexpr int KBYTES = kKeys * RB;
  static constexpr int VPIECE = VP ? 1024 + 64 : 1024;  // bytes per 1 KB piece of V in LDS
  static constexpr int VBYTES = kKeys * RB / 1024 * VPIECE;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int PIECES = kKeys * NC / 64;                   // 1 KB pieces per operand
  static constexpr int LOADS = PIECES >= kWaves ? PIECES / kWaves : 1;  // pieces per loading wave
  static constexpr int LWAVES = PIECES / LOADS;                       // waves that load
  static_assert(LOADS * LWAVES == PIECES && LWAVES <= kWaves, "tile split over the waves");
  static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// gfx950 memory operations used below, as small wrappers whose bodies exist
// in the device pass only (the host pass compiles the kernel for its launch
// stub and never runs it).
//
// A buffer resource (the four descriptor words) over `bytes` bytes at
// `base`: loads at offsets past the end return zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)p, (int)(uint32_t)((p >> 32) & 0xffffu), bytes, 0x00020000};
}
// 16 bytes per lane from rsrc + voffset straight into LDS at lds + 16 * lane
// (lds uniform over the wave).  Issued as inline assembly: the compiler
// then does not treat the transfer as a pending LDS store, which would make
// it wait for every load in flight before any LDS read of the tile ring;
// completion is awaited explicitly (finish_tile) before a barrier publishes
// the tile.
__device__ __forceinline__ void load_lds16(const i32x4& rsrc_in, uint8_t* lds, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  // the descriptor is the same in every lane; say so, so that it is held in
  // scalar registers as the instruction requires
  const i32x4 rsrc = {__builtin_amdgcn_readfirstlane(rsrc_in[0]), __builtin_amdgcn_readfirstlane(rsrc_in[1]),
                      __builtin_amdgcn_readfirstlane(rsrc_in[2]), __builtin_amdgcn_readfirstlane(rsrc_in[3])};
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
#endif
}
// 16 bytes per lane from the global address src straight into LDS at
// lds + 16 * lane (lds uniform over the wave): the per-lane-address form,
// for rows gathered from the cache.  Inline assembly for the same reason as
// load_lds16: the compiler must not wait on the transfer before LDS reads.
__device__ __forceinline__ void load_lds16_ptr(const uint8_t* src, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(m0), "v"(src)
      : "memory", "m0");
#endif
}
// ds_read_b64_tr_b16 of 4 16-bit values at an LDS address.
__device__ __forceinline__ s16x4 read_tr16(const uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)lds);
#else
  return s16x4{};
#endif
}

// LDS of the kernel: the tile buffers, then (fp8 prefix) a staging
// ring of kStage tiles of fp8 codes (per loading wave 512 bytes of K codes,
// then 512 of V).  Codes wait in it from their transfer until the tile is
// published: at most tiles it + 2 .. it + kAhead, four (the prologue publishes
// tile 0 before it issues tile 4).
constexpr int kStage = kAhead - 1;
// The placed-row V form needs d = 128 and the tile-wide transfers of a
// prompt without a cached prefix (a prefix tile is gathered row by row with
// K and V rows in the same order; the fp8 prefix has no LDS to spare).
template <int D, bool PREFIX, bool FP8P>
constexpr bool v_placed() { return D == 128 && !PREFIX && !FP8P; }
// With a cached prefix in a paged cache, the block ids of the prefix (up to
// tbl_max blocks) are copied to LDS after the tile ring (and the staging
// ring) when the workgroup checks them, so gathering a tile's rows reads
// its block ids from LDS: a global read of the table would make the wave
// wait for its tile transfers still in flight (the vector-memory counter is
// in order).  An fp8 prefix gives one of the 8 tile buffers to it (7 still
// hold the tiles it - 1 .. it + kAhead in use).  At d = 128 the rings and
// the table fill the 160 KB.
template <bool FP8P>
constexpr int ring_bufs() { return FP8P ? kAhead + 2 : kBufs; }
template <bool PREFIX, bool FP8P>
constexpr int tbl_max() { return !PREFIX ? 0 : FP8P ? 4096 : 8192; }
template <int D, bool PREFIX, bool FP8P>
constexpr int prefill_lds_bytes() {
  return ring_bufs<FP8P>() * Geo<D, v_placed<D, PREFIX, FP8P>()>::BUF + (FP8P ? kStage * 2 * kKeys * D : 0) +
         tbl_max<PREFIX, FP8P>() * 4;
}

template <int D, bool CAUSAL, bool MASK, bool PREFIX, bool FP8P>
__global__ void __launch_bounds__(kThreads, 1) prefill_mfma_kernel(const PrefillLaunch a, int hw) {
  static_assert(PREFIX || !FP8P, "fp8 rows come only from a cached prefix");
  constexpr bool VPL = v_placed<D, PREFIX, FP8P>();
  using GE = Geo<D, VPL>;
  constexpr int NB = ring_bufs<FP8P>();     // tile buffers in the ring
  constexpr int S8 = kKeys * D;             // bytes of one operand's fp8 codes per tile
  constexpr int DK = D / 16;  // 16-wide d chunks of the QK^T contraction
  constexpr int DT = D / 32;  // 32-row d tiles of the output
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform over the wave
  const int hh = lane >> 5, lc = lane & 31;
  const int b = blockIdx.z;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int rows_wg = 32 * kBlocks / hw;  // query rows of the workgroup
  const int bph = rows_wg / 32;           // column blocks per head
  const int qtile = gridDim.y - 1 - blockIdx.y;  // heaviest (causal) first
  const int h0 = blockIdx.x * hw;
  const int g = h0 / G;
  const int q_wg = qtile * rows_wg;
  const int n_max = a.n_max;
  const int qlen = a.q_lens ? min(max(a.q_lens[b], 0), n_max) : n_max;
  const int P = a.positions ? max(a.positions[b], 0) : 0;
  // Keys are indexed from kbase: the cached prefix (positions 0 .. P-1, read
  // from the cache) when it is attended, else the first new token.  Query t
  // sits at position P + t, i.e. at key index t + QO; Ltot keys exist.
  constexpr bool prefix = PREFIX;  // a.has_cache && a.attend_prefix
  const int kbase = prefix ? 0 : P;
  const int QO = P - kbase;
  const int Ltot = QO + qlen;

  // this wave's two column blocks: head hb[cb], first row rb[cb]
  int hb[kCB], rb[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int j = kCB * wave + cb;
    hb[cb] = h0 + j / bph;
    rb[cb] = q_wg + 32 * (j % bph);
  }
  const int row_lo = min(rb[0], rb[kCB - 1]), row_hi = max(rb[0], rb[kCB - 1]) + 32;

  if (q_wg >= qlen) {  // the whole tile is padding rows: zeros
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      float* out_h = a.out + ((int64_t)b * a.num_q_heads + hb[cb]) * n_max * D;
      for (int r = 0; r < 32; ++r) {
        const int t = rb[cb] + r;
        if (t < n_max)
          for (int d = lane; d < D; d += 64) out_h[(int64_t)t * D + d] = 0.f;
      }
    }
    return;
  }
  // Tile t holds keys 32t - ksh .. 32t - ksh + 31.  With an fp8 prefix the
  // grid is shifted so that a tile starts at key P: no tile then holds both
  // cached and new keys (keys below 0 are absent, masked in the first tile).
  const int ksh = FP8P ? (kKeys - P % kKeys) % kKeys : 0;
  const int key_end = CAUSAL ? min(Ltot, QO + q_wg + rows_wg) : Ltot;  // workgroup bound
  const int wave_end = CAUSAL ? min(Ltot, QO + row_hi) : Ltot;          // this wave's bound
  const int ntiles = (key_end + ksh + kKeys - 1) / kKeys;
  const int wave_tiles = (wave_end + ksh + kKeys - 1) / kKeys;
  // Whether every prefix position lies in the cache (a valid block id for
  // each of its blocks): one scan of the sequence's table row by the
  // workgroup.  Prefix positions outside the cache are masked keys.
  bool prefix_ok = true;
  constexpr bool TBL = PREFIX;
  constexpr int kTblMax = tbl_max<PREFIX, FP8P>();
  // prefix block ids (TBL), after the tile ring and the fp8 staging ring
  int32_t* const tbl = reinterpret_cast<int32_t*>(smem + NB * GE::BUF + (FP8P ? kStage * 2 * S8 : 0));
  bool tbl_ok = false;  // uniform: every prefix block id is in tbl
  if (PREFIX && P > 0) {
    // the flag lives in the first bytes of the tile ring (no static LDS: with
    // an fp8 prefix the dynamic LDS is the whole 160 KB); a barrier after it
    // is read keeps the first tile transfers from overwriting it early
    int& bad = *reinterpret_cast<int*>(smem);
    if (tid == 0) bad = 0;
    __syncthreads();
    const CacheView& cv = a.c;
    if (cv.paged) {
      const int nb = (P + kBlockTokens - 1) / kBlockTokens;
      int mine = nb > cv.max_blocks;
      const int32_t* row = cv.block_table + (int64_t)b * cv.max_blocks;
      for (int j = tid; j < min(nb, cv.max_blocks); j += kThreads) {
        const int32_t blk = row[j];
        mine |= (blk < 0) | ((int64_t)blk >= cv.num_blocks);
        if (TBL && j < kTblMax) tbl[j] = blk;
      }
      if (mine) bad = 1;
      tbl_ok = TBL && nb <= min(cv.max_blocks, kTblMax);
    } else if (tid == 0 && (int64_t)P > cv.capacity) {
      bad = 1;
    }
    __syncthreads();
    prefix_ok = __builtin_amdgcn_readfirstlane(bad) == 0;  // uniform (the loop bounds depend on it)
    __syncthreads();
  }
  // fp8 prefix: the dequantisation scales of KV head g.  The tile that
  // starts at key P (the first new key) is where the output takes the V
  // scale, before its PV product.
  float ksc = 1.f, vsc = 1.f;
  if constexpr (FP8P) {
    ksc = a.k_scale[g];
    vsc = a.v_scale[g];
  }
  // Tiles below fast_end need no mask: every key is real, in the cache and
  // causally visible to every query of the wave.
  // With an fp8 prefix, a K scale <= 0 (which cannot be folded into the
  // score scale of the running maximum) makes every step masked.
  const int fast_end = (MASK || !prefix_ok || (FP8P && !(ksc > 0.f)))
                           ? 0
                           : min(wave_tiles, ((CAUSAL ? min(Ltot, QO + row_lo + 1) : Ltot) + ksh) / kKeys);

  const int64_t head_bytes = (int64_t)n_max * D * 2;
  const uint8_t* kg = a.k + ((int64_t)b * a.num_kv_heads + g) * head_bytes;
  const uint8_t* vg = a.v + ((int64_t)b * a.num_kv_heads + g) * head_bytes;
  const uint8_t* mrow = MASK ? a.key_mask + (int64_t)b * a.key_mask_stride : nullptr;

  // ---- Q fragments (B operand of S^T = K Q^T): row rb + lc, d 16c + 8hh ----
  int tq[kCB];
  U4 qf[kCB][DK];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    tq[cb] = rb[cb] + lc;
    const uint8_t* qg = a.q + ((int64_t)b * a.num_q_heads + hb[cb]) * n_max * D * 2;
#pragma unroll
    for (int c = 0; c < DK; ++c)
    {
      qf[cb][c] = (tq[cb] < n_max) ? *reinterpret_cast<const U4*>(qg + ((int64_t)tq[cb] * D + 16 * c + 8 * hh) * 2)
                                   : U4{0, 0, 0, 0};
    }
  }

  // ---- staging of one K/V tile: global -> LDS directly ----
  // Each wave moves GE::LOADS 1 KB pieces of K and of V per tile with
  // buffer loads that write LDS (lane i fills bytes 16i .. 16i+15 of the
  // piece); a lane fetches the global chunk whose swizzled slot that is.
  // The buffer resource of a tile starts at its first key and holds only
  // the keys below min(q_len, end of the workgroup's last tile): loads past
  // it return zeros, so rows of absent keys are staged as zeros.  With a key
  // mask, rows of masked keys are zeroed by the loading wave once its loads
  // have landed, so no non-finite padding reaches the PV product.
  const int key_lim = min(Ltot, ntiles * kKeys - ksh);
  // per lane, tile independent: the rows of its K and V slots and the
  // global offsets of the chunks that fill them
  int koff[GE::LOADS], voff[GE::LOADS], lrow[GE::LOADS], vrow[GE::LOADS];
#pragma unroll
  for (int i = 0; i < GE::LOADS; ++i) {
    const int slot = (wave * GE::LOADS + i) * 64 + lane;  // 16-byte slot in the tile
    const int r = slot / GE::NC, cs = slot % GE::NC;
    lrow[i] = r;
    koff[i] = r * GE::RB + (cs ^ GE::swz_k(r)) * 16;
    if constexpr (VPL) {  // piece pc, row lane / 16 of it: key pc % 4 + 4 (lane / 16) + 16 (pc / 4)
      const int pc = wave * GE::LOADS + i;
      vrow[i] = (pc & 3) + 4 * (lane >> 4) + 16 * (pc >> 2);
      voff[i] = vrow[i] * GE::RB + (lane & 15) * 16;
    } else {
      vrow[i] = r;
      voff[i] = r * GE::RB + (cs ^ GE::swz_v(r)) * 16;
    }
  }
  // With a prefix, every tile is gathered row by row: key index k is cache
  // position kbase + k (below P) or new token k - QO.  A row that is absent
  // (k >= Ltot) or outside the cache is read from new token 0 (a valid
  // address) and zeroed once it has landed, like a masked key's V row.
  constexpr bool zero_rows = MASK || PREFIX;
  // A key is valid if it is a real token (< q_len) and, with a key mask, its
  // mask byte (at absolute position P + key) is nonzero.  The byte is read at
  // a clamped index and the terms are combined bitwise, so the test has no
  // branch (a branchy form of this test was miscompiled).
  const int mask_last = MASK ? (int)min<int64_t>(a.key_mask_stride, (int64_t)INT32_MAX) - 1 : 0;
  auto key_valid = [&](int key) -> bool {
    bool ok = key < Ltot;
    if (FP8P) ok = ok & (key >= 0);  // the shifted first tile
    if (MASK) {
      const int mi = FP8P ? max(kbase + key, 0) : kbase + key;
      const uint8_t mb = mrow[min(mi, mask_last)];  // always inside the mask row
      ok = ok & (kbase + key <= mask_last) & (mb != 0);
    }
    if (PREFIX && !prefix_ok) {  // uniform: only with prefix positions outside the cache
      const int ka = kbase + key;
      ok = ok & ((ka >= P) || (position_offset(a.c, b, g, ka) >= 0));
    }
    return ok;
  };
  // With a key mask or a prefix, per lane and tile in flight: bit i = this
  // lane's V piece of load i belongs to a masked key; bit 4 (fp8 prefix) =
  // the tile's keys are cached rows whose codes are in the staging ring.  A
  // queue, oldest tile in the low byte: load_tile appends at byte `slot`
  // (the number of tiles already queued), finish_tile pops the low byte.
  static_assert(GE::LOADS <= 4, "per-tile flags fit a byte");
  static_assert(!FP8P || GE::LOADS == 1, "fp8 staging: one piece of K and V per loading wave");
  uint64_t pending = 0;
  // fp8 prefix, a tile of cached keys: lane L fetches the 16 codes of the
  // two slots 2(L % 32) and 2(L % 32) + 1 of its wave's piece (K for L < 32,
  // V above) into the staging ring at 16 L.  The two slots are adjacent
  // chunks of one row, and the swizzle XORs chunk indices with a value that
  // keeps such a pair together, so their codes are one aligned 16 bytes of
  // the cached row.
  const int f_op = lane >> 5;
  const int f_slot = wave * 64 + 2 * (lane & 31);
  const int f_row = f_slot / GE::NC;
  const int f_chunk = (((f_slot % GE::NC) ^ (f_op ? GE::swz_v(f_row) : GE::swz_k(f_row))) >> 1) * 16;
  // the cache operand this lane fetches codes of, chosen once (a per-lane
  // choice between the two kernel-argument pointers inside the loop became a
  // per-lane load of the argument, waited for with the tile transfers)
  const uintptr_t f_cache =
      (uintptr_t)a.c.k + (f_op ? (uintptr_t)a.c.v - (uintptr_t)a.c.k : (uintptr_t)0);
  uint8_t* const stage = smem + NB * GE::BUF;  // [kStage][pieces][K 512 B, V 512 B] (fp8 prefix)
  // per lane (tbl_ok): offset of its K chunk within a block of the cache
  // (head g, row lrow % 16); its V chunk is voff - koff further
  int64_t tile_row_off[GE::LOADS];
#pragma unroll
  for (int i = 0; i < GE::LOADS; ++i)
    tile_row_off[i] = (int64_t)g * a.c.head_stride + (int64_t)(lrow[i] % kBlockTokens) * a.c.row_stride +
                      (koff[i] - lrow[i] * GE::RB);
  // cache offset of prefix position ka (0 <= ka < P) from the block ids in
  // LDS (tbl_ok), -1 for an invalid id, as position_offset gives
  auto tbl_offset = [&](int ka) -> int64_t {
    const CacheView& cv = a.c;
    const int32_t blk = tbl[ka / kBlockTokens];
    if (blk < 0 || (int64_t)blk >= cv.num_blocks) return -1;
    return (int64_t)blk * cv.block_stride + (int64_t)g * cv.head_stride + (int64_t)(ka % kBlockTokens) * cv.row_stride;
  };
  auto load_tile = [&](int t, int slot) {
    const int kt0 = t * kKeys - ksh;
    uint8_t* kl = smem + (t % NB) * GE::BUF;
    uint8_t* vl = kl + GE::KBYTES;
    if (wave >= GE::LWAVES) return;
    if constexpr (zero_rows) {
      uint32_t info = 0;
#pragma unroll
      for (int i = 0; i < GE::LOADS; ++i) {
        const int key = kt0 + vrow[i];  // the key of this lane's V slot
        // without a prefix, rows at or past key_lim arrive as zeros already
        if ((prefix || key < key_lim) && !key_valid(key)) info |= 1u << i;
      }
      pending |= (uint64_t)info << (8 * slot);
    }
    if constexpr (PREFIX) {
      if (FP8P && kt0 < P) {  // uniform: a tile of cached keys (the grid has no mixed tile)
        const int key = kt0 + f_row;
        const uint8_t* src = kg;  // new token 0: the stand-in for rows outside the cache
        if (key >= 0) {
          const int64_t off = tbl_ok ? tbl_offset(kbase + key) : position_offset(a.c, b, g, kbase + key);
          if (off >= 0) src = reinterpret_cast<const uint8_t*>(f_cache + off + f_chunk);
        }
        // issued twice (the same bytes to the same place): every tile then
        // takes two transfers per lane, and the waits stay constants
        load_lds16_ptr(src, stage + (t % kStage) * 2 * S8 + wave * 1024);
        load_lds16_ptr(src, stage + (t % kStage) * 2 * S8 + wave * 1024);
        pending |= (uint64_t)16 << (8 * slot);
        return;
      }
      if (FP8P && kt0 >= P) {  // uniform: new tokens only, contiguous in k / v
        // one bounded buffer resource per operand: rows at or past Ltot read
        // as zeros (and are zeroed again as absent keys).  With a bf16 prefix
        // this measured slower (the row-by-row path below serves it).
        const int nbytes = max(Ltot - kt0, 0) * GE::RB;
        const i32x4 kr = make_rsrc(kg + (int64_t)(kt0 - P) * GE::RB, nbytes);
        const i32x4 vr = make_rsrc(vg + (int64_t)(kt0 - P) * GE::RB, nbytes);
#pragma unroll
        for (int i = 0; i < GE::LOADS; ++i) {
          const int piece = wave * GE::LOADS + i;
          load_lds16(kr, kl + piece * 1024, koff[i]);
          load_lds16(vr, vl + piece * GE::VPIECE, voff[i]);
        }
        return;
      }
      if (tbl_ok && prefix_ok && kt0 + kKeys <= P) {  // uniform: cached rows only, every id valid
        // a tile is whole blocks (kt0 is a multiple of kKeys), so a lane's row
        // sits at the same place in its block in every tile
        static_assert(kKeys % kBlockTokens == 0, "tiles of whole cache blocks");
#pragma unroll
        for (int i = 0; i < GE::LOADS; ++i) {
          const int64_t off = (int64_t)tbl[(kt0 + lrow[i]) / kBlockTokens] * a.c.block_stride + tile_row_off[i];
          const int piece = wave * GE::LOADS + i;
          load_lds16_ptr(a.c.k + off, kl + piece * 1024);
          load_lds16_ptr(a.c.v + off + (voff[i] - koff[i]), vl + piece * GE::VPIECE);
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < GE::LOADS; ++i) {
        const int key = kt0 + lrow[i];
        const int ka = kbase + key;
        const uint8_t* rk = kg;  // new token 0: the stand-in for absent rows
        const uint8_t* rv = vg;
        if (key < Ltot) {
          if (ka >= P) {
            rk = kg + (int64_t)(ka - P) * GE::RB;
            rv = vg + (int64_t)(ka - P) * GE::RB;
          } else {
            const int64_t off = tbl_ok ? tbl_offset(ka) : position_offset(a.c, b, g, ka);
            if (off >= 0) {
              rk = a.c.k + off;
              rv = a.c.v + off;
            }
          }
        }
        const int piece = wave * GE::LOADS + i;
        load_lds16_ptr(rk + (koff[i] - lrow[i] * GE::RB), kl + piece * 1024);
        load_lds16_ptr(rv + (voff[i] - lrow[i] * GE::RB), vl + piece * GE::VPIECE);
      }
      return;
    }
    const int nbytes = max(key_lim - kt0, 0) * GE::RB;
    const i32x4 kr = make_rsrc(kg + (int64_t)kt0 * GE::RB, nbytes);
    const i32x4 vr = make_rsrc(vg + (int64_t)kt0 * GE::RB, nbytes);
#pragma unroll
    for (int i = 0; i < GE::LOADS; ++i) {
      const int piece = wave * GE::LOADS + i;
      load_lds16(kr, kl + piece * 1024, koff[i]);
      load_lds16(vr, vl + piece * GE::VPIECE, voff[i]);
    }
  };
  // Waits until at most `younger` tiles' loads of this wave are in flight
  // (so the oldest pending tile, t, has landed), then (fp8 prefix) expands
  // the staged codes of a tile of cached keys into its bf16 slots and (key
  // mask, prefix) zeroes its masked V rows.  Each loading lane issues two
  // transfers per tile and load.
  auto finish_tile = [&](int t, auto younger) {
    constexpr int vm = decltype(younger)::value * 2 * GE::LOADS;
    static_assert(vm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((vm & 15) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8));  // vmcnt(vm)
    if constexpr (zero_rows) {
      // the LDS accesses below touch bytes the transfers wrote: keep them after the wait
      __asm__ volatile("" ::: "memory");
      uint8_t* vl = smem + (t % NB) * GE::BUF + GE::KBYTES;
      const uint32_t info = (uint32_t)pending & 0xffu;
      pending >>= 8;
      if constexpr (FP8P) {
        if (info & 16u) {  // uniform
          uint8_t* kl = smem + (t % NB) * GE::BUF;
          const uint8_t* st = stage + (t % kStage) * 2 * S8 + wave * 1024 + (lane >> 1) * 16;
          const int gk = (koff[0] - lrow[0] * GE::RB) >> 4, gv = (voff[0] - lrow[0] * GE::RB) >> 4;
          const U2 ck = *reinterpret_cast<const U2*>(st + (gk & 1) * 8);
          const U2 cv = *reinterpret_cast<const U2*>(st + 512 + (gv & 1) * 8);
          U4 wk, wv;
          fp8x4_to_bf16x4(ck.x, wk.x, wk.y);
          fp8x4_to_bf16x4(ck.y, wk.z, wk.w);
          fp8x4_to_bf16x4(cv.x, wv.x, wv.y);
          fp8x4_to_bf16x4(cv.y, wv.z, wv.w);
          *reinterpret_cast<U4*>(kl + wave * 1024 + lane * 16) = wk;
          *reinterpret_cast<U4*>(vl + wave * 1024 + lane * 16) = wv;
        }
      }
#pragma unroll
      for (int i = 0; i < GE::LOADS; ++i)
        if (info & (1u << i)) *reinterpret_cast<U4*>(vl + (wave * GE::LOADS + i) * GE::VPIECE + lane * 16) = U4{0, 0, 0, 0};
    }
  };

  // S^T of the tile in buffer `buf`, both column blocks: keys
  // kt0 + 8*(r/4) + 4hh + r%4, query rb[cb] + lc.  Each K fragment feeds the
  // two column blocks.
  auto scores = [&](int buf, f32x16 (&s)[kCB]) {
    const uint8_t* kl = smem + buf * GE::BUF;
#pragma unroll
    for (int cc = 0; cc < DK; ++cc) {
      const U4 kf = *reinterpret_cast<const U4*>(kl + lc * GE::RB + ((2 * cc + hh) ^ GE::swz_k(lc)) * 16);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) s[cb] = mfma(kf, qf[cb][cc], cc == 0 ? f32x16{} : s[cb]);
    }
  };

  // ---- accumulators ----
  f32x16 o[kCB][DT];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][dt][r] = 0.f;
  float mrun[kCB], lpart[kCB];  // lpart: this lane's half of the row sum
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    mrun[cb] = -INFINITY;
    lpart[cb] = 0.f;
  }
  const float c = a.scale * kLog2e;

  // Softmax of the scores of the tile at kt0 into bf16 weights pf (and the
  // row-sum halves); alpha receives the factor by which o must be rescaled
  // once the previous tile's PV product is in, and `resc` whether any lane
  // of the wave needs it.
  auto softmax = [&](auto masked, int kt0, int buf, f32x16 (&s)[kCB], U4 (&pf)[kCB][2], float (&alpha)[kCB], bool& resc) {
    float ct = c;  // score scale (log2 domain) of the tile
    if constexpr (FP8P) {
      if (kt0 < P) {  // uniform: a tile of cached keys (codes: the K scale is due)
        if (ksc > 0.f) {
          ct = c * ksc;
        } else if constexpr (decltype(masked)::value) {
          // every step is masked then; the scale goes in before the mask
#pragma unroll
          for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) s[cb][r] *= ksc;
        }
      }
    }
    if constexpr (decltype(masked)::value) {
      // causal edge, keys beyond q_len, key mask (keys kt0 + 8gq + 4hh + e)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          const int key = kt0 + 8 * gq + 4 * hh + e;
          const bool kok = key_valid(key);
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) {
            const bool ok = kok & (!CAUSAL || key <= tq[cb] + QO);
            s[cb][r] = ok ? s[cb][r] : -INFINITY;
          }
        }
    }
    bool any_need = false;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      // running maximum of this query (log2 domain), raised lazily
      // a balanced tree (depth 4): both waves of a SIMD reach it together
      float t8[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) t8[r] = fmaxf(s[cb][2 * r], s[cb][2 * r + 1]);
#pragma unroll
      for (int r = 0; r < 4; ++r) t8[r] = fmaxf(t8[2 * r], t8[2 * r + 1]);
      float tm = fmaxf(fmaxf(t8[0], t8[1]), fmaxf(t8[2], t8[3]));
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
        tm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * ct;
      }
      const bool need = tm > mrun[cb] + kRescale;
      const float mnew = need ? tm : mrun[cb];
      alpha[cb] = need ? __builtin_amdgcn_exp2f(mrun[cb] - mnew) : 1.f;  // argument < -64 or -inf: 0
      any_need |= need && mrun[cb] != -INFINITY;  // nothing accumulated yet: nothing to rescale
      mrun[cb] = mnew;
      const float msub = (mnew == -INFINITY) ? 0.f : mnew;
      float l = lpart[cb] * alpha[cb];
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[cb][r], ct, -msub));
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        pf[cb][m] = U4{pack_bf16(p[8 * m], p[8 * m + 1]), pack_bf16(p[8 * m + 2], p[8 * m + 3]),
                       pack_bf16(p[8 * m + 4], p[8 * m + 5]), pack_bf16(p[8 * m + 6], p[8 * m + 7])};
        l = dot2_ones(pf[cb][m].x, l);
        l = dot2_ones(pf[cb][m].y, l);
        l = dot2_ones(pf[cb][m].z, l);
        l = dot2_ones(pf[cb][m].w, l);
      }
      lpart[cb] = l;
    }
    resc = __any(any_need);
    if constexpr (FP8P) {
      // the tile that starts at key P: the cached keys' V codes accumulated
      // so far take the V scale before its PV product (with any rescale of
      // the running maximum); l is not scaled
      if (kt0 == P) {
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) alpha[cb] *= vsc;
        resc = true;
      }
    }
  };

  // O^T += V^T P^T for the tile in buffer `buf`; each V^T fragment feeds
  // the two column blocks.  V^T fragments come from row-major V with
  // ds_read_b64_tr_b16: in each group of 16 lanes, lane j reads 4 values of
  // d at row j / 4 and receives, per element e, the value that lane
  // 4e + i/4 read at position i % 4 (i = its own index in the group), so
  // lane i ends with rows kb + 0..3 at one d.  Lane l of the A operand needs
  // d = 32 dt + l % 32 and the 8 keys of its operand slots, 4h + 0..3 and
  // 8 + 4h + 0..3 of the 16-key slab (h = l / 32): two reads.
  const int tr_e = (lane & 15) >> 2, tr_q = lane & 3, tr_dh = (lane >> 4) & 1;
  // One V^T fragment (A operand of the PV product, key slab m, d tile dt).
  // Placed V rows: key r = 16 m + 8 u + 4 h + e is in piece e + 4 m, row
  // 2 u + h, so the address is one per-lane base plus constants.
  const int vbase = tr_e * GE::VPIECE + hh * GE::RB + (2 * tr_dh + (tr_q >> 1)) * 16 + 8 * (tr_q & 1);
  auto v_frag = [&](const uint8_t* vl, int m, int dt) -> U4 {
    s16x4 half[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (VPL) {
        half[u] = read_tr16(vl + vbase + m * 4 * GE::VPIECE + u * 2 * GE::RB + dt * 64);
      } else {
        const int ch = 4 * dt + 2 * tr_dh + (tr_q >> 1);  // 16-byte chunk of d
        const int r = 16 * m + 8 * u + 4 * hh + tr_e;
        half[u] = read_tr16(vl + r * GE::RB + ((ch ^ GE::swz_v(r)) * 16) + 8 * (tr_q & 1));
      }
    }
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 h0 = __builtin_bit_cast(u32x2, half[0]), h1 = __builtin_bit_cast(u32x2, half[1]);
    return U4{h0[0], h0[1], h1[0], h1[1]};
  };
  auto pv = [&](int buf, const U4 (&pf)[kCB][2], f32x16 (&o)[kCB][DT]) {
    const uint8_t* vl = smem + buf * GE::BUF + GE::KBYTES;
#pragma unroll
    for (int f = 0; f < 2 * DT; ++f) {
      const U4 vf = v_frag(vl, f / DT, f % DT);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) o[cb][f % DT] = mfma(vf, pf[cb][f / DT], o[cb][f % DT]);
    }
  };

  auto rescale = [&](const float (&alpha)[kCB], f32x16 (&o)[kCB][DT]) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[cb][dt] *= alpha[cb];
  };

  // Step it: scores of tile it + 1, softmax of tile it and the PV product of
  // tile it - 1.  Tile it + kAhead is loaded meanwhile and tile it + 2,
  // loaded kAhead - 2 steps earlier, is published by the barrier that ends
  // the step.  Buffers t % NB hold tiles it - 1 .. it + kAhead.  Every wave
  // runs the same number of steps (ntiles + 1), so the barriers match.  The
  // three parts are independent: the compiler interleaves them, and the
  // other wave of the SIMD fills the matrix or vector units while this one
  // waits.
  //
  // Fast step (tiles 1 <= it < fast_end: no mask, a predecessor, all three
  // parts).  It does not rescale o itself: when its softmax moves a running
  // maximum (resc), the caller rescales o before the next PV product.
  auto fast_step = [&](int it, f32x16 (&s_cur)[kCB], f32x16 (&s_nxt)[kCB], const U4 (&p_prev)[kCB][2],
                       U4 (&p_cur)[kCB][2], float (&alpha)[kCB], bool& resc, f32x16 (&o)[kCB][DT]) {
    load_tile(it + kAhead, kAhead - 2);
    // after the transfers' (uniform) branch, in the block of the products
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) pin(s_cur[cb]);
    scores((it + 1) % NB, s_nxt);
    softmax(std::false_type{}, it * kKeys - ksh, it % NB, s_cur, p_cur, alpha, resc);
    pv((it + NB - 1) % NB, p_prev, o);
    finish_tile(it + 2, std::integral_constant<int, kAhead - 2>{});
    // the weights and row sums are complete here, beside this step's matrix
    // products: left to itself the compiler moves their computation down to
    // the next step's PV product, which for the second step of the loop
    // body means into a block of its own between the steps
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      settle(p_cur[cb][0]);
      settle(p_cur[cb][1]);
      keep(lpart[cb]);
    }
    __syncthreads();
  };
  // General step: masked softmax, the parts this step has, and the rescale.
  auto slow_step = [&](int it, f32x16 (&s_cur)[kCB], f32x16 (&s_nxt)[kCB], const U4 (&p_prev)[kCB][2],
                       U4 (&p_cur)[kCB][2], f32x16 (&o)[kCB][DT]) {
    load_tile(it + kAhead, kAhead - 2);
    float alpha[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) alpha[cb] = 1.f;
    bool resc = false;
    if (it + 1 < wave_tiles) scores((it + 1) % NB, s_nxt);
    if (it < wave_tiles) softmax(std::true_type{}, it * kKeys - ksh, it % NB, s_cur, p_cur, alpha, resc);
    if (it >= 1 && it - 1 < wave_tiles) pv((it + NB - 1) % NB, p_prev, o);
    finish_tile(it + 2, std::integral_constant<int, kAhead - 2>{});
    if (resc) rescale(alpha, o);
    __syncthreads();
  };

  // prologue: tiles 0 .. kAhead - 1 in flight, tiles 0 and 1 published,
  // scores of tile 0
  if constexpr (FP8P) {
    // tile 0 is published (its staged codes expanded) before tile 4 is issued
    // into the staging slot it used
#pragma unroll
    for (int t = 0; t < kAhead - 1; ++t) load_tile(t, t);
    finish_tile(0, std::integral_constant<int, kAhead - 2>{});
    load_tile(kAhead - 1, kAhead - 2);
  } else {
#pragma unroll
    for (int t = 0; t < kAhead; ++t) load_tile(t, t);
    finish_tile(0, std::integral_constant<int, kAhead - 1>{});
  }
  finish_tile(1, std::integral_constant<int, kAhead - 2>{});
  __syncthreads();
  f32x16 sA[kCB], sB[kCB];
  U4 pA[kCB][2], pB[kCB][2];
  if (wave_tiles > 0) scores(0, sA);
  slow_step(0, sA, sB, pA, pB, o);  // the first real tile never rescales (and has no PV)
  // here sB holds the scores of tile 1 and pB the weights of tile 0
  int it = 1;
  bool resc = false;
  float alpha[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) alpha[cb] = 1.f;
  auto advance = [&]() {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      sA[cb] = sB[cb];
      pA[cb][0] = pB[cb][0];
      pA[cb][1] = pB[cb][1];
    }
  };
  advance();
  // nothing the compiler tracks may be in flight in the fast loop: its waits
  // would then also wait for the tile transfers
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int c = 0; c < DK; ++c) settle(qf[cb][c]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // Two steps per iteration with the score and weight buffers trading roles,
  // so the step-to-step hand-over needs no register copies (advance copies
  // once when a step is left over).  A step whose softmax moved a running
  // maximum rescales o before the next step's PV product.
  while (it + 1 < fast_end) {
    fast_step(it, sA, sB, pA, pB, alpha, resc, o);
    if (resc) rescale(alpha, o);
    fast_step(it + 1, sB, sA, pB, pA, alpha, resc, o);
    if (resc) rescale(alpha, o);
    it += 2;
  }
  if (it < fast_end) {
    fast_step(it, sA, sB, pA, pB, alpha, resc, o);
    if (resc) rescale(alpha, o);
    advance();
    ++it;
  }
  for (; it <= ntiles; ++it) {
    slow_step(it, sA, sB, pA, pB, o);
    advance();
  }

  // ---- epilogue: O^T[d][q] / l[q] -> out[q][d]; rows >= q_len are 0 ----
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart[cb]), __float_as_uint(lpart[cb]), false, false);
    const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (tq[cb] < n_max) {
      float* out_h = a.out + ((int64_t)b * a.num_q_heads + hb[cb]) * n_max * D;
      const bool live = tq[cb] < qlen;
      const float inv = (live && l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          float4 w;
          w.x = live ? o[cb][dt][4 * rg] * inv : 0.f;
          w.y = live ? o[cb][dt][4 * rg + 1] * inv : 0.f;
          w.z = live ? o[cb][dt][4 * rg + 2] * inv : 0.f;
          w.w = live ? o[cb][dt][4 * rg + 3] * inv : 0.f;
          *reinterpret_cast<float4*>(out_h + (int64_t)tq[cb] * D + 32 * dt + 8 * rg + 4 * hh) = w;
        }
    }
  }

  // ---- cache write: the K/V rows of this workgroup's query tile ----
  // One workgroup owns each (sequence, KV head, query tile), so the tiles'
  // rows (those below q_len) are written exactly once, as kv_append writes
  // them: token i goes to position positions[b] + i, skipped outside the
  // cache.  They were just staged from these addresses, so the reads hit L2.
  if (a.write_cache) {
    constexpr int CPR = D * 2 / 16;  // 16-byte chunks per row
    const int nrows = min(rows_wg, qlen - q_wg);
    const int p0 = a.positions ? a.positions[b] : 0;
    const CacheView cv = a.c;
    for (int idx = tid; idx < nrows * CPR; idx += kThreads) {
      const int i = q_wg + idx / CPR, ch = idx % CPR;
      const int64_t off = position_offset(cv, b, g, (int64_t)p0 + i);
      if (off < 0) continue;
      const int64_t src = (int64_t)i * GE::RB + ch * 16;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 xk = *reinterpret_cast<const u32x4*>(kg + src);
      const u32x4 xv = *reinterpret_cast<const u32x4*>(vg + src);
      *reinterpret_cast<u32x4*>(cv.k + off + ch * 16) = xk;
      *reinterpret_cast<u32x4*>(cv.v + off + ch * 16) = xv;
    }
  }
}

template <int D, bool CAUSAL, bool MASK, bool PREFIX, bool FP8P>
int launch_typed(const PrefillLaunch& a, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int hw = G < kBlocks ? G : kBlocks;
  const int rows = 32 * kBlocks / hw;
  const dim3 grid(a.num_q_heads / hw, (a.n_max + rows - 1) / rows, a.batch);
  static_assert(prefill_lds_bytes<D, PREFIX, FP8P>() <= 160 * 1024, "LDS of one workgroup");
  const size_t lds = prefill_lds_bytes<D, PREFIX, FP8P>();
  hipLaunchKernelGGL((prefill_mfma_kernel<D, CAUSAL, MASK, PREFIX, FP8P>), grid, dim3(kThreads), lds, s, a, hw);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ELAUNCH;
}

template <int D, bool PREFIX, bool FP8P>
int launch_flags(const PrefillLaunch& a, hipStream_t s) {
  if (a.causal)
    return a.key_mask ? launch_typed<D, true, true, PREFIX, FP8P>(a, s)
                      : launch_typed<D, true, false, PREFIX, FP8P>(a, s);
  return a.key_mask ? launch_typed<D, false, true, PREFIX, FP8P>(a, s)
                    : launch_typed<D, false, false, PREFIX, FP8P>(a, s);
}

template <int D>
int launch_prefix(const PrefillLaunch& a, hipStream_t s) {
  if (!(a.has_cache && a.attend_prefix)) return launch_flags<D, false, false>(a, s);
  return a.cache_dtype == KVATTN_FP8_E4M3 ? launch_flags<D, true, true>(a, s) : launch_flags<D, true, false>(a, s);
}

}  // namespace

bool prefill_mfma_supports(const PrefillLaunch& a) {
  if (a.dtype != KVATTN_BF16) return false;
  if (a.head_dim != 64 && a.head_dim != 128) return false;
  // a cached prefix is read from a bf16 cache or an fp8 cache (its codes
  // expanded to bf16 in LDS, the scales applied as factors)
  if (a.has_cache && a.attend_prefix && a.cache_dtype != KVATTN_BF16 && a.cache_dtype != KVATTN_FP8_E4M3) return false;
  // the running maximum is taken as max(scores) * scale, which needs scale > 0
  if (!(a.scale > 0.f)) return false;
  if ((int64_t)a.n_max * a.head_dim * 2 >= ((int64_t)1 << 31) - 4096) return false;  // 32-bit buffer offsets
  const int G = a.num_q_heads / a.num_kv_heads;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

int launch_prefill_mfma(const PrefillLaunch& a, hipStream_t s) {
  return a.head_dim == 64 ? launch_prefix<64>(a, s) : launch_prefix<128>(a, s);
}

}  // namespace kvattn
