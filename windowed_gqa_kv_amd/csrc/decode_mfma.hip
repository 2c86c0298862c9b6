// Split-KV decode on CDNA4 matrix cores (bf16 / fp16 cache, fp32 math),
// head sizes 64, 128 and 256, any number of new tokens per step.
//
// Decode streams the cache once per (batch, KV head): its cost is HBM bytes,
// not arithmetic.  The G*curr query rows that share one KV head (query heads
// of the group x new tokens) form the N dimension of small MFMAs, so every K/V
// byte fetched from HBM is used by all of them and the vector ALUs are left
// for the softmax.  Without that, the fp32 FMAs of the rows sharing a KV head
// at head size 256 would need most of the chip's vector-ALU rate to keep up
// with HBM.
//
// Semantics: query row t of batch b sits at position total_b - curr + t and
// sees cache slots [0, total_b) through the causal band and the window
// ("[NPUW] Support GQA sliding-window and smooth-softmax in DecomposeGQA",
// section "Sliding window (local_window_size)"); the sink enters only the
// final denominator (same page, section "smooth_softmax / head_sink").
//
// Schedule: one balanced round.  A row tile is 16 query rows of one (batch,
// KV head); its keys are the union of its rows' allowed intervals, cut into
// 16-key units.  Every workgroup computes the same split of the units (the
// lengths live on the device); the grid is exactly as many workgroups as the
// GPU holds at once, so all of them stream from the first microsecond and
// finish together.  With at least two workgroups per row tile, each tile
// gets whole workgroups in proportion to its units and every slice stays
// inside one tile (a slice that crosses a tile boundary drains its stream
// there).  With fewer, the slices are equal cuts of the flattened unit list
// and may cross tile boundaries.  Each piece (slice x tile) leaves one fp32
// partial (acc, max, sum).  At the end every workgroup bumps the arrival
// counter of each tile it touched; the last arrival of a tile merges its
// partials, folds the sink and writes O.  Each merge is the work of one wave,
// so a workgroup that completes several tiles merges them side by side.
//
// Per 16-key unit: each wave streams its units into a private ring of LDS
// stages with wave-wide LDS DMA loads (global_load_lds_dwordx4: 1 KB per
// instruction, no registers held while in flight), several units ahead of
// the one it computes.  K rows are read from LDS straight into the A operand
// of v_mfma_f32_16x16x32 (S^T = K Q^T, Q in registers); V is read with the
// transposing LDS load ds_read_b64_tr_b16 straight into the A operand of
// v_mfma_f32_16x16x16 (O^T += V^T P^T), whose B operand layout is exactly
// the score accumulator layout.  Rows are stored with an XOR swizzle of their
// 16-byte chunks (chosen per lane in the DMA source address) so that both
// LDS read patterns are free of bank conflicts.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace gqa {
namespace {

constexpr int kRowsPerTile = 16;
constexpr int kSub = 16;              // keys per unit (MFMA M)
constexpr int kWaves = 4;
constexpr float kRescaleLog2 = 8.0f;
constexpr int kMaxTiles = kDecodeMaxTiles;  // row tiles per call on this path
constexpr int kMaxGrid = 2048;        // workgroups per launch (upper bound)
constexpr int kCachedTiles = 160;     // tiles whose lengths the setup keeps in LDS
constexpr int kNonTemporal = 2;       // cache-policy bits of a load: nt (gfx950)

// LDS staging of one wave: kStages units of K and V in flight, 16 KB per
// wave for head sizes up to 128 (two workgroups share a CU, so one wave's
// softmax overlaps another's loads) and 32 KB at head size 256 (two stages of
// 16 KB units; one workgroup per CU).
// An FP8 (E4M3) cache (KV8) streams units of D bytes per key row into kStages
// row-major fp8 stages and converts the unit about to be computed into one
// 16-bit K + V buffer of the usual layout; the footprint is unchanged.
template <int D, bool KV8 = false>
struct Ring {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kSlots = D / 8;                     // 16-byte chunks per key row
  static constexpr int kUnitBytes = kSub * kRowBytes;      // K (or V) bytes of one 16-bit unit
  static constexpr int kInBytes = KV8 ? kSub * D : kUnitBytes;  // K (or V) bytes of one streamed unit
  static constexpr int kDmaPerUnit = kInBytes / 1024;      // wave-wide 16-byte DMA loads
  static constexpr int kBudget = D >= 256 ? 32768 : 16384;
  static constexpr int kBufBytes = KV8 ? 2 * kUnitBytes : 0;
  static constexpr int kStages = (kBudget - kBufBytes) / (2 * kInBytes);
  static constexpr int kBufOff = kStages * 2 * kInBytes;  // the converted K + V unit (KV8)
  static constexpr int kWaveBytes = kBufOff + kBufBytes;
  static_assert(kInBytes % 1024 == 0, "a unit is whole DMA instructions");
  static_assert(kStages >= 2, "at least two units in flight");
  static_assert((kStages - 1) * 2 * kDmaPerUnit <= 63, "vmcnt range");
};

// Chunk slot of 16-byte chunk cc of key row `key` (0..15) is cc ^ swz(key).
// The K read (16 rows x one chunk column per 16 lanes) and the transposing V
// read (4 rows x 2 chunks per 16 lanes) then hit every LDS bank equally.
template <int D>
__device__ __forceinline__ int swz(int key) {
  if constexpr (D >= 128)
    return (2 * key + (key >> 3)) & 15;
  else
    return (2 * (key >> 1) + (key >> 3)) & 7;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Wait until at most `pending` units (of M loads each) are still in flight.
template <int M, int S>
__device__ __forceinline__ void wait_units(int pending) {
  if constexpr (S > 1) {
    if (pending >= S - 1) {
      wait_vm<(S - 1) * M>();
      return;
    }
    wait_units<M, S - 1>(pending);
  } else {
    wait_vm<0>();
  }
}

// LDS reads of data that arrived by LDS DMA.  They are written as inline
// assembly that also waits for its own results: the compiler would otherwise
// place a wait for every outstanding DMA load (vmcnt(0)) in front of each
// LDS read, which serialises the stream.  The DMA waits are explicit
// (wait_units) and precede these blocks.  Their vector results are only ever
// consumed whole, as MFMA operands: this compiler mis-assigns sub-registers
// when single elements of a vector-typed inline-asm result are used.
__device__ __forceinline__ void lds_read2_b128(u32x4& a0, u32x4& a1, uint32_t p0, uint32_t p1) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1)
      : "v"(p0), "v"(p1)
      : "memory");
}
__device__ __forceinline__ void lds_read4_tr16(u32x2& a0, u32x2& a1, u32x2& a2, u32x2& a3, uint32_t p0,
                                               uint32_t p1, uint32_t p2, uint32_t p3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3)
      : "memory");
}

// s_waitcnt vmcnt(p * M) for a wave-uniform p in [0, P].
template <int M, int P>
__device__ __forceinline__ void wait_vm_multiple(int p) {
  if constexpr (P > 0) {
    if (p >= P) {
      wait_vm<P * M>();
      return;
    }
    wait_vm_multiple<M, P - 1>(p);
  } else {
    wait_vm<0>();
  }
}

template <bool IS_BF16>
__device__ __forceinline__ f32x4 mma_qk(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (IS_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <bool IS_BF16>
__device__ __forceinline__ f32x4 mma_pv(u32x2 a, u32x2 b, f32x4 c) {
  if constexpr (IS_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}


// Partials travel between workgroups (possibly on different XCDs, whose L2s
// are not coherent with each other): writers use device-scope relaxed atomic
// stores, which write through to the coherent level, and wait for them to
// complete before bumping an arrival counter; only the workgroup that merges a
// tile then acquires at device scope.  No workgroup writes back or
// invalidates a whole cache on the streaming path.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four consecutive floats at byte offset `off` of a partial with the cache
// policy of the device-scope store above (SC1), 16 bytes wide: a lane's four
// accumulators of a 16-column block are contiguous, so the 16 lanes of a row
// write whole 64-byte lines in one instruction instead of a quarter line in
// each of four.  A raw buffer store over the partial's bytes (out-of-range
// offsets are dropped by the hardware), which the compiler tracks like any
// other store; the writers' vmcnt(0) before their arrivals waits for it.
constexpr int kCpolSC1 = 16;                  // cache-policy bit SC1 (device scope) on gfx94x/gfx950
constexpr int kRawBufferWord3 = 0x00020000;   // raw (untyped) buffer resource, gfx9 data format field
__device__ __forceinline__ void coherent_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCpolSC1);
}

// A row tile and the union of its rows' allowed intervals.
struct Tile {
  int b, g, rt, bg;
  BatchSpan sp;
  int lo, hi;        // union key interval (empty when lo > hi)
  int rows_tile;     // query rows in this tile (<= 16)
};
// With a caller mask the union interval starts at a multiple of 16 keys (the
// keys before a row's band are masked like any other excluded key), so that a
// lane's four mask entries of a unit form one aligned load.
__device__ __forceinline__ Tile make_tile(const AttnArgs& a, int rows, int nrt, int t, bool align16) {
  Tile x;
  x.bg = t / nrt;
  x.rt = t - x.bg * nrt;
  x.b = x.bg / a.Hkv;
  x.g = x.bg - x.b * a.Hkv;
  x.sp = batch_span(a, x.b);
  const int r_first = kRowsPerTile * x.rt;
  x.rows_tile = min(kRowsPerTile, rows - r_first);
  x.lo = row_lo(a, x.sp.q_off + r_first / a.G);
  x.hi = row_hi(a, x.sp.q_off + (r_first + x.rows_tile - 1) / a.G, x.sp.valid);
  if (align16 && x.lo <= x.hi) x.lo &= ~(kSub - 1);
  return x;
}
__device__ __forceinline__ int units_of(const Tile& x) {
  return x.lo <= x.hi ? (x.hi - x.lo) / kSub + 1 : 0;
}
// The workgroup whose slice holds unit u when slice k is [floor(U k / G), floor(U (k+1) / G)).
__device__ __forceinline__ int owner_of(int u, int U, int G) {
  return (int)((((int64_t)u + 1) * G - 1) / U);
}

template <bool IS_BF16, int D>
__device__ __forceinline__ void store_row4(const AttnArgs& a, int b, int h, int t, int d0, f32x4 x) {
  uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)t * a.o_ss + d0;
  *reinterpret_cast<u32x2*>(op) = u32x2{pack2<IS_BF16>(x[0], x[1]), pack2<IS_BF16>(x[2], x[3])};
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts within
// each row of 16 lanes, then the totals of the lower rows (read lanes).
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}
__device__ __forceinline__ int wave_sum(int v, int lane) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v, lane), 63);
}
// floor(x * i / n) for 0 <= x < 2^31 and 0 <= i, n <= 2048, in 32-bit integers.
__device__ __forceinline__ int mul_div(int x, int i, int n) {
  const int q = x / n, r = x - q * n;
  return q * i + (r * i) / n;
}

// LSE-combine of two partial states (max M in log2 units, sum Ls, acc) that
// share a lane layout; an empty state has M = -inf and contributes nothing.
template <int QPL>
__device__ __forceinline__ void lse_combine(float& M, float& Ls, f32x4 (&acc)[QPL], float Mo, float Lo,
                                            const float (&ao)[QPL * 4]) {
  const float Mn = fmaxf(M, Mo);
  const float fa = Mn == -INFINITY ? 0.0f : fast_exp2(M - Mn);
  const float fb = Mn == -INFINITY ? 0.0f : fast_exp2(Mo - Mn);
  Ls = Ls * fa + Lo * fb;
#pragma unroll
  for (int q = 0; q < QPL; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[q][e] = acc[q][e] * fa + ao[4 * q + e] * fb;
  M = Mn;
}

// Merge of one row tile's split partials by MW waves of a workgroup, wave cw
// over the cw-th 1 / MW of the columns (no LDS: every wave reads all maxima
// and sums, which its factors need, and only its own accumulator columns):
// log-sum-exp over the splits, sink folded into the denominator, normalised,
// narrowed with round-to-nearest-even and stored.
// Split x of the tile is the partial at gpart + x * PART (acc [16][D], then
// 16 maxima in log2 units, then 16 sums).  The tile's rows are padded to
// Rp = 2^lrp and each row gets 64 / Rp lanes; a lane owns QPL output quads of
// its row (a chunk) and merges them over its splits, NB splits in flight at
// once.  Where a row has more lanes than the wave's quads, several lanes
// share a chunk as split groups, combined with shuffles at the end.
template <bool IS_BF16, int D, int QPL, int MW>
__device__ __forceinline__ void merge_tile_q(const AttnArgs& a, int lrp, int R, int rt, int xb, int xg,
                                             const float* __restrict__ gpart, int nvalid, int lane, int cw) {
  constexpr int PART = kRowsPerTile * D + 2 * kRowsPerTile;
  constexpr int Q4 = D / 4;  // output quads per row
  constexpr int NCA = Q4 / QPL;  // chunks per row
  constexpr int NC = NCA / MW;   // chunks per row of this wave (from cw NC on)
  static_assert(NCA % MW == 0, "whole chunks per wave");
  // splits per lane in flight: 64 loaded quads per lane, or 128 at D = 256,
  // whose kernel runs one workgroup per CU and has the registers to spare
  constexpr int NB = (D >= 256 ? 32 : 16) / QPL;
  static_assert(Q4 % QPL == 0, "whole chunks");
  const int L = 64 >> lrp;           // lanes per row
  const int r = lane >> (6 - lrp);
  const int sub = lane & (L - 1);
  const int CL = min(L, NC);         // lanes of a row on distinct chunks
  const int SG = L / CL;             // split groups per row (> 1 only with QPL == 1)
  const int sg = sub / CL;
  const bool row_ok = r < R;
  const int rr = row_ok ? r : 0;
  const int row = kRowsPerTile * rt + rr;
  const int h = xg * a.G + row % a.G;
  const float sink = a.use_sink ? sink_log2(a, h) : 0.0f;
  // NC / CL passes, the same number in every lane and wave
  for (int c = cw * NC + sub % CL; c < (cw + 1) * NC; c += CL) {
    float M = -INFINITY, Ls = 0.0f;
    f32x4 acc[QPL];
#pragma unroll
    for (int q = 0; q < QPL; ++q) acc[q] = f32x4{};
    for (int x0 = sg; x0 < nvalid; x0 += SG * NB) {
      float mv[NB], lv[NB];
      f32x4 v[NB][QPL];
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const int xs = min(x0 + e * SG, nvalid - 1);  // clamped: in bounds, ignored below
        const float* p = gpart + (int64_t)xs * PART;
        mv[e] = p[kRowsPerTile * D + rr];
        lv[e] = p[kRowsPerTile * D + kRowsPerTile + rr];
#pragma unroll
        for (int q = 0; q < QPL; ++q) v[e][q] = *reinterpret_cast<const f32x4*>(p + rr * D + 4 * (c * QPL + q));
      }
      // The batch's loads are all in flight before any of them is used: left
      // alone, the compiler sinks them below the branch and issues them one
      // round trip at a time.
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        asm volatile("" ::"v"(mv[e]), "v"(lv[e]));
#pragma unroll
        for (int q = 0; q < QPL; ++q) asm volatile("" ::"v"(v[e][q]));
      }
      float mb = M;
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        if (x0 + e * SG >= nvalid) mv[e] = -INFINITY;
        mb = fmaxf(mb, mv[e]);
      }
      if (mb == -INFINITY) continue;  // nothing seen yet by this lane
      const float fa = fast_exp2(M - mb);  // 0 while M is -inf
      Ls *= fa;
#pragma unroll
      for (int q = 0; q < QPL; ++q) acc[q] *= fa;
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const float f = fast_exp2(mv[e] - mb);  // 0 for empty or ignored splits
        Ls += (mv[e] == -INFINITY ? 0.0f : lv[e]) * f;
#pragma unroll
        for (int q = 0; q < QPL; ++q) acc[q] += v[e][q] * f;
      }
      M = mb;
    }
    // combine the split groups of the row (lanes sub ^ CL, sub ^ 2 CL, ...)
    for (int off = CL; off < L; off <<= 1) {
      const float Mo = __shfl_xor(M, off, 64);
      const float Lo = __shfl_xor(Ls, off, 64);
      float ao[QPL * 4];
#pragma unroll
      for (int q = 0; q < QPL; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) ao[4 * q + e] = __shfl_xor(acc[q][e], off, 64);
      lse_combine<QPL>(M, Ls, acc, Mo, Lo, ao);
    }
    if (row_ok && sg == 0) {
      float fac;
      if (M == -INFINITY) {
        fac = 0.0f;
      } else if (a.use_sink) {
        const float M2 = fmaxf(M, sink);
        const float e1 = fast_exp2(M - M2);
        fac = e1 / (Ls * e1 + fast_exp2(sink - M2));
      } else {
        fac = 1.0f / Ls;
      }
      // an FP8 V cache holds V / v_scale, an INT8 one V / v_scales[g] (1 otherwise)
      fac *= a.v_scales != nullptr ? a.v_scales[xg] : a.v_scale;
#pragma unroll
      for (int q = 0; q < QPL; ++q) store_row4<IS_BF16, D>(a, xb, h, row / a.G, 4 * (c * QPL + q), acc[q] * fac);
    }
  }
}

// Quads per lane for a tile of R rows: the row's lanes (64 / Rp) cover its
// D / 4 output quads once where they can, at most 8 quads per lane.
// The caller has acquired the other workgroups' partials (see the arrivals).
template <bool IS_BF16, int D, int MW>
__device__ __forceinline__ void merge_tile(const AttnArgs& a, int rows, int nrt, int tt,
                                           const float* __restrict__ gpart, int nvalid, int lane, int cw) {
  // the tile's coordinates (no lengths needed here)
  const int bg = tt / nrt, rt = tt - bg * nrt;
  const int xb = bg / a.Hkv, xg = bg - xb * a.Hkv;
  const int R = min(kRowsPerTile, rows - kRowsPerTile * rt);
  const int lrp = R <= 1 ? 0 : (R <= 2 ? 1 : (R <= 4 ? 2 : (R <= 8 ? 3 : 4)));  // log2 of padded rows
  const int qpl = ((D / 4 / MW) << lrp) / 64;  // this wave's quads of a row / lanes of a row
  if (qpl <= 1)
    merge_tile_q<IS_BF16, D, 1, MW>(a, lrp, R, rt, xb, xg, gpart, nvalid, lane, cw);
  else if (qpl == 2)
    merge_tile_q<IS_BF16, D, 2, MW>(a, lrp, R, rt, xb, xg, gpart, nvalid, lane, cw);
  else if (qpl == 4)
    merge_tile_q<IS_BF16, D, 4, MW>(a, lrp, R, rt, xb, xg, gpart, nvalid, lane, cw);
  else
    merge_tile_q<IS_BF16, D, 8, MW>(a, lrp, R, rt, xb, xg, gpart, nvalid, lane, cw);
}

// MASK = 1 / 2: a caller boolean (uint8) / additive (fp32) mask over
// [B, Hq, curr, capacity], the key index being the cache slot.  FUSE: the
// step's append is part of the launch (16-bit caches, no mask); a separate
// instance, so that the other instances keep their code.
template <bool IS_BF16, int D, bool SOFTCAP, int MASK, int KVQ, bool FUSE = false>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a, int rows, int nrt,
                                                     float* __restrict__ part, unsigned* __restrict__ counters) {
  constexpr bool KV8 = KVQ != 0;  // one-byte codes: FP8 (KVQ = 1) or INT8 (KVQ = 2)
  using RG = Ring<D, KV8>;
  using KT = std::conditional_t<KV8, uint8_t, uint16_t>;  // cache element
  constexpr int KQ = D / 32;    // k-steps of 16x16x32 over the head dim
  constexpr int DB = D / 16;    // 16-wide output blocks
  constexpr int S = RG::kStages;
  constexpr int PART = kRowsPerTile * D + 2 * kRowsPerTile;  // floats per partial
  constexpr int MERGE = D / 4 + 2;                            // floats per lane in a merge slot
  // The rings hold the LDS stages while streaming and the wave merge slots
  // between pieces.
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kWaves * RG::kWaveBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds[kRowsPerTile * 2 * D];  // Q tile, swizzled like K
  __shared__ int pre[kMaxTiles + 2];  // unit prefix sum over tiles (then workgroups per tile)
  __shared__ int wsum[4];
  __shared__ int split_s[5];  // U, Gs, slice start and end, first tile (T <= 64)
  __shared__ int flag[256];
  // (q_off, valid, lo, hi) of each tile, kept by the setup when there are
  // few tiles, so that starting a piece needs no memory round trip
  __shared__ int4 tcache[kCachedTiles];
  float (*merge_lds)[MERGE * 64] = reinterpret_cast<float (*)[MERGE * 64]>(&ring[0]);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 15;
  const int q4 = lane >> 4;
  const int G = gridDim.x;
  // The slice this workgroup streams.  Workgroups are dispatched to the 8
  // XCDs in turn (workgroup b on XCD b mod 8), and a row tile's slices are
  // consecutive: numbering the slices XCD-major puts each tile's
  // contributors, its partials and its merge on one XCD (bitwise the same
  // result; the fused step measured 0.1-0.65 us faster, the rest unchanged).
  const int k = G % 8 == 0 ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int T = a.B * a.Hkv * nrt;

  // ---- the step's append, fused: new row t of (b, g) into the cache slot of
  // position total_b - curr + t (mod the ring), with the skip rule of the
  // append kernel.  Its 16-byte chunks are spread over the whole grid, a few
  // threads of waves 1-3 per workgroup.  Nobody reads these slots in this
  // launch. ----
  constexpr int kAppendChunks = D / 8;
  const int ap_items = FUSE ? a.B * a.Hkv * a.Lq * kAppendChunks : 0;
  u32x4 ap_k = u32x4{}, ap_v = u32x4{};
  auto ap_coords = [&](int i, int& b, int& g, int& t, int& c) {
    c = i % kAppendChunks;
    int r = i / kAppendChunks;
    t = r % a.Lq;
    r /= a.Lq;
    g = r % a.Hkv;
    b = r / a.Hkv;
  };
  auto ap_load = [&](int i, u32x4& kx, u32x4& vx) {
    int b, g, t, c;
    ap_coords(i, b, g, t, c);
    kx = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.k_new) + b * a.kn_sb + g * a.kn_sh +
                                         (int64_t)t * a.kn_ss + 8 * c);
    vx = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.v_new) + b * a.vn_sb + g * a.vn_sh +
                                         (int64_t)t * a.vn_ss + 8 * c);
  };
  auto ap_store = [&](int i, const u32x4& kx, const u32x4& vx) {
    int b, g, t, c;
    ap_coords(i, b, g, t, c);
    const int64_t total = (int64_t)a.seqlens[b] + 1;
    if (total < a.Lq || (!a.ring && total > a.Lk)) return;
    int64_t slot = total - a.Lq + t;
    if (a.ring) slot %= a.ring;
    uint16_t* kc = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.k));
    uint16_t* vc = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.v));
    *reinterpret_cast<u32x4*>(kc + b * a.k_sb + g * a.k_sh + slot * a.k_ss + 8 * c) = kx;
    *reinterpret_cast<u32x4*>(vc + b * a.v_sb + g * a.v_sh + slot * a.v_ss + 8 * c) = vx;
  };
  // Waves 1-3 do the whole append at the start, while wave 0 alone
  // computes the split below: nothing in the append waits for the split,
  // and wave 0's path to the first K/V request stays free of it.
  if constexpr (FUSE) {
    if (w > 0) {
      for (int i = k + G * (tid - 64); i < ap_items; i += G * (256 - 64)) {
        ap_load(i, ap_k, ap_v);
        ap_store(i, ap_k, ap_v);
      }
    }
  }

  // ---- the split of the work (the same in every workgroup) ----
  // Exclusive prefix sum of f(t) over the row tiles into out[0..T].
  auto block_scan = [&](int* out, auto f) {
    int carry = 0;
    if (tid == 0) out[0] = 0;
    for (int base = 0; base < T; base += 256) {
      const int t = base + tid;
      const int incl = wave_incl_scan(t < T ? f(t) : 0, lane);
      if (lane == 63) wsum[w] = incl;
      __syncthreads();
      int before = carry;
      for (int x = 0; x < w; ++x) before += wsum[x];
      if (t < T) out[t + 1] = before + incl;
      carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
      __syncthreads();
    }
  };
  const bool cached = T <= kCachedTiles;
  // Slices.  With at least two workgroups per row tile, tile t gets
  // n_t = ceil(u_t / L) workgroups of its own (u_t its units, L the smallest
  // load for which they fit the grid) and its units are cut evenly among them:
  // no slice crosses a tile boundary, where a workgroup's stream would drain
  // and restart.  Otherwise workgroup k < Gs streams units
  // [floor(U k / Gs), floor(U (k+1) / Gs)) of the tiles' concatenation.
  // Either way no slice is empty and the workgroups holding a tile's units
  // are consecutive.
  const bool aligned = 2 * T <= G;
  int* const pren = pre + T + 1;  // aligned: prefix sum of n_t (2T + 2 <= kMaxTiles + 2 entries)
  int U, Gs, ustart, uend, t_first;
  if (T <= 64) {
    // One tile per lane of wave 0, which computes the whole split in
    // registers (no LDS round trips, no barriers inside) and publishes it;
    // the other waves wait at one barrier.  The split is integer work on
    // the scalar unit, which all waves of a CU share: when every wave
    // computed it, the first K/V request came ~1.5 us later.
    if (w == 0) {
      Tile x{};
      int ut = 0;
      if (lane < T) {
        x = make_tile(a, rows, nrt, lane, MASK != 0);
        ut = units_of(x);
      }
      const int incl = wave_incl_scan(ut, lane);
      const int u_all = __builtin_amdgcn_readlane(incl, 63);
      const int pre_l = incl - ut;  // pre[lane]
      if (lane == 0) pre[0] = 0;
      if (lane < T) {
        pre[lane + 1] = incl;
        if (cached) tcache[lane] = int4{x.sp.q_off, x.sp.valid, x.lo, x.hi};
      }
      int g_used, us = 0, ue = 0, tf = 0;
      if (aligned) {
        // L = ceil(U / (G - T)) always fits, since sum_t ceil(u_t / L) < U / L + T
        int lo = max(1, (u_all + G - 1) / G), hi = max(1, (u_all + (G - T) - 1) / (G - T));
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (wave_sum((ut + mid - 1) / mid, lane) <= G) hi = mid; else lo = mid + 1;  // 0 past the last tile
        }
        const int nt = (ut + lo - 1) / lo;
        const int nincl = wave_incl_scan(nt, lane);
        const int pren_l = nincl - nt;  // pren[lane]
        g_used = __builtin_amdgcn_readlane(nincl, 63);
        if (lane == 0) pren[0] = 0;
        if (lane < T) pren[lane + 1] = nincl;  // read by the arrivals at the end
        if (k < g_used) {
          // the largest t with pren[t] <= k (a prefix of the lanes; never an empty tile)
          tf = 63 - __builtin_clzll(__ballot(lane < T && pren_l <= k));
          const int u_t = __builtin_amdgcn_readlane(ut, tf);
          const int p_t = __builtin_amdgcn_readlane(pre_l, tf);
          const int n_t = __builtin_amdgcn_readlane(nt, tf);
          const int i = k - __builtin_amdgcn_readlane(pren_l, tf);
          us = p_t + mul_div(u_t, i, n_t);
          ue = p_t + mul_div(u_t, i + 1, n_t);
        }
      } else {
        g_used = min(G, u_all);
        if (k < g_used) {
          us = mul_div(u_all, k, g_used);
          ue = mul_div(u_all, k + 1, g_used);
          // first tile holding unit us: the largest t with pre[t] <= us
          tf = 63 - __builtin_clzll(__ballot(lane < T && pre_l <= us));
        }
      }
      if (lane == 0) {
        split_s[0] = u_all;
        split_s[1] = g_used;
        split_s[2] = us;
        split_s[3] = ue;
        split_s[4] = tf;
      }
    }
    __syncthreads();
    U = split_s[0];
    Gs = split_s[1];
    ustart = split_s[2];
    uend = split_s[3];
    t_first = split_s[4];
  } else {
    block_scan(pre, [&](int t) {
      const Tile x = make_tile(a, rows, nrt, t, MASK != 0);
      if (cached) tcache[t] = int4{x.sp.q_off, x.sp.valid, x.lo, x.hi};
      return units_of(x);
    });
    U = pre[T];
    if (aligned) {
      // L = ceil(U / (G - T)) always fits, since sum_t ceil(u_t / L) < U / L + T
      int lo = max(1, (U + G - 1) / G), hi = max(1, (U + (G - T) - 1) / (G - T));
      // every wave runs the search on its own (same result, no barriers)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        int c = 0;
        for (int t = lane; t < T; t += 64) c += (pre[t + 1] - pre[t] + mid - 1) / mid;
        if (wave_sum(c, lane) <= G) hi = mid; else lo = mid + 1;
      }
      const int L = lo;
      block_scan(pren, [&](int t) { return (pre[t + 1] - pre[t] + L - 1) / L; });
      Gs = pren[T];
      ustart = uend = t_first = 0;
      if (k < Gs) {
        int lo2 = 0, hi2 = T;  // invariant: pren[lo2] <= k < pren[hi2]
        while (hi2 - lo2 > 1) {
          const int mid = (lo2 + hi2) >> 1;
          if (pren[mid] <= k) lo2 = mid; else hi2 = mid;
        }
        t_first = lo2;
        const int ut = pre[lo2 + 1] - pre[lo2];
        const int n = pren[lo2 + 1] - pren[lo2], i = k - pren[lo2];
        ustart = pre[lo2] + mul_div(ut, i, n);
        uend = pre[lo2] + mul_div(ut, i + 1, n);
      }
    } else {
      Gs = min(G, U);
      ustart = uend = t_first = 0;
      if (k < Gs) {
        ustart = mul_div(U, k, Gs);
        uend = mul_div(U, k + 1, Gs);
        // first tile holding unit ustart: the largest t with pre[t] <= ustart
        int lo2 = 0, hi2 = T;  // invariant: pre[lo2] <= ustart < pre[hi2]
        while (hi2 - lo2 > 1) {
          const int mid = (lo2 + hi2) >> 1;
          if (pre[mid] <= ustart) lo2 = mid; else hi2 = mid;
        }
        t_first = lo2;
      }
    }
  }

  // tiles nobody streams (no allowed key for any of their rows) output zeros
  for (int t = k; t < T; t += G) {
    if (pre[t + 1] != pre[t]) continue;
    const Tile x = make_tile(a, rows, nrt, t, MASK != 0);
    for (int idx = tid; idx < x.rows_tile * (D / 4); idx += 256) {
      const int row = kRowsPerTile * x.rt + idx / (D / 4);
      store_row4<IS_BF16, D>(a, x.b, x.g * a.G + row % a.G, row / a.G, 4 * (idx % (D / 4)), f32x4{});
    }
  }
  if (k >= Gs) return;
  // workgroups first .. first + nvalid - 1 hold the units of (non-empty) tile t
  auto contributors = [&](int t, int& first, int& nvalid) {
    if (aligned) {
      first = pren[t];
      nvalid = pren[t + 1] - pren[t];
    } else {
      first = owner_of(pre[t], U, Gs);
      nvalid = owner_of(pre[t + 1] - 1, U, Gs) - first + 1;
    }
  };
  int t_last = t_first - 1;  // last tile this workgroup touches

  const float c_l2 = SOFTCAP ? 1.0f : a.scale_log2;
  unsigned char* const my_ring = ring + w * RG::kWaveBytes;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)(lds_void*)my_ring;  // LDS byte address
  const uint32_t q_addr = (uint32_t)(uintptr_t)(lds_void*)q_lds;
  // Per-lane LDS read offsets, the same for every unit.  K (and Q) operand:
  // row n, chunk 4 ks + q4.  V^T operand (transposing read): rows
  // 4 q4 + (n >> 2), columns 16 db + 4 (n & 3) .. + 3.
  uint32_t k_off[KQ], v_off[DB];
#pragma unroll
  for (int ks = 0; ks < KQ; ++ks) k_off[ks] = n * RG::kRowBytes + 16 * ((4 * ks + q4) ^ swz<D>(n));
  {
    const int v_key = 4 * q4 + (n >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_off[db] = RG::kUnitBytes + v_key * RG::kRowBytes + 16 * ((2 * db + ((n >> 1) & 1)) ^ swz<D>(v_key)) +
                  8 * (n & 1);
  }

  // ---- stream the slice, one piece (slice x tile) at a time ----
  int u = ustart;
  int t = t_first;
  while (u < uend) {
    while (pre[t + 1] <= u) ++t;  // skip tiles without units
    const int ua = u - pre[t];
    const int ub = min(uend, pre[t + 1]) - pre[t];
    u = pre[t] + ub;
    t_last = t;
    Tile x;
    if (cached) {
      // the same values make_tile computes, without loading the lengths again
      const int4 c = tcache[t];
      x.bg = t / nrt;
      x.rt = t - x.bg * nrt;
      x.b = x.bg / a.Hkv;
      x.g = x.bg - x.b * a.Hkv;
      x.sp.q_off = c.x;
      x.sp.valid = c.y;
      x.lo = c.z;
      x.hi = c.w;
      x.rows_tile = min(kRowsPerTile, rows - kRowsPerTile * x.rt);
    } else {
      x = make_tile(a, rows, nrt, t, MASK != 0);
    }
    // the piece's key range (wave-uniform: scalar registers)
    const int c_lo = __builtin_amdgcn_readfirstlane(x.lo + kSub * ua);
    const int c_hi = __builtin_amdgcn_readfirstlane(min(x.hi, x.lo + kSub * ub - 1));
    // INT8 caches: the KV head's K scale joins the softmax scale (raw scores
    // are in code units)
    const float kq = KVQ == 2 ? a.k_scales[x.g] : 1.0f;
    const float c_l2p = SOFTCAP ? 1.0f : c_l2 * kq;
    const float soc = a.scale_over_cap * kq;
    // an additive mask value in this head's code-score units
    const float bmul = KVQ == 2 ? a.bias_mul / kq : a.bias_mul;

    // this lane's query row (padding rows carry zeros and are never stored)
    const int my_r = kRowsPerTile * x.rt + n;
    const bool row_ok = n < x.rows_tile;
    const int my_t = row_ok ? my_r / a.G : 0;
    const int my_p = x.sp.q_off + my_t;
    const int lo_eff = max(row_lo(a, my_p), c_lo);
    const int hi_eff = min(row_hi(a, my_p, x.sp.valid), c_hi);
    const int p_first = x.sp.q_off + (kRowsPerTile * x.rt) / a.G;
    const int p_last = x.sp.q_off + (kRowsPerTile * x.rt + x.rows_tile - 1) / a.G;

    const KT* __restrict__ Kg = reinterpret_cast<const KT*>(a.k) + x.b * a.k_sb + x.g * a.k_sh;
    const KT* __restrict__ Vg = reinterpret_cast<const KT*>(a.v) + x.b * a.v_sb + x.g * a.v_sh;
    // with the append fused in, positions new_lo .. valid - 1 come from the
    // step's new rows
    const KT* __restrict__ Kn = reinterpret_cast<const KT*>(a.k_new) + x.b * a.kn_sb + x.g * a.kn_sh;
    const KT* __restrict__ Vn = reinterpret_cast<const KT*>(a.v_new) + x.b * a.vn_sb + x.g * a.vn_sh;
    const int new_lo = __builtin_amdgcn_readfirstlane(x.sp.valid - a.Lq);

    // Q tile -> LDS by DMA, shared by the 4 waves (instruction i by wave i % 4).
    // Padding rows load the tile's last real row (in bounds, finite); MFMA
    // columns are independent, so they only produce unused output rows.
    constexpr int QDMA = kRowsPerTile * 2 * D / 1024;
#pragma unroll
    for (int i = 0; i < QDMA; ++i) {
      if (i % kWaves != w) continue;
      const int pos = 64 * i + lane;
      const int r = pos / RG::kSlots;
      const int cc = (pos % RG::kSlots) ^ swz<D>(r);
      const int qr = kRowsPerTile * x.rt + min(r, x.rows_tile - 1);
      const uint16_t* src = reinterpret_cast<const uint16_t*>(a.q) + x.b * a.q_sb +
                            (x.g * a.G + qr % a.G) * a.q_sh + (int64_t)(qr / a.G) * a.q_ss + 8 * cc;
      __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)(q_lds + 1024 * i), 16, 0, 0);
    }

    // units of this wave: ua + w, ua + w + 4, ...
    const int nw = ub - ua > w ? (ub - ua - w + 3) / 4 : 0;
    // A rolling cache keeps position j in slot j mod ring.  The piece spans
    // fewer than `ring` positions (the host checks capacity >= W + curr - 1),
    // so after removing the whole turns before c_lo one conditional wrap maps
    // every key.  Caches that are not rings take the plain addresses (a
    // wave-uniform branch per unit).
    const int turns = a.ring ? c_lo - c_lo % a.ring : 0;
    // A unit whose 16 rows are consecutive cache rows (the usual case) is
    // loaded from a scalar base, its first row, plus a per-lane 32-bit offset
    // built from full-rate integer operations: lane chunk 64 i + lane is row
    // kRowsDma i + lr, chunk lc (swizzled on 16-bit caches).  With row
    // strides below 2^24 elements every such offset fits 32 bits (at most 16
    // rows of 2^25 bytes); larger strides take the per-lane path.  Per-lane
    // 64-bit row addresses cost six quarter-rate multiplies per K/V load
    // pair.
    constexpr int kChunksDma = KV8 ? D / 16 : RG::kSlots;  // 16-byte chunks per streamed row
    constexpr int kRowsDma = 64 / kChunksDma;               // rows per wave-wide load
    const int lr = lane / kChunksDma, lc = lane % kChunksDma;
    const uint32_t rbk = (uint32_t)a.k_ss * (uint32_t)sizeof(KT);
    const uint32_t rbv = (uint32_t)a.v_ss * (uint32_t)sizeof(KT);
    const uint32_t lane_k = (uint32_t)lr * rbk, lane_v = (uint32_t)lr * rbv;
    const bool small_strides = a.k_ss < (int64_t(1) << 24) && a.v_ss < (int64_t(1) << 24);
    // Other units (the piece ends inside them, they reach the step's new
    // rows, or they wrap around a rolling cache) take per-lane row
    // addresses; rows past the piece end are clamped to its last key (a real
    // key, finite, masked out for every query row): no per-lane branches.
    auto issue_t = [&](int s, int j, auto ring_tag, auto fuse_tag) {
      const int kb = c_lo + kSub * (w + 4 * j);
      unsigned char* kdst = my_ring + s * 2 * RG::kInBytes;
      unsigned char* vdst = kdst + RG::kInBytes;
      int s0 = kb;  // the slot of the unit's first row
      bool whole = small_strides && kb + kSub - 1 <= c_hi;
      if constexpr (decltype(fuse_tag)::value) whole = whole && kb + kSub - 1 < new_lo;
      if constexpr (decltype(ring_tag)::value) {
        s0 -= turns;
        s0 = s0 >= a.ring ? s0 - a.ring : s0;
        whole = whole && s0 + kSub - 1 < a.ring;
      }
      // (not in the fused step at head size 256, whose registers are full:
      // the extra path spills it)
      constexpr bool kWholeUnits = !(FUSE && D >= 256);
      if (kWholeUnits && whole) {
        const char* kbase = reinterpret_cast<const char*>(Kg + (int64_t)s0 * a.k_ss);
        const char* vbase = reinterpret_cast<const char*>(Vg + (int64_t)s0 * a.v_ss);
        // the offsets are rebuilt per unit (a few full-rate operations):
        // hoisted out of the loop they would hold 4 * kDmaPerUnit registers
        uint32_t lk = lane_k, lv = lane_v;
        asm volatile("" : "+v"(lk), "+v"(lv));
#pragma unroll
        for (int i = 0; i < RG::kDmaPerUnit; ++i) {
          const uint32_t c16 = 16u * (uint32_t)(KV8 ? lc : lc ^ swz<D>(kRowsDma * i + lr));
          __builtin_amdgcn_global_load_lds(
              (global_void*)(kbase + (size_t)((uint32_t)(kRowsDma * i) * rbk) + (size_t)(lk + c16)),
              (lds_void*)(kdst + 1024 * i), 16, 0, kNonTemporal);
          __builtin_amdgcn_global_load_lds(
              (global_void*)(vbase + (size_t)((uint32_t)(kRowsDma * i) * rbv) + (size_t)(lv + c16)),
              (lds_void*)(vdst + 1024 * i), 16, 0, kNonTemporal);
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < RG::kDmaPerUnit; ++i) {
        const int pos = 64 * i + lane;                 // 16-byte chunk position in the unit
        // 16-bit caches: swizzled chunks (global chunk cc of key row `key`);
        // fp8 caches: row-major (byte offset 16 pos = key * D + 16 cc)
        const int key = KV8 ? pos / (D / 16) : pos / RG::kSlots;
        const int cc = KV8 ? pos % (D / 16) : (pos % RG::kSlots) ^ swz<D>(key);
        int row = min(kb + key, c_hi);
        constexpr int kEl = KV8 ? 16 : 8;  // elements per 16-byte chunk
        const KT* ks;
        const KT* vs;
        if constexpr (decltype(fuse_tag)::value) {
          // this step's own rows come from k_new / v_new
          const bool nw_row = row >= new_lo;
          int slot = row;
          if constexpr (decltype(ring_tag)::value) {
            slot -= turns;
            slot = slot >= a.ring ? slot - a.ring : slot;
          }
          ks = nw_row ? Kn + (int64_t)(row - new_lo) * a.kn_ss : Kg + (int64_t)slot * a.k_ss;
          vs = nw_row ? Vn + (int64_t)(row - new_lo) * a.vn_ss : Vg + (int64_t)slot * a.v_ss;
        } else {
          if constexpr (decltype(ring_tag)::value) {
            row -= turns;
            row = row >= a.ring ? row - a.ring : row;
          }
          ks = Kg + (int64_t)row * a.k_ss;
          vs = Vg + (int64_t)row * a.v_ss;
        }
        // K/V bytes are read once per call: non-temporal (streaming) loads
        __builtin_amdgcn_global_load_lds((global_void*)(ks + kEl * cc), (lds_void*)(kdst + 1024 * i), 16, 0,
                                         kNonTemporal);
        __builtin_amdgcn_global_load_lds((global_void*)(vs + kEl * cc), (lds_void*)(vdst + 1024 * i), 16, 0,
                                         kNonTemporal);
      }
    };
    auto issue = [&](int s, int j) {
      if constexpr (FUSE) {
        if (a.ring)
          issue_t(s, j, std::true_type{}, std::true_type{});
        else
          issue_t(s, j, std::false_type{}, std::true_type{});
        return;
      }
      if (a.ring) {
        issue_t(s, j, std::true_type{}, std::false_type{});
      } else {
        issue_t(s, j, std::false_type{}, std::false_type{});
      }
    };
    const int npro = min(nw, S);
    for (int j = 0; j < npro; ++j) issue(j, j);
    // Q landed once only the prologue units are younger; then every wave's
    // part is in LDS after the barrier (no fence: nothing else to order).
    wait_vm_multiple<2 * RG::kDmaPerUnit, S>(npro);
    __builtin_amdgcn_s_barrier();
    u32x4 qf[KQ];
#pragma unroll
    for (int ks = 0; ks < KQ; ks += 2)
      lds_read2_b128(qf[ks], qf[ks + 1], q_addr + k_off[ks], q_addr + k_off[ks + 1]);

    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.0f;

    // Caller mask: this lane's row (padding rows read the tile's first row)
    // and, per unit, its keys kb + 4 q4 .. + 3 -- one aligned 4-byte (boolean)
    // or 16-byte (additive) load, a unit ahead; entries past the capacity are
    // read one by one.  The loads are younger than the unit's DMA, so the
    // counted waits below only grow stronger.
    uint32_t mb_cur = 0, mb_nxt = 0;
    f32x4 mf_cur = f32x4{}, mf_nxt = f32x4{};
    const char* mrow = nullptr;
    if constexpr (MASK != 0) {
      const int mr = kRowsPerTile * x.rt + (row_ok ? n : 0);
      mrow = reinterpret_cast<const char*>(a.mask) +
             (MASK == 1 ? 1 : 4) * (x.b * a.m_sb + (int64_t)(x.g * a.G + mr % a.G) * a.m_sh +
                                    (int64_t)(mr / a.G) * a.m_sq);
    }
    auto mask_load = [&](int kb) {
      const int k0 = kb + 4 * q4;
      if constexpr (MASK == 1) {
        if (k0 + 3 < a.Lk) {
          mb_nxt = *(const __attribute__((address_space(1))) uint32_t*)(mrow + k0);
        } else {
          uint32_t v = 0;
          for (int e = 0; e < 4; ++e)
            if (k0 + e < a.Lk) v |= (uint32_t)(*(const __attribute__((address_space(1))) uint8_t*)(mrow + k0 + e)) << (8 * e);
          mb_nxt = v;
        }
      } else if constexpr (MASK == 2) {
        const auto* fp = (const __attribute__((address_space(1))) float*)mrow;
        if (k0 + 3 < a.Lk) {
          mf_nxt = *(const __attribute__((address_space(1))) f32x4*)(fp + k0);
        } else {
          for (int e = 0; e < 4; ++e) mf_nxt[e] = k0 + e < a.Lk ? fp[k0 + e] : 0.0f;
        }
      }
    };
    if constexpr (MASK != 0)
      if (nw > 0) mask_load(c_lo + kSub * w);

    for (int j = 0; j < nw; ++j) {
      const int s = j % S;
      wait_units<2 * RG::kDmaPerUnit, S>(min(S - 1, nw - 1 - j));
      const int kb = c_lo + kSub * (w + 4 * j);
      if constexpr (MASK == 1) mb_cur = mb_nxt;
      if constexpr (MASK == 2) mf_cur = mf_nxt;
      if constexpr (MASK != 0)
        if (j + 1 < nw) mask_load(kb + 4 * kSub);
      if constexpr (KV8) {
        // one-byte stage -> the 16-bit K + V buffer, in the layout of the
        // 16-bit path (bf16 / fp16 chunk g of key row r at slot g ^ swz(r));
        // every E4M3 and every INT8 code is exact in both types.  The stage's
        // bytes are read into registers first.  INT8 codes take three
        // instructions per pair to convert, so their stage is refilled before
        // the conversion runs (measured: 2 us faster at head size 256); FP8
        // codes, one instruction per pair, refill after it (0.3 us faster at
        // head size 128).
        constexpr bool kEarlyRefill = KVQ == 2;
        const unsigned char* s8 = my_ring + s * 2 * RG::kInBytes;
        unsigned char* bb = my_ring + RG::kBufOff;
        u32x4 raw[2][RG::kDmaPerUnit];
#pragma unroll
        for (int tsr = 0; tsr < 2; ++tsr)
#pragma unroll
          for (int i = 0; i < RG::kDmaPerUnit; ++i)
            raw[tsr][i] = *reinterpret_cast<const u32x4*>(s8 + tsr * RG::kInBytes + 16 * (64 * i + lane));
        if constexpr (kEarlyRefill) {
          // every read has returned before the refill may overwrite the stage
#pragma unroll
          for (int tsr = 0; tsr < 2; ++tsr)
#pragma unroll
            for (int i = 0; i < RG::kDmaPerUnit; ++i) asm volatile("" ::"v"(raw[tsr][i]));
          asm volatile("" ::: "memory");
          if (j + S < nw) issue(s, j + S);
        }
#pragma unroll
        for (int tsr = 0; tsr < 2; ++tsr)
#pragma unroll
          for (int i = 0; i < RG::kDmaPerUnit; ++i) {
            const int pos = 64 * i + lane;
            const int key = pos / (D / 16), c = pos % (D / 16);
            uint32_t hw[8];  // two 16-bit values per word, byte order kept
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t cw = raw[tsr][i][q];
              if constexpr (KVQ == 2) {
                // INT8 codes (|c| <= 127) are exact in bf16 and fp16
                hw[2 * q] = pack2<IS_BF16>((float)(int8_t)(cw & 0xffu), (float)(int8_t)((cw >> 8) & 0xffu));
                hw[2 * q + 1] = pack2<IS_BF16>((float)(int8_t)((cw >> 16) & 0xffu), (float)(int8_t)(cw >> 24));
              } else if constexpr (IS_BF16) {
                hw[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw, 1.0f, false));
                hw[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw, 1.0f, true));
              } else {
                hw[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw, 1.0f, false));
                hw[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw, 1.0f, true));
              }
            }
            unsigned char* rowp = bb + tsr * RG::kUnitBytes + key * RG::kRowBytes;
            *reinterpret_cast<u32x4*>(rowp + 16 * ((2 * c) ^ swz<D>(key))) = u32x4{hw[0], hw[1], hw[2], hw[3]};
            *reinterpret_cast<u32x4*>(rowp + 16 * ((2 * c + 1) ^ swz<D>(key))) = u32x4{hw[4], hw[5], hw[6], hw[7]};
          }
        // A wave's LDS operations complete in order, so the counted waits of
        // the operand reads below also cover these writes; the stage's reads
        // have returned (their values are converted above) before a late
        // refill.
        if constexpr (!kEarlyRefill) {
          asm volatile("" ::: "memory");
          if (j + S < nw) issue(s, j + S);
        }
      }
      const uint32_t st = KV8 ? ring_addr + RG::kBufOff : ring_addr + s * 2 * RG::kUnitBytes;
      // S^T = K Q^T
      u32x4 kf[KQ];
#pragma unroll
      for (int ks = 0; ks < KQ; ks += 2) lds_read2_b128(kf[ks], kf[ks + 1], st + k_off[ks], st + k_off[ks + 1]);
      f32x4 sc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) sc = mma_qk<IS_BF16>(kf[ks], qf[ks], sc);
      if constexpr (SOFTCAP) {  // an additive mask value enters the cap with the logit
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sc[r];
          if constexpr (MASK == 2) x = fmaf(mf_cur[r], bmul, x);
          sc[r] = a.cap_log2 * tanh_fast(x * soc);
        }
      }
      const bool interior = (a.window < 0 || kb >= p_last - a.window + 1) &&
                            (!a.causal || kb + kSub - 1 <= p_first) && (kb + kSub - 1 <= c_hi);
      if (!interior) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j2 = kb + 4 * q4 + r;
          sc[r] = (j2 < lo_eff || j2 > hi_eff) ? -INFINITY : sc[r];
        }
      }
      if constexpr (MASK == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = ((mb_cur >> (8 * r)) & 0xffu) ? sc[r] : -INFINITY;
      }
      if constexpr (MASK == 2) {  // -inf (or NaN) removes the key
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sc[r] = mf_cur[r] > -INFINITY ? (SOFTCAP ? sc[r] : fmaf(mf_cur[r], bmul, sc[r])) : -INFINITY;
      }
      // online softmax: lanes n, n+16, n+32, n+48 share row n
      float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bm = fmaxf(bm, xor16(bm));
      bm = fmaxf(bm, xor32(bm));
      const float m_new = fmaxf(m_run, bm);
      const bool need = (m_new - m_run) * c_l2p > kRescaleLog2;
      if (__any(need)) {
        const float alpha = need ? fast_exp2((m_run - m_new) * c_l2p) : 1.0f;
        m_run = need ? m_new : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
      }
      const float mb = m_run == -INFINITY ? 0.0f : m_run * c_l2p;
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = fast_exp2(fmaf(sc[r], c_l2p, -mb));
        l_run += pv[r];
      }
      const u32x2 pp = u32x2{pack2<IS_BF16>(pv[0], pv[1]), pack2<IS_BF16>(pv[2], pv[3])};
      // O^T += V^T P^T, V^T read transposed out of the row-major stage
      u32x2 vf[DB];
#pragma unroll
      for (int db = 0; db < DB; db += 4)
        lds_read4_tr16(vf[db], vf[db + 1], vf[db + 2], vf[db + 3], st + v_off[db], st + v_off[db + 1],
                       st + v_off[db + 2], st + v_off[db + 3]);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mma_pv<IS_BF16>(vf[db], pp, o[db]);
      // refill this stage (its LDS reads are consumed above)
      if constexpr (!KV8)
        if (j + S < nw) issue(s, j + S);
    }

    // ---- merge the 4 waves through LDS (lane-to-lane: identical layouts) ----
    // Every wave writes its state to its slot (accumulators as one 16-byte
    // entry per lane and output block, then m and l); after one barrier,
    // wave w merges the four states of output blocks [w DB/4, (w+1) DB/4)
    // and stores them to the partial, and wave 0 also stores the rows'
    // maxima and sums.  (A tree of two halving steps put three barriers and
    // four serial LDS passes between the last unit and the stores.)
    static_assert(kWaves * MERGE * 64 * 4 <= kWaves * RG::kWaveBytes, "merge slots fit the rings");
    static_assert(DB % kWaves == 0, "whole output blocks per wave");
    constexpr int DBW = DB / kWaves;
    __syncthreads();  // every wave's last unit is consumed: the rings are free
    {
      float* ml = merge_lds[w];
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(ml + 4 * (db * 64 + lane)) = o[db];
      ml[(D / 4) * 64 + lane] = m_run;
      ml[(D / 4 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    {
      float mv[kWaves], lv[kWaves];
      float M = -INFINITY;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        mv[i] = merge_lds[i][(D / 4) * 64 + lane];
        lv[i] = merge_lds[i][(D / 4 + 1) * 64 + lane];
        M = fmaxf(M, mv[i]);
      }
      float f[kWaves];
      float l_m = 0.0f;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        f[i] = mv[i] == -INFINITY ? 0.0f : fast_exp2((mv[i] - M) * c_l2p);  // 0 for an empty state
        l_m += lv[i] * f[i];
      }
      f32x4 om[DBW];
#pragma unroll
      for (int q = 0; q < DBW; ++q) {
        const int db = DBW * w + q;
        om[q] = f32x4{};
#pragma unroll
        for (int i = 0; i < kWaves; ++i)
          om[q] += *reinterpret_cast<const f32x4*>(merge_lds[i] + 4 * (db * 64 + lane)) * f[i];
      }
      float l_row = l_m + xor16(l_m);
      l_row += xor32(l_row);
      if (row_ok) {
        float* p = part + (int64_t)(k + t) * PART;  // slot k + t: unique per piece
        const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(p, 0, PART * 4, kRawBufferWord3);
#pragma unroll
        for (int q = 0; q < DBW; ++q) coherent_store4(pr, 4 * (n * D + 16 * (DBW * w + q) + 4 * q4), om[q]);
        if (w == 0 && q4 == 0) {
          coherent_store(p + kRowsPerTile * D + n, M == -INFINITY ? -INFINITY : M * c_l2p);
          coherent_store(p + kRowsPerTile * D + kRowsPerTile + n, l_row);
        }
      }
    }
    __syncthreads();  // the merge slots are ring stages again for the next piece
    ++t;
  }

  // ---- arrivals: the last workgroup to finish a tile merges its partials ----
  // Every writer waits until its write-through stores have completed
  // (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int base = t_first; base <= t_last; base += 256) {
    // one arrival per touched tile, all in flight together
    const int nbt = min(256, t_last - base + 1);
    if (tid < nbt) {
      const int tt = base + tid;
      int f = 0;
      if (pre[tt + 1] != pre[tt]) {
        int first, nvalid;
        contributors(tt, first, nvalid);
        f = __hip_atomic_fetch_add(&counters[tt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            (unsigned)(nvalid - 1);
      }
      flag[tid] = f;
    }
    __syncthreads();
    // The other workgroups' device-scope stores were complete before their
    // arrivals, which this workgroup has seen; a merging wave acquires them
    // (an L2 invalidate) before it reads.  Below head size 256 each tile
    // this workgroup completed goes to one wave, in turn, so that merges run
    // side by side.  At head size 256 (partials of 16.5 KB, one workgroup
    // per CU) every wave merges a quarter of the columns of each tile: wave
    // 0 acquires once and the barrier orders the other waves' loads after
    // it (an acquire per wave measured slower than one wave per tile; at
    // head size 128 the split merge is ~1 us slower, at 256 ~1.8 us faster).
    constexpr int MW = D >= 256 ? kWaves : 1;
    if constexpr (MW > 1) {
      bool any = false;
      for (int c0 = 0; c0 < nbt; c0 += 64) any |= __ballot(c0 + lane < nbt && flag[c0 + lane]) != 0;
      if (any) {  // the same in every wave (flag[] is shared)
        if (w == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
      }
    }
    int cnt = 0;
    for (int c0 = 0; c0 < nbt; c0 += 64) {
      uint64_t mask = __ballot(c0 + lane < nbt && flag[c0 + lane]);
      while (mask) {
        const int i = c0 + __builtin_ctzll(mask);
        mask &= mask - 1;
        if (MW == 1 && cnt++ % kWaves != w) continue;
        const int tt = base + i;
        int first, nvalid;
        contributors(tt, first, nvalid);
        nvalid = min(nvalid, Gs - first);  // never past the slots this call wrote
        if constexpr (MW == 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        merge_tile<IS_BF16, D, MW>(a, rows, nrt, tt, part + (int64_t)(first + tt) * PART, nvalid, lane,
                                   MW == 1 ? 0 : w);
        if ((MW == 1 || w == 0) && lane == 0)  // ready for the next call
          __hip_atomic_store(&counters[tt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // flag[] is rewritten by the next batch of tiles
  }
}

// Workgroups that fit on the device at once for one kernel instance.
template <typename K>
int resident_grid(K kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return std::max(1, std::min(kMaxGrid, cus * per_cu));
}

// The grid of one kernel instance on the current device (computed once per
// device; a benign race computes the same value).
template <bool IS_BF16, int D, bool SOFTCAP, int MASK, int KVQ, bool FUSE>
int grid_of() {
  static int grid_cache[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  int G = grid_cache[dev];
  if (G == 0) G = grid_cache[dev] = resident_grid(decode_kernel<IS_BF16, D, SOFTCAP, MASK, KVQ, FUSE>);
  return G;
}

// The instance a call runs on, as compile-time arguments of op.run<...>().
template <bool IS_BF16, int D, typename Op>
auto visit_d(const AttnArgs& a, bool softcap, const Op& op) {
  if (a.fuse_append)  // 16-bit caches, no mask (the host guarantees both)
    return softcap ? op.template run<IS_BF16, D, true, 0, 0, true>()
                   : op.template run<IS_BF16, D, false, 0, 0, true>();
  if (a.kv_fp8 == 2) {  // INT8 caches
    if (a.mask_kind == 1)
      return softcap ? op.template run<IS_BF16, D, true, 1, 2>() : op.template run<IS_BF16, D, false, 1, 2>();
    if (a.mask_kind == 2)
      return softcap ? op.template run<IS_BF16, D, true, 2, 2>() : op.template run<IS_BF16, D, false, 2, 2>();
    return softcap ? op.template run<IS_BF16, D, true, 0, 2>() : op.template run<IS_BF16, D, false, 0, 2>();
  }
  if (a.kv_fp8) {
    if (a.mask_kind == 1)
      return softcap ? op.template run<IS_BF16, D, true, 1, 1>() : op.template run<IS_BF16, D, false, 1, 1>();
    if (a.mask_kind == 2)
      return softcap ? op.template run<IS_BF16, D, true, 2, 1>() : op.template run<IS_BF16, D, false, 2, 1>();
    return softcap ? op.template run<IS_BF16, D, true, 0, 1>() : op.template run<IS_BF16, D, false, 0, 1>();
  }
  if (a.mask_kind == 1)
    return softcap ? op.template run<IS_BF16, D, true, 1, 0>() : op.template run<IS_BF16, D, false, 1, 0>();
  if (a.mask_kind == 2)
    return softcap ? op.template run<IS_BF16, D, true, 2, 0>() : op.template run<IS_BF16, D, false, 2, 0>();
  return softcap ? op.template run<IS_BF16, D, true, 0, 0>() : op.template run<IS_BF16, D, false, 0, 0>();
}
template <typename Op, typename R>
R visit(const AttnArgs& a, int dtype, bool softcap, const Op& op, R unsupported) {
  if (dtype == kBF16) {
    if (a.D == 128) return visit_d<true, 128>(a, softcap, op);
    if (a.D == 256) return visit_d<true, 256>(a, softcap, op);
    if (a.D == 64) return visit_d<true, 64>(a, softcap, op);
  } else if (dtype == kF16) {
    if (a.D == 128) return visit_d<false, 128>(a, softcap, op);
    if (a.D == 256) return visit_d<false, 256>(a, softcap, op);
    if (a.D == 64) return visit_d<false, 64>(a, softcap, op);
  }
  return unsupported;
}

struct LaunchOp {
  const AttnArgs& a;
  const DecodeGeometry& geo;
  float* ws;
  hipStream_t stream;
  template <bool IS_BF16, int D, bool SOFTCAP, int MASK, int KVQ, bool FUSE = false>
  hipError_t run() const {
    const int G = grid_of<IS_BF16, D, SOFTCAP, MASK, KVQ, FUSE>();
    unsigned* counters = reinterpret_cast<unsigned*>(ws);
    float* part = ws + geo.counter_floats;
    hipLaunchKernelGGL((decode_kernel<IS_BF16, D, SOFTCAP, MASK, KVQ, FUSE>), dim3(G), dim3(256), 0, stream, a,
                       geo.rows, geo.row_tiles, part, counters);
    return hipGetLastError();
  }
};
struct GridOp {
  template <bool IS_BF16, int D, bool SOFTCAP, int MASK, int KVQ, bool FUSE = false>
  int run() const {
    return grid_of<IS_BF16, D, SOFTCAP, MASK, KVQ, FUSE>();
  }
};

}  // namespace

bool decode_mfma_supported(int dtype, int head_size) {
  return (dtype == kBF16 || dtype == kF16) && (head_size == 64 || head_size == 128 || head_size == 256);
}

DecodeGeometry decode_geometry(int B, int Hkv, int G, int curr, int head_size) {
  DecodeGeometry geo;
  geo.rows = G * curr;
  geo.row_tiles = (geo.rows + kRowsPerTile - 1) / kRowsPerTile;
  geo.tiles = (int64_t)B * Hkv * geo.row_tiles;
  // One 32-bit arrival counter per row tile in a region of fixed size (the
  // most tiles a launch takes), so that calls of any shape find their
  // counters at zero in a shared workspace; then one partial per piece, at
  // most grid + tiles pieces per call.
  geo.counter_floats = kMaxTiles;
  geo.part_floats = (size_t)(kRowsPerTile * head_size + 2 * kRowsPerTile);
  geo.ws_floats = geo.counter_floats + (size_t)(kMaxGrid + geo.tiles) * geo.part_floats;
  geo.fits = geo.tiles <= kMaxTiles;
  return geo;
}

size_t decode_mfma_scratch_floats(const AttnArgs& a, int dtype, bool softcap, const DecodeGeometry& geo) {
  const int grid = visit(a, dtype, softcap, GridOp{}, 0);
  return geo.counter_floats + (size_t)(grid + geo.tiles) * geo.part_floats;
}

hipError_t launch_decode_mfma(const AttnArgs& a, int dtype, bool softcap, const DecodeGeometry& geo,
                              float* ws, hipStream_t stream) {
  if (a.B == 0 || a.Lq == 0) return hipSuccess;
  return visit(a, dtype, softcap, LaunchOp{a, geo, ws, stream}, hipErrorInvalidValue);
}

}  // namespace gqa
