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
// 16-key units.  Every workgroup computes the same prefix sum of units over
// all row tiles (the lengths live on the device) and takes an equal
// contiguous slice of the flattened unit list; the grid is exactly as many
// workgroups as the GPU holds at once, so all of them stream from the first
// microsecond and finish together.  A slice may cross tile boundaries; each
// piece (slice x tile) leaves one fp32 partial (acc, max, sum).  At the end
// every workgroup bumps the arrival counter of each tile it touched; the last
// arrival of a tile merges its partials, folds the sink and writes O.
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

#include "kernels.h"

namespace gqa {
namespace {

constexpr int kRowsPerTile = 16;
constexpr int kSub = 16;              // keys per unit (MFMA M)
constexpr int kWaves = 4;
constexpr float kRescaleLog2 = 8.0f;
constexpr int kMaxTiles = 2048;       // row tiles per call on this path
constexpr int kMaxGrid = 2048;        // workgroups per launch (upper bound)

// LDS staging of one wave: kStages units of K and V, 32 KB in flight.
template <int D>
struct Ring {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kSlots = D / 8;                     // 16-byte chunks per key row
  static constexpr int kUnitBytes = kSub * kRowBytes;      // K (or V) bytes of one unit
  static constexpr int kDmaPerUnit = kUnitBytes / 1024;    // wave-wide 16-byte DMA loads
  static constexpr int kStages = 32768 / (2 * kUnitBytes);
  static constexpr int kWaveBytes = kStages * 2 * kUnitBytes;
  static_assert(kUnitBytes % 1024 == 0, "a unit is whole DMA instructions");
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

// A row tile and the union of its rows' allowed intervals.
struct Tile {
  int b, g, rt, bg;
  BatchSpan sp;
  int lo, hi;        // union key interval (empty when lo > hi)
  int rows_tile;     // query rows in this tile (<= 16)
};
__device__ __forceinline__ Tile make_tile(const AttnArgs& a, int rows, int nrt, int t) {
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

template <bool IS_BF16, int D, bool SOFTCAP>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a, int rows, int nrt,
                                                     float* __restrict__ part, unsigned* __restrict__ counters) {
  using RG = Ring<D>;
  constexpr int KQ = D / 32;    // k-steps of 16x16x32 over the head dim
  constexpr int DB = D / 16;    // 16-wide output blocks
  constexpr int S = RG::kStages;
  constexpr int PART = kRowsPerTile * D + 2 * kRowsPerTile;  // floats per partial
  constexpr int MERGE = D / 4 + 2;                            // floats per lane in a merge slot
  constexpr int XB = 64;                                      // partials per combine batch
  // The rings hold the LDS stages while streaming, the wave merge slots
  // between pieces and the combine's per-split maxima and sums at the end.
  static_assert(2 * MERGE * 64 * 4 <= kWaves * RG::kWaveBytes, "merge slots fit the rings");
  static_assert((2 * XB * kRowsPerTile + 4 * kRowsPerTile) * 4 <= kWaves * RG::kWaveBytes, "combine fits");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kWaves * RG::kWaveBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds[kRowsPerTile * 2 * D];  // Q tile, swizzled like K
  __shared__ int pre[kMaxTiles + 1];  // unit prefix sum over tiles
  __shared__ int wsum[4];
  __shared__ int flag[256];
  float (*merge_lds)[MERGE * 64] = reinterpret_cast<float (*)[MERGE * 64]>(&ring[0]);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 15;
  const int q4 = lane >> 4;
  const int G = gridDim.x;
  const int k = blockIdx.x;
  const int T = a.B * a.Hkv * nrt;

  // ---- prefix sum of 16-key units over all row tiles (same in every workgroup) ----
  {
    int carry = 0;
    if (tid == 0) pre[0] = 0;
    for (int base = 0; base < T; base += 256) {
      const int t = base + tid;
      int u = 0;
      if (t < T) u = units_of(make_tile(a, rows, nrt, t));
      int incl = u;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (lane == 63) wsum[w] = incl;
      __syncthreads();
      int before = carry;
      for (int x = 0; x < w; ++x) before += wsum[x];
      if (t < T) pre[t + 1] = before + incl;
      carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
      __syncthreads();
    }
  }
  const int U = pre[T];

  // tiles nobody streams (no allowed key for any of their rows) output zeros
  for (int t = k; t < T; t += G) {
    if (pre[t + 1] != pre[t]) continue;
    const Tile x = make_tile(a, rows, nrt, t);
    for (int idx = tid; idx < x.rows_tile * (D / 4); idx += 256) {
      const int row = kRowsPerTile * x.rt + idx / (D / 4);
      store_row4<IS_BF16, D>(a, x.b, x.g * a.G + row % a.G, row / a.G, 4 * (idx % (D / 4)), f32x4{});
    }
  }
  // Slices: workgroup k < Gs streams units [floor(U k / Gs), floor(U (k+1) / Gs)).
  // With Gs <= U no slice is empty, so the owners of a tile's units are
  // exactly the consecutive workgroups between its first and last owner.
  const int Gs = min(G, U);
  if (k >= Gs) return;

  const int ustart = (int)((int64_t)U * k / Gs);
  const int uend = (int)((int64_t)U * (k + 1) / Gs);
  // first tile holding unit ustart: the largest t with pre[t] <= ustart
  int t_first = 0;
  {
    int lo = 0, hi = T;  // invariant: pre[lo] <= ustart < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= ustart) lo = mid; else hi = mid;
    }
    t_first = lo;
  }
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
    const Tile x = make_tile(a, rows, nrt, t);
    const int c_lo = x.lo + kSub * ua;
    const int c_hi = min(x.hi, x.lo + kSub * ub - 1);

    // this lane's query row (padding rows carry zeros and are never stored)
    const int my_r = kRowsPerTile * x.rt + n;
    const bool row_ok = n < x.rows_tile;
    const int my_t = row_ok ? my_r / a.G : 0;
    const int my_h = x.g * a.G + (row_ok ? my_r % a.G : 0);
    const int my_p = x.sp.q_off + my_t;
    const int lo_eff = max(row_lo(a, my_p), c_lo);
    const int hi_eff = min(row_hi(a, my_p, x.sp.valid), c_hi);
    const int p_first = x.sp.q_off + (kRowsPerTile * x.rt) / a.G;
    const int p_last = x.sp.q_off + (kRowsPerTile * x.rt + x.rows_tile - 1) / a.G;

    const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + x.b * a.k_sb + x.g * a.k_sh;
    const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + x.b * a.v_sb + x.g * a.v_sh;

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
    // Rows past the piece end are clamped to its last key (a real key,
    // finite, masked out for every query row): no per-lane branches.
    auto issue = [&](int s, int j) {
      const int kb = c_lo + kSub * (w + 4 * j);
      unsigned char* kdst = my_ring + s * 2 * RG::kUnitBytes;
      unsigned char* vdst = kdst + RG::kUnitBytes;
#pragma unroll
      for (int i = 0; i < RG::kDmaPerUnit; ++i) {
        const int pos = 64 * i + lane;                 // 16-byte chunk position in the unit
        const int key = pos / RG::kSlots;
        const int cc = (pos % RG::kSlots) ^ swz<D>(key);  // the global chunk stored there
        const int row = min(kb + key, c_hi);
        __builtin_amdgcn_global_load_lds((global_void*)(Kg + (int64_t)row * a.k_ss + 8 * cc),
                                         (lds_void*)(kdst + 1024 * i), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((global_void*)(Vg + (int64_t)row * a.v_ss + 8 * cc),
                                         (lds_void*)(vdst + 1024 * i), 16, 0, 0);
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

    for (int j = 0; j < nw; ++j) {
      const int s = j % S;
      wait_units<2 * RG::kDmaPerUnit, S>(min(S - 1, nw - 1 - j));
      const int kb = c_lo + kSub * (w + 4 * j);
      const uint32_t st = ring_addr + s * 2 * RG::kUnitBytes;
      // S^T = K Q^T
      u32x4 kf[KQ];
#pragma unroll
      for (int ks = 0; ks < KQ; ks += 2) lds_read2_b128(kf[ks], kf[ks + 1], st + k_off[ks], st + k_off[ks + 1]);
      f32x4 sc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) sc = mma_qk<IS_BF16>(kf[ks], qf[ks], sc);
      if constexpr (SOFTCAP) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = a.cap_log2 * tanh_f32(sc[r] * a.scale_over_cap);
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
      // online softmax: lanes n, n+16, n+32, n+48 share row n
      float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run, bm);
      const bool need = (m_new - m_run) * c_l2 > kRescaleLog2;
      if (__any(need)) {
        const float alpha = need ? fast_exp2((m_run - m_new) * c_l2) : 1.0f;
        m_run = need ? m_new : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
      }
      const float mb = m_run == -INFINITY ? 0.0f : m_run * c_l2;
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = fast_exp2(fmaf(sc[r], c_l2, -mb));
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
      if (j + S < nw) issue(s, j + S);
    }

    // ---- merge the 4 waves through LDS (lane-to-lane: identical layouts) ----
    auto put = [&](int slot) {
      float* ml = merge_lds[slot];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) ml[(4 * db + r) * 64 + lane] = o[db][r];
      ml[(D / 4) * 64 + lane] = m_run;
      ml[(D / 4 + 1) * 64 + lane] = l_run;
    };
    auto take = [&](int slot) {
      const float* ml = merge_lds[slot];
      const float m_b = ml[(D / 4) * 64 + lane];
      const float l_b = ml[(D / 4 + 1) * 64 + lane];
      const float M = fmaxf(m_run, m_b);
      if (M == -INFINITY) return;
      const float fa = fast_exp2((m_run - M) * c_l2);
      const float fb = fast_exp2((m_b - M) * c_l2);
      l_run = l_run * fa + l_b * fb;
      m_run = M;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[db][r] = o[db][r] * fa + ml[(4 * db + r) * 64 + lane] * fb;
    };
    __syncthreads();
    if (w >= 2) put(w - 2);
    __syncthreads();
    if (w < 2) take(w);
    __syncthreads();
    if (w == 1) put(0);
    __syncthreads();
    if (w == 0) {
      take(0);
      float l_row = l_run + __shfl_xor(l_run, 16, 64);
      l_row += __shfl_xor(l_row, 32, 64);
      if (row_ok) {
        float* p = part + (int64_t)(k + t) * PART;  // slot k + t: unique per piece
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) coherent_store(p + n * D + 16 * db + 4 * q4 + r, o[db][r]);
        if (q4 == 0) {
          coherent_store(p + kRowsPerTile * D + n, m_run == -INFINITY ? -INFINITY : m_run * c_l2);
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
  float* lf = reinterpret_cast<float*>(&ring[0]);  // [XB][16] maxima, then factors
  float* ls = lf + XB * kRowsPerTile;                     // [XB][16] sums
  float* rowM = ls + XB * kRowsPerTile;
  float* rowL = rowM + kRowsPerTile;
  float* rowA = rowL + kRowsPerTile;
  float* rowS = rowA + kRowsPerTile;
  bool acquired = false;
  for (int base = t_first; base <= t_last; base += 256) {
  // one arrival per touched tile, all in flight together
  const int nbt = min(256, t_last - base + 1);
  if (tid < nbt) {
    const int tt = base + tid;
    int f = 0;
    if (pre[tt + 1] != pre[tt]) {
      const int nvalid = owner_of(pre[tt + 1] - 1, U, Gs) - owner_of(pre[tt], U, Gs) + 1;
      f = __hip_atomic_fetch_add(&counters[tt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          (unsigned)(nvalid - 1);
    }
    flag[tid] = f;
  }
  __syncthreads();
  for (int i = 0; i < nbt; ++i) {
    if (!flag[i]) continue;
    const int tt = base + i;
    const int first = owner_of(pre[tt], U, Gs);
    const int nvalid = owner_of(pre[tt + 1] - 1, U, Gs) - first + 1;
    if (!acquired) {
      // acquire at device scope once: the plain loads below then see the
      // other workgroups' write-through stores
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      acquired = true;
    }
    const Tile x = make_tile(a, rows, nrt, tt);
    const float* gpart = part + (int64_t)(first + tt) * PART;

    // Merge the nvalid partials in batches.  Per batch: (1) every thread
    // issues the loads of all its partial accumulators of the batch (output
    // quads x splits, clamped indices, all in flight together), then (2) the
    // per-(split, row) maxima and sums are fetched into LDS -- one round trip
    // for both; (3) one thread per row moves the row's running max, rescales
    // its running sum and turns the batch's maxima into factors exp2(m_x - M);
    // (4) TQ threads per output quad accumulate factor * acc over disjoint
    // splits (all relative to the same M), reduced with shuffles at the end.
    const int items = x.rows_tile * (D / 4);
    // threads per output quad: the largest power of two with items * TQ <= 256
    const int TQ = items <= 16 ? 16 : (items <= 32 ? 8 : (items <= 64 ? 4 : (items <= 128 ? 2 : 1)));
    const int t_sub = tid % TQ;
    constexpr int IPT = (kRowsPerTile * (D / 4) + 255) / 256;  // output quads per thread when TQ == 1
    constexpr int NPT = 32 / IPT;                               // splits per output quad and batch
    const int XBt = min(XB, NPT * TQ);
    int it_r[IPT], it_d[IPT];
    bool it_ok[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
      const int item = (tid / TQ) + q * (256 / TQ);
      it_ok[q] = item < items;
      const int ic = it_ok[q] ? item : 0;
      it_r[q] = ic / (D / 4);
      it_d[q] = ic % (D / 4);
    }
    // sink logits of the tile's rows, fetched now so that the load overlaps the partials'
    float sink_row = 0.0f;
    if (a.use_sink && tid < x.rows_tile) {
      const int row = kRowsPerTile * x.rt + tid;
      sink_row = sink_log2(a, x.g * a.G + row % a.G);
    }
    f32x4 acc[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) acc[q] = f32x4{};
    if (tid < kRowsPerTile) {
      rowM[tid] = -INFINITY;
      rowL[tid] = 0.0f;
    }
    for (int xb = 0; xb < nvalid; xb += XBt) {
      const int nb = min(XBt, nvalid - xb);
      f32x4 v[IPT][NPT];
#pragma unroll
      for (int q = 0; q < IPT; ++q)
#pragma unroll
        for (int e = 0; e < NPT; ++e) {
          const int xs = min(t_sub + e * TQ, nb - 1);
          v[q][e] = *reinterpret_cast<const f32x4*>(gpart + (int64_t)(xb + xs) * PART + it_r[q] * D + 4 * it_d[q]);
        }
      // the previous batch's factor reads are complete before they are
      // overwritten (LDS-only fences: no DMA load is in flight here)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      for (int pr = tid; pr < nb * x.rows_tile; pr += 256) {
        const int xs = pr / x.rows_tile, r = pr % x.rows_tile;
        const float* p = gpart + (int64_t)(xb + xs) * PART + kRowsPerTile * D;
        lf[xs * kRowsPerTile + r] = p[r];
        ls[xs * kRowsPerTile + r] = p[kRowsPerTile + r];
      }
      __syncthreads();
      if (tid < x.rows_tile) {
        const int r = tid;
        float mb = -INFINITY;
        for (int xs = 0; xs < nb; ++xs) mb = fmaxf(mb, lf[xs * kRowsPerTile + r]);
        const float Mo = rowM[r];
        const float Mn = fmaxf(Mo, mb);
        float L = 0.0f, alpha = 1.0f;
        if (Mn != -INFINITY) {
          alpha = fast_exp2(Mo - Mn);  // 0 while nothing was seen
          L = rowL[r] * alpha;
          for (int xs = 0; xs < nb; ++xs) {
            const float f = fast_exp2(lf[xs * kRowsPerTile + r] - Mn);
            lf[xs * kRowsPerTile + r] = f;
            L += ls[xs * kRowsPerTile + r] * f;
          }
        } else {
          for (int xs = 0; xs < nb; ++xs) lf[xs * kRowsPerTile + r] = 0.0f;
        }
        rowM[r] = Mn;
        rowL[r] = L;
        rowA[r] = alpha;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < IPT; ++q) {
        if (!it_ok[q]) continue;
        const int r = it_r[q];
        acc[q] *= rowA[r];
#pragma unroll
        for (int e = 0; e < NPT; ++e) {
          const int xs = t_sub + e * TQ;
          acc[q] += v[q][e] * (xs < nb ? lf[xs * kRowsPerTile + r] : 0.0f);
        }
      }
    }
    if (tid < x.rows_tile) rowS[tid] = sink_row;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
      for (int off = TQ / 2; off > 0; off >>= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q][e] += __shfl_xor(acc[q][e], off, 64);
      if (!it_ok[q] || t_sub != 0) continue;
      const int r = it_r[q], dq = it_d[q];
      const int row = kRowsPerTile * x.rt + r;
      const int h = x.g * a.G + row % a.G;
      const float M = rowM[r], L = rowL[r];
      float fac;
      if (M == -INFINITY) {
        fac = 0.0f;
      } else if (a.use_sink) {
        const float tsk = rowS[r];
        const float M2 = fmaxf(M, tsk);
        const float e1 = fast_exp2(M - M2);
        fac = e1 / (L * e1 + fast_exp2(tsk - M2));
      } else {
        fac = 1.0f / L;
      }
      store_row4<IS_BF16, D>(a, x.b, h, row / a.G, 4 * dq, acc[q] * fac);
    }
    if (tid == 0)  // ready for the next call
      __hip_atomic_store(&counters[tt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
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

template <bool IS_BF16, int D, bool SOFTCAP>
hipError_t launch_t(const AttnArgs& a, const DecodeGeometry& geo, float* ws, hipStream_t stream) {
  auto kernel = decode_kernel<IS_BF16, D, SOFTCAP>;
  static int grid_cache[16] = {0};  // per device; a benign race computes the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  int G = grid_cache[dev];
  if (G == 0) G = grid_cache[dev] = resident_grid(kernel);
  unsigned* counters = reinterpret_cast<unsigned*>(ws);
  float* part = ws + geo.counter_floats;
  hipLaunchKernelGGL(kernel, dim3(G), dim3(256), 0, stream, a, geo.rows, geo.row_tiles, part, counters);
  return hipGetLastError();
}

template <bool IS_BF16, int D>
hipError_t launch_d(const AttnArgs& a, bool softcap, const DecodeGeometry& geo, float* ws, hipStream_t stream) {
  return softcap ? launch_t<IS_BF16, D, true>(a, geo, ws, stream) : launch_t<IS_BF16, D, false>(a, geo, ws, stream);
}

}  // namespace

bool decode_mfma_supported(int dtype, int head_size) {
  return (dtype == kBF16 || dtype == kF16) && (head_size == 64 || head_size == 128 || head_size == 256);
}

DecodeGeometry decode_geometry(int B, int Hkv, int G, int curr, int head_size) {
  DecodeGeometry geo;
  geo.rows = G * curr;
  geo.row_tiles = (geo.rows + kRowsPerTile - 1) / kRowsPerTile;
  geo.tiles = (int64_t)B * Hkv * geo.row_tiles;
  // one 32-bit arrival counter per row tile (256-byte aligned), then one
  // partial per piece: at most grid + tiles pieces per call
  geo.counter_floats = (size_t)(geo.tiles + 63) / 64 * 64;
  geo.ws_floats = geo.counter_floats +
                  (size_t)(kMaxGrid + geo.tiles) * (size_t)(kRowsPerTile * head_size + 2 * kRowsPerTile);
  geo.fits = geo.tiles <= kMaxTiles;
  return geo;
}

hipError_t launch_decode_mfma(const AttnArgs& a, int dtype, bool softcap, const DecodeGeometry& geo,
                              float* ws, hipStream_t stream) {
  if (a.B == 0 || a.Lq == 0) return hipSuccess;
  if (dtype == kBF16) {
    if (a.D == 128) return launch_d<true, 128>(a, softcap, geo, ws, stream);
    if (a.D == 256) return launch_d<true, 256>(a, softcap, geo, ws, stream);
    if (a.D == 64) return launch_d<true, 64>(a, softcap, geo, ws, stream);
  } else if (dtype == kF16) {
    if (a.D == 128) return launch_d<false, 128>(a, softcap, geo, ws, stream);
    if (a.D == 256) return launch_d<false, 256>(a, softcap, geo, ws, stream);
    if (a.D == 64) return launch_d<false, 64>(a, softcap, geo, ws, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
