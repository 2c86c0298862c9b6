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
// Per 16-key unit: K goes straight from HBM into the A operand of
// v_mfma_f32_16x16x32 (S^T = K Q^T, Q in registers); V is read with 16-byte
// coalesced loads, transposed through a wave-private LDS slice and fed to
// v_mfma_f32_16x16x16 (O^T += V^T P^T), whose B operand layout is exactly the
// score accumulator layout.  Each wave keeps the next unit's loads in flight
// while it computes the current one.
#include <algorithm>

#include "kernels.h"

namespace gqa {
namespace {

constexpr int kRowsPerTile = 16;
constexpr int kSub = 16;              // keys per unit (MFMA M)
constexpr int kVtStride = 24;         // elements per V^T row in LDS (16 keys + pad)
constexpr float kRescaleLog2 = 8.0f;
constexpr int kMaxTiles = 2048;       // row tiles per call on this path
constexpr int kMaxGrid = 2048;        // workgroups per launch (upper bound)

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

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
  constexpr int KQ = D / 32;    // k-steps of 16x16x32 over the head dim
  constexpr int DB = D / 16;    // 16-wide output blocks
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int KPL = D / 32;   // keys per lane in the V transpose
  constexpr int PART = kRowsPerTile * D + 2 * kRowsPerTile;  // floats per partial
  constexpr int MERGE = D / 4 + 2;                            // floats per lane in a merge slot
  constexpr int XB = 64;                                      // partials per combine batch
  // V^T slices of the 4 waves; between pieces the same bytes hold the merge
  // slots, and in the combine the per-split maxima and sums.
  static_assert(2 * MERGE * 64 * 4 <= 4 * D * kVtStride * 2, "merge slots fit the V^T slices");
  static_assert(2 * XB * kRowsPerTile + 3 * kRowsPerTile <= 4 * D * kVtStride / 2, "combine fits LDS");
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[4][D * kVtStride];
  __shared__ int pre[kMaxTiles + 1];  // unit prefix sum over tiles
  __shared__ int wsum[4];
  __shared__ int flag;
  float (*merge_lds)[MERGE * 64] = reinterpret_cast<float (*)[MERGE * 64]>(&vt_lds[0][0]);

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
  uint16_t* vt = vt_lds[w];
  const int vdc = lane % CPR, vkg = lane / CPR;

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

    // units of this wave: ua + w, ua + w + 4, ...
    const int nw = ub - ua > w ? (ub - ua - w + 3) / 4 : 0;
    // Loads are unconditional: a row past the piece end is clamped to the
    // piece's last key (a real key, finite, masked out for every query row),
    // so there is no per-lane branch and the wait counters keep the next
    // unit's loads in flight while the current one is computed.
    u32x4 kr[2][KQ], vr[2][KPL];
    auto issue = [&](int slot, int j) {
      const int kb = c_lo + kSub * (w + 4 * j);
      const int jk = min(kb + n, c_hi);
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks)
        kr[slot][ks] = *reinterpret_cast<const u32x4*>(Kg + (int64_t)jk * a.k_ss + 32 * ks + 8 * q4);
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int jv = min(kb + vkg * KPL + e, c_hi);
        vr[slot][e] = *reinterpret_cast<const u32x4*>(Vg + (int64_t)jv * a.v_ss + 8 * vdc);
      }
    };
    if (nw > 0) issue(0, 0);
    u32x4 qf[KQ];
    {
      // padding rows load a row of the group (in bounds) and are zeroed
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + x.b * a.q_sb + my_h * a.q_sh +
                           (int64_t)my_t * a.q_ss + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
        const u32x4 z = {0u, 0u, 0u, 0u};
        qf[ks] = row_ok ? v : z;
      }
    }

    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.0f;

    auto compute = [&](int slot, int j) {
      const int kb = c_lo + kSub * (w + 4 * j);
      // V -> V^T in this wave's LDS slice (reads of the previous unit are
      // issued before these writes in program order)
      wave_lds_fence();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * vdc + e;
        uint16_t* dst = vt + d * kVtStride + vkg * KPL;
        uint32_t pk[KPL / 2];
#pragma unroll
        for (int y = 0; y < KPL / 2; ++y) {
          const uint32_t x0 = vr[slot][2 * y][e >> 1], x1 = vr[slot][2 * y + 1][e >> 1];
          pk[y] = (e & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
        }
        if constexpr (KPL == 8) {
          *reinterpret_cast<u32x4*>(dst) = u32x4{pk[0], pk[1], pk[2], pk[3]};
        } else if constexpr (KPL == 4) {
          *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
        } else {
          *reinterpret_cast<uint32_t*>(dst) = pk[0];
        }
      }
      // S^T = K Q^T
      f32x4 sc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) sc = mma_qk<IS_BF16>(kr[slot][ks], qf[ks], sc);
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
      // O^T += V^T P^T
      wave_lds_fence();
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 vf = *reinterpret_cast<const u32x2*>(vt + (16 * db + n) * kVtStride + 4 * q4);
        o[db] = mma_pv<IS_BF16>(vf, pp, o[db]);
      }
    };

    // two-slot pipeline: the next unit's loads go out before this unit's math
    for (int j = 0; j < nw; j += 2) {
      if (j + 1 < nw) issue(1, j + 1);
      compute(0, j);
      if (j + 1 >= nw) break;
      if (j + 2 < nw) issue(0, j + 2);
      compute(1, j + 1);
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
    __syncthreads();  // the merge slots are V^T slices again for the next piece
    ++t;
  }

  // ---- arrivals: the last workgroup to finish a tile merges its partials ----
  // Every writer waits until its write-through stores have completed
  // (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  float* lf = reinterpret_cast<float*>(&vt_lds[0][0]);  // [XB][16] maxima, then factors
  float* ls = lf + XB * kRowsPerTile;                     // [XB][16] sums
  float* rowM = ls + XB * kRowsPerTile;
  float* rowL = rowM + kRowsPerTile;
  float* rowA = rowL + kRowsPerTile;
  bool acquired = false;
  for (int tt = t_first; tt <= t_last; ++tt) {
    if (pre[tt + 1] == pre[tt]) continue;
    const int first = owner_of(pre[tt], U, Gs);
    const int last = owner_of(pre[tt + 1] - 1, U, Gs);
    const int nvalid = last - first + 1;
    if (tid == 0)
      flag = __hip_atomic_fetch_add(&counters[tt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(nvalid - 1);
    __syncthreads();
    const bool is_last = flag;
    __syncthreads();
    if (!is_last) continue;
    if (!acquired) {
      // acquire at device scope once: the plain loads below then see the
      // other workgroups' write-through stores
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      acquired = true;
    }
    const Tile x = make_tile(a, rows, nrt, tt);
    const float* gpart = part + (int64_t)(first + tt) * PART;

    // Merge the nvalid partials, XB at a time.  Per batch: (1) every (split,
    // row) max and sum is fetched in parallel into LDS; (2) one thread per row
    // moves the row's running max, rescales its running sum and turns the
    // batch's maxima into factors exp2(m_x - M); (3) TQ threads per output
    // quad accumulate factor * acc over disjoint splits (all relative to the
    // same M), reduced with shuffles at the end.
    const int items = x.rows_tile * (D / 4);
    // threads per output quad: the largest power of two with items * TQ <= 256
    const int TQ = items <= 16 ? 16 : (items <= 32 ? 8 : (items <= 64 ? 4 : (items <= 128 ? 2 : 1)));
    const int t_sub = tid % TQ;
    constexpr int IPT = (kRowsPerTile * (D / 4) + 255) / 256;  // output quads per thread when TQ == 1
    f32x4 acc[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) acc[q] = f32x4{};
    if (tid < kRowsPerTile) {
      rowM[tid] = -INFINITY;
      rowL[tid] = 0.0f;
    }
    for (int xb = 0; xb < nvalid; xb += XB) {
      const int nb = min(XB, nvalid - xb);
      __syncthreads();
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
        const int item = (tid / TQ) + q * (256 / TQ);
        if (item >= items) break;
        const int r = item / (D / 4), dq = item % (D / 4);
        acc[q] *= rowA[r];
#pragma unroll 8
        for (int xs = t_sub; xs < nb; xs += TQ) {
          const float* p = gpart + (int64_t)(xb + xs) * PART + r * D + 4 * dq;
          acc[q] += *reinterpret_cast<const f32x4*>(p) * lf[xs * kRowsPerTile + r];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
      for (int off = TQ / 2; off > 0; off >>= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q][e] += __shfl_xor(acc[q][e], off, 64);
      const int item = (tid / TQ) + q * (256 / TQ);
      if (item >= items || t_sub != 0) continue;
      const int r = item / (D / 4), dq = item % (D / 4);
      const int row = kRowsPerTile * x.rt + r;
      const int h = x.g * a.G + row % a.G;
      const float M = rowM[r], L = rowL[r];
      float fac;
      if (M == -INFINITY) {
        fac = 0.0f;
      } else if (a.use_sink) {
        const float tsk = sink_log2(a, h);
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
