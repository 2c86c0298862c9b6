// Flash-style prompt attention on CDNA4 matrix cores (bf16 / fp16 inputs,
// fp32 accumulation), head sizes 64 and 128.
//
// What it computes is the definition in include/gqa.h; the method is the
// streaming path of "Attention Kernel Design" (section "Compute paths": visit
// KV blocks with an online softmax, keep one score tile and per-row running
// max / denominator / unnormalized output; causal and padding frontiers skip
// whole blocks), with the absolute-position window of "[NPUW] Support GQA
// sliding-window and smooth-softmax in DecomposeGQA" (section "Sliding window
// (local_window_size)") as one more frontier and the sink folded into the
// final denominator (same page, section "smooth_softmax / head_sink").
//
// Layout of the work.
//   * Workgroup = 4 waves = 128 query rows of one (batch, query head); wave w
//     owns rows [32w, 32w+32).  Key tiles of 64 rows are staged in LDS (double
//     buffered, one barrier per tile) and shared by the 4 waves.
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (A = K tile from LDS, B = Q held in
//     registers for the whole kernel), so each lane ends up owning one query
//     row and 16 keys of every 32-key sub-tile.  The K rows fed to the MFMA M
//     index are permuted (key_of_m) so that those 16 keys come as two runs of
//     8 consecutive keys -- exactly the B-operand layout the P*V MFMA needs.
//     P therefore goes from the score accumulators to the next MFMA without
//     an LDS round trip.
//   * O^T += V^T P^T on the same MFMA: V is transposed once while it is
//     written to LDS (4 keys x 8 dims per thread, 8-byte writes), so every
//     MFMA operand is a single 16-byte LDS read.
//   * Online softmax in fp32 with exp2, the scale folded into one FMA, a lazy
//     rescale (the running max only moves when it grows by more than 2^8),
//     and masks evaluated only on boundary sub-tiles; sub-tiles a wave cannot
//     see are skipped.
//   * Work items are ordered (batch, KV head)-major so that the query heads
//     sharing one K/V land on the same XCD (its own L2), heaviest row blocks
//     first within each KV head.
#include "kernels.h"

namespace gqa {
namespace {

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per LDS tile
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

template <bool IS_BF16>
__device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (IS_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// MFMA M index -> key within a 32-key sub-tile.  With m = 8a + 4h + c the
// accumulator register r = 4a + c of lane half h then holds key
// 16*(r/8) + 8h + r%8: two runs of 8 consecutive keys per lane.
__device__ __forceinline__ int key_of_m(int m) {
  const int a = m >> 3, hh = (m >> 2) & 1, c = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + c;
}
// XOR swizzles of 16-byte chunks (bank-conflict-free 16-byte LDS reads).
__device__ __forceinline__ int k_swz(int r) { return (r & 3) | ((r >> 1) & 4); }
__device__ __forceinline__ int v_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

template <bool IS_BF16, int D, bool SOFTCAP>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(AttnArgs a, int nrb, int items,
                                                           int per_xcd) {
  constexpr int KS = D / 16;    // k-steps of the QK^T contraction
  constexpr int DB = D / 32;    // 32-wide output blocks
  constexpr int CPR = D / 8;    // 16-byte chunks per K row
  constexpr int KPT = D / 32;   // keys per thread in the V transpose (and K chunks per thread)
  constexpr int TILE = BN * D;  // elements of one K (or V^T) tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2 * TILE];

  // ---- work item: XCD-major, KV-head-major, heavy row blocks first ----
  const int id = blockIdx.x;
  const int item = (id & 7) * per_xcd + (id >> 3);
  if (item >= items) return;
  const int per_bg = a.G * nrb;
  const int bg = item / per_bg;
  const int rem = item - bg * per_bg;
  const int rb = nrb - 1 - rem / a.G;
  const int hl = rem % a.G;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int h = g * a.G + hl;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 31;
  const int h2 = lane >> 5;

  const BatchSpan sp = batch_span(a, b);
  const int row0 = rb * BM;
  const int rows_here = min(BM, a.Lq - row0);
  const int kv_lo = row_lo(a, sp.q_off + row0);
  const int kv_hi = row_hi(a, sp.q_off + row0 + rows_here - 1, sp.valid);

  const int wrow0 = row0 + 32 * w;
  const int wrows = min(32, a.Lq - wrow0);  // may be <= 0
  const int pw0 = sp.q_off + wrow0;
  const int pw1 = pw0 + max(wrows, 1) - 1;
  const int w_lo = row_lo(a, pw0);
  const int w_hi = row_hi(a, pw1, sp.valid);
  const int my_row = wrow0 + n;
  const int my_p = sp.q_off + my_row;
  const int my_lo = row_lo(a, my_p);
  const int my_hi = row_hi(a, my_p, sp.valid);

  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + b * a.k_sb + g * a.k_sh;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + b * a.v_sb + g * a.v_sh;

  // Q rows stay in registers (B operand of S^T = K Q^T).
  u32x4 qf[KS];
  {
    const bool ok = my_row < a.Lq;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + b * a.q_sb + h * a.q_sh +
                         (int64_t)(ok ? my_row : 0) * a.q_ss + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[ks] = ok ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : z;
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // raw-score units (log2 units with a softcap)
  float l_run = 0.0f;       // partial sum over this lane's keys

  const int nblk = kv_lo <= kv_hi ? (kv_hi - kv_lo + BN) / BN : 0;

  u32x4 kst[KPT], vst[KPT];
  // Global -> registers for the tile starting at key kb.  Keys past kv_hi
  // are never read; zeros stand in for them.
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CPR, cc = c % CPR;
      const int j = kb + r;
      u32x4 z = {0u, 0u, 0u, 0u};
      kst[i] = j <= kv_hi ? *reinterpret_cast<const u32x4*>(Kg + (int64_t)j * a.k_ss + 8 * cc) : z;
    }
    const int dc = tid % CPR, kg = tid / CPR;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = kb + kg * KPT + i;
      u32x4 z = {0u, 0u, 0u, 0u};
      vst[i] = j <= kv_hi ? *reinterpret_cast<const u32x4*>(Vg + (int64_t)j * a.v_ss + 8 * dc) : z;
    }
  };
  // Registers -> LDS: K row-major (swizzled), V transposed to [D][BN] (swizzled).
  auto lstore = [&](int buf) {
    uint16_t* Ks = lds[buf];
    uint16_t* Vt = lds[buf] + TILE;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(Ks + r * D + 8 * (cc ^ k_swz(r))) = kst[i];
    }
    const int dc = tid % CPR, kg = tid / CPR;
    const int key0 = kg * KPT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * dc + e;
      const int chunk = key0 >> 3;
      uint16_t* dst = Vt + d * BN + 8 * (chunk ^ v_swz(d)) + (key0 & 7);
      if constexpr (KPT == 4) {
        const uint32_t x0 = vst[0][e >> 1], x1 = vst[1][e >> 1];
        const uint32_t x2 = vst[2][e >> 1], x3 = vst[3][e >> 1];
        u32x2 pk;
        if (e & 1) {
          pk[0] = (x0 >> 16) | (x1 & 0xffff0000u);
          pk[1] = (x2 >> 16) | (x3 & 0xffff0000u);
        } else {
          pk[0] = (x0 & 0xffffu) | (x1 << 16);
          pk[1] = (x2 & 0xffffu) | (x3 << 16);
        }
        *reinterpret_cast<u32x2*>(dst) = pk;
      } else {
        static_assert(KPT == 2, "head size 64 or 128");
        const uint32_t x0 = vst[0][e >> 1], x1 = vst[1][e >> 1];
        const uint32_t pk = (e & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
        *reinterpret_cast<uint32_t*>(dst) = pk;
      }
    }
  };

  const float c_l2 = SOFTCAP ? 1.0f : a.scale_log2;  // raw units -> log2 units
  const int kr0 = key_of_m(n);                        // this lane's K row in a sub-tile

  if (nblk > 0) {
    gload(kv_lo);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < nblk; ++it) {
    const int kb = kv_lo + it * BN;
    const int buf = it & 1;
    if (it + 1 < nblk) gload(kb + BN);

    const uint16_t* Ks = lds[buf];
    const uint16_t* Vt = lds[buf] + TILE;
    // Scores of the two 32-key sub-tiles.  A sub-tile this wave cannot see is
    // skipped and its accumulator is never read (every consumer below tests
    // act[]); no register fill stands in for it.
    bool act[2];
    f32x16 s[2];
    float bm = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int k0 = kb + 32 * sub;
      act[sub] = wrows > 0 && k0 <= w_hi && k0 + 31 >= w_lo;
      if (!act[sub]) continue;
      const int r = 32 * sub + kr0;
      const uint16_t* kp = Ks + r * D;
      const int sw = k_swz(r);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kp + 8 * ((2 * ks + h2) ^ sw));
        acc = mma32<IS_BF16>(kf, qf[ks], acc);
      }
      if constexpr (SOFTCAP) {
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) acc[r2] = a.cap_log2 * tanh_f32(acc[r2] * a.scale_over_cap);
      }
      // masks only where the sub-tile crosses a frontier of some row of this wave
      const bool interior = (a.window < 0 || k0 >= pw1 - a.window + 1) &&
                            (!a.causal || k0 + 31 <= pw0) && (k0 + 31 < sp.valid);
      if (!interior) {
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) {
          const int j = k0 + 16 * (r2 >> 3) + 8 * h2 + (r2 & 7);
          acc[r2] = (j < my_lo || j > my_hi) ? -INFINITY : acc[r2];
        }
      }
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) bm = fmaxf(bm, acc[r2]);
      s[sub] = acc;
    }

    // ---- online softmax (lane owns row n; lanes n and n+32 share the row) ----
    bm = fmaxf(bm, xor32(bm));
    const float m_new = fmaxf(m_run, bm);
    const bool need = (m_new - m_run) * c_l2 > kRescaleLog2;  // false while both are -inf
    if (__any(need)) {
      const float alpha = need ? fast_exp2((m_run - m_new) * c_l2) : 1.0f;
      m_run = need ? m_new : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) o[db][r2] *= alpha;
    }
    const float mb = m_run == -INFINITY ? 0.0f : m_run * c_l2;
    u32x4 pb[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (!act[sub]) continue;
      float pv[16];
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) {
        pv[r2] = fast_exp2(fmaf(s[sub][r2], c_l2, -mb));
        l_run += pv[r2];
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2)
          pb[sub][t][q2] = pack2<IS_BF16>(pv[8 * t + 2 * q2], pv[8 * t + 2 * q2 + 1]);
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 32 * db + n;
      const uint16_t* vp = Vt + d * BN;
      const int sw = v_swz(d);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (!act[sub]) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int chunk = 4 * sub + 2 * t + h2;
          const u32x4 vf = *reinterpret_cast<const u32x4*>(vp + 8 * (chunk ^ sw));
          o[db] = mma32<IS_BF16>(vf, pb[sub][t], o[db]);
        }
      }
    }

    if (it + 1 < nblk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: fold the sink, normalize, narrow, store ----
  if (my_row >= a.Lq) return;
  const float l_row = l_run + xor32(l_run);
  float fac;
  if (my_lo > my_hi) {
    fac = 0.0f;
  } else if (a.use_sink) {
    const float mt = m_run * c_l2;
    const float ts = sink_log2(a, h);
    const float M = fmaxf(mt, ts);
    const float e1 = fast_exp2(mt - M);
    fac = e1 / (l_row * e1 + fast_exp2(ts - M));
  } else {
    fac = 1.0f / l_row;
  }
  uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)my_row * a.o_ss;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 pk;
      pk[0] = pack2<IS_BF16>(o[db][4 * q4] * fac, o[db][4 * q4 + 1] * fac);
      pk[1] = pack2<IS_BF16>(o[db][4 * q4 + 2] * fac, o[db][4 * q4 + 3] * fac);
      *reinterpret_cast<u32x2*>(op + 32 * db + 8 * q4 + 4 * h2) = pk;
    }
}

template <bool IS_BF16, int D>
hipError_t launch_t(const AttnArgs& a, bool softcap, hipStream_t stream) {
  const int nrb = (a.Lq + BM - 1) / BM;
  const int items = a.B * a.Hq * nrb;
  const int per_xcd = (items + 7) / 8;
  dim3 grid(8 * per_xcd), block(256);
  if (softcap)
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, true>), grid, block, 0, stream, a, nrb, items, per_xcd);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, false>), grid, block, 0, stream, a, nrb, items, per_xcd);
  return hipGetLastError();
}

}  // namespace

bool prefill_mfma_supported(int dtype, int head_size) {
  return (dtype == kBF16 || dtype == kF16) && (head_size == 64 || head_size == 128);
}

hipError_t launch_prefill_mfma(const AttnArgs& a, int dtype, bool softcap, hipStream_t stream) {
  if (a.B == 0 || a.Lq == 0) return hipSuccess;
  if (dtype == kBF16) {
    if (a.D == 128) return launch_t<true, 128>(a, softcap, stream);
    if (a.D == 64) return launch_t<true, 64>(a, softcap, stream);
  } else if (dtype == kF16) {
    if (a.D == 128) return launch_t<false, 128>(a, softcap, stream);
    if (a.D == 64) return launch_t<false, 64>(a, softcap, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
