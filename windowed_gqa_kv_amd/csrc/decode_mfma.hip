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
// Structure.
//   split kernel: grid (splits, B*Hkv*row_tiles).  A workgroup takes one
//     chunk of the union key range of a 16-row tile; its 4 waves take 16-key
//     sub-tiles round-robin.  Per sub-tile: K goes straight from HBM into the
//     A operand of v_mfma_f32_16x16x32 (S^T = K Q^T, Q held in registers); V
//     is loaded with 16-byte coalesced reads, transposed through a wave-private
//     LDS slice and fed to v_mfma_f32_16x16x16 (O^T += V^T P^T), whose B
//     operand layout is exactly the score accumulator layout.  The next
//     sub-tile's K/V loads are in flight while the current one is computed.
//     The 4 waves merge (max, sum, acc) through LDS and one fp32 partial per
//     (tile, split) goes to the workspace.
//   combine kernel: one workgroup per (batch, KV head, row tile) merges the
//     partials with the log-sum-exp rule, folds the sink, normalizes and
//     narrows to the output type.
#include <algorithm>

#include "kernels.h"

namespace gqa {
namespace {

constexpr int kRowsPerTile = 16;
constexpr int kSub = 16;              // keys per sub-tile (MFMA M)
constexpr int kVtStride = 24;         // elements per V^T row in LDS (16 keys + pad)
constexpr float kRescaleLog2 = 8.0f;

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

// Union of the allowed intervals of the rows of one tile.
struct TileSpan {
  int lo, hi;
};
__device__ __forceinline__ TileSpan tile_span(const AttnArgs& a, const BatchSpan& sp, int rows, int rt) {
  const int r_first = kRowsPerTile * rt;
  const int r_last = min(rows, r_first + kRowsPerTile) - 1;
  TileSpan t;
  t.lo = row_lo(a, sp.q_off + r_first / a.G);
  t.hi = row_hi(a, sp.q_off + r_last / a.G, sp.valid);
  return t;
}

template <bool IS_BF16, int D, bool SOFTCAP>
__global__ __launch_bounds__(256) void decode_split_kernel(AttnArgs a, int rows, int nrt, int chunk,
                                                           int nsplit, float* __restrict__ ws) {
  constexpr int KQ = D / 32;    // k-steps of 16x16x32 over the head dim
  constexpr int DB = D / 16;    // 16-wide output blocks
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int KPL = D / 32;   // keys per lane in the V transpose
  constexpr int PART = kRowsPerTile * D + 2 * kRowsPerTile;  // floats per partial
  constexpr int MERGE = D / 4 + 2;                            // floats per lane in a merge slot
  // V^T slices of the 4 waves; after the key loop the same bytes hold the
  // two merge slots (2 * MERGE * 64 floats <= 4 * D * kVtStride halves).
  static_assert(2 * MERGE * 64 * 4 <= 4 * D * kVtStride * 2, "merge slots fit the V^T slices");
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[4][D * kVtStride];
  float (*merge_lds)[MERGE * 64] = reinterpret_cast<float (*)[MERGE * 64]>(&vt_lds[0][0]);

  const int s = blockIdx.x;
  const int rt = blockIdx.y % nrt;
  const int bg = blockIdx.y / nrt;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const BatchSpan sp = batch_span(a, b);
  const TileSpan ts = tile_span(a, sp, rows, rt);
  const int c_lo = ts.lo + s * chunk;
  const int c_hi = min(ts.hi, c_lo + chunk - 1);
  if (c_lo > c_hi) return;  // nothing in this split (the combine skips it)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 15;
  const int q4 = lane >> 4;

  // this lane's query row (padding rows carry zeros and are never stored)
  const int my_r = kRowsPerTile * rt + n;
  const bool row_ok = my_r < rows;
  const int my_t = row_ok ? my_r / a.G : 0;
  const int my_h = g * a.G + (row_ok ? my_r % a.G : 0);
  const int my_p = sp.q_off + my_t;
  const int lo_eff = max(row_lo(a, my_p), c_lo);
  const int hi_eff = min(row_hi(a, my_p, sp.valid), c_hi);
  const int p_first = sp.q_off + (kRowsPerTile * rt) / a.G;
  const int p_last = sp.q_off + (min(rows, kRowsPerTile * rt + kRowsPerTile) - 1) / a.G;

  u32x4 qf[KQ];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + b * a.q_sb + my_h * a.q_sh +
                         (int64_t)my_t * a.q_ss + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[ks] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * ks) : z;
    }
  }
  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + b * a.k_sb + g * a.k_sh;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + b * a.v_sb + g * a.v_sh;

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float c_l2 = SOFTCAP ? 1.0f : a.scale_log2;

  const int nsub = (c_hi - c_lo + kSub) / kSub;
  const int vdc = lane % CPR, vkg = lane / CPR;
  u32x4 kr[KQ], vr[KPL];
  auto gload = [&](int kb) {
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks) {
      const int j = kb + n;
      u32x4 z = {0u, 0u, 0u, 0u};
      kr[ks] = j <= c_hi ? *reinterpret_cast<const u32x4*>(Kg + (int64_t)j * a.k_ss + 32 * ks + 8 * q4) : z;
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int j = kb + vkg * KPL + i;
      u32x4 z = {0u, 0u, 0u, 0u};
      vr[i] = j <= c_hi ? *reinterpret_cast<const u32x4*>(Vg + (int64_t)j * a.v_ss + 8 * vdc) : z;
    }
  };

  uint16_t* vt = vt_lds[w];
  int sb = w;
  if (sb < nsub) gload(c_lo + kSub * sb);
  for (; sb < nsub; sb += 4) {
    const int kb = c_lo + kSub * sb;
    u32x4 kc[KQ], vc[KPL];
#pragma unroll
    for (int i = 0; i < KQ; ++i) kc[i] = kr[i];
#pragma unroll
    for (int i = 0; i < KPL; ++i) vc[i] = vr[i];
    if (sb + 4 < nsub) gload(kb + 4 * kSub);

    // V -> V^T in this wave's LDS slice
    wave_lds_fence();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * vdc + e;
      uint16_t* dst = vt + d * kVtStride + vkg * KPL;
      uint32_t pk[KPL / 2];
#pragma unroll
      for (int i = 0; i < KPL / 2; ++i) {
        const uint32_t x0 = vc[2 * i][e >> 1], x1 = vc[2 * i + 1][e >> 1];
        pk[i] = (e & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
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
    for (int ks = 0; ks < KQ; ++ks) sc = mma_qk<IS_BF16>(kc[ks], qf[ks], sc);
    if constexpr (SOFTCAP) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = a.cap_log2 * tanh_f32(sc[r] * a.scale_over_cap);
    }
    const bool interior = (a.window < 0 || kb >= p_last - a.window + 1) &&
                          (!a.causal || kb + kSub - 1 <= p_first) && (kb + kSub - 1 <= c_hi);
    if (!interior) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kb + 4 * q4 + r;
        if (j < lo_eff || j > hi_eff) sc[r] = -INFINITY;
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
  if (w != 0) return;
  take(0);

  float l_row = l_run + __shfl_xor(l_run, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  const int rows_tile = min(kRowsPerTile, rows - kRowsPerTile * rt);
  if (n >= rows_tile) return;
  float* part = ws + ((int64_t)(bg * nrt + rt) * nsplit + s) * PART;
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *reinterpret_cast<f32x4*>(part + n * D + 16 * db + 4 * q4) = o[db];
  if (q4 == 0) {
    part[kRowsPerTile * D + n] = m_run == -INFINITY ? -INFINITY : m_run * c_l2;
    part[kRowsPerTile * D + kRowsPerTile + n] = l_row;
  }
}

template <bool IS_BF16, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(AttnArgs a, int rows, int nrt, int chunk,
                                                             int nsplit, const float* __restrict__ ws) {
  constexpr int PART = kRowsPerTile * D + 2 * kRowsPerTile;
  const int rt = blockIdx.x % nrt;
  const int bg = blockIdx.x / nrt;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const BatchSpan sp = batch_span(a, b);
  const TileSpan ts = tile_span(a, sp, rows, rt);
  const int nvalid = ts.lo <= ts.hi ? min(nsplit, (ts.hi - ts.lo) / chunk + 1) : 0;
  const int rows_tile = min(kRowsPerTile, rows - kRowsPerTile * rt);
  const float* base = ws + (int64_t)(bg * nrt + rt) * nsplit * PART;
  for (int idx = threadIdx.x; idx < rows_tile * (D / 4); idx += blockDim.x) {
    const int r = idx / (D / 4);
    const int dq = idx % (D / 4);
    float M = -INFINITY;
    for (int s = 0; s < nvalid; ++s) M = fmaxf(M, base[s * PART + kRowsPerTile * D + r]);
    float L = 0.0f;
    f32x4 acc = f32x4{};
    if (M != -INFINITY) {
      for (int s = 0; s < nvalid; ++s) {
        const float* p = base + s * PART;
        const float f = fast_exp2(p[kRowsPerTile * D + r] - M);
        L += p[kRowsPerTile * D + kRowsPerTile + r] * f;
        const f32x4 x = *reinterpret_cast<const f32x4*>(p + r * D + 4 * dq);
        acc += x * f;
      }
    }
    const int row = kRowsPerTile * rt + r;
    const int t = row / a.G;
    const int h = g * a.G + row % a.G;
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
    uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)t * a.o_ss + 4 * dq;
    *reinterpret_cast<u32x2*>(op) =
        u32x2{pack2<IS_BF16>(acc[0] * fac, acc[1] * fac), pack2<IS_BF16>(acc[2] * fac, acc[3] * fac)};
  }
}

template <bool IS_BF16, int D>
hipError_t launch_t(const AttnArgs& a, bool softcap, const DecodeGeometry& geo, float* ws,
                    hipStream_t stream) {
  dim3 g1(geo.splits, a.B * a.Hkv * geo.row_tiles), block(256);
  if (softcap)
    hipLaunchKernelGGL((decode_split_kernel<IS_BF16, D, true>), g1, block, 0, stream, a, geo.rows,
                       geo.row_tiles, geo.chunk, geo.splits, ws);
  else
    hipLaunchKernelGGL((decode_split_kernel<IS_BF16, D, false>), g1, block, 0, stream, a, geo.rows,
                       geo.row_tiles, geo.chunk, geo.splits, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(a.B * a.Hkv * geo.row_tiles);
  hipLaunchKernelGGL((decode_combine_kernel<IS_BF16, D>), g2, block, 0, stream, a, geo.rows,
                     geo.row_tiles, geo.chunk, geo.splits, (const float*)ws);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(int dtype, int head_size) {
  return (dtype == kBF16 || dtype == kF16) && (head_size == 64 || head_size == 128 || head_size == 256);
}

DecodeGeometry decode_geometry(int B, int Hkv, int G, int curr, int64_t capacity, int window,
                               int causal, int head_size) {
  DecodeGeometry geo;
  geo.rows = G * curr;
  geo.row_tiles = (geo.rows + kRowsPerTile - 1) / kRowsPerTile;
  geo.chunk = 256;
  // longest union range of one row tile: its rows span at most curr positions
  int64_t range = capacity;
  if (causal && window > 0) range = std::min<int64_t>(capacity, (int64_t)window + curr - 1);
  geo.splits = (int)std::max<int64_t>(1, (range + geo.chunk - 1) / geo.chunk);
  geo.ws_floats = (size_t)B * Hkv * geo.row_tiles * geo.splits *
                  (size_t)(kRowsPerTile * head_size + 2 * kRowsPerTile);
  return geo;
}

hipError_t launch_decode_mfma(const AttnArgs& a, int dtype, bool softcap, const DecodeGeometry& geo,
                              float* ws, hipStream_t stream) {
  if (a.B == 0 || a.Lq == 0) return hipSuccess;
  if (dtype == kBF16) {
    if (a.D == 128) return launch_t<true, 128>(a, softcap, geo, ws, stream);
    if (a.D == 256) return launch_t<true, 256>(a, softcap, geo, ws, stream);
    if (a.D == 64) return launch_t<true, 64>(a, softcap, geo, ws, stream);
  } else if (dtype == kF16) {
    if (a.D == 128) return launch_t<false, 128>(a, softcap, geo, ws, stream);
    if (a.D == 256) return launch_t<false, 256>(a, softcap, geo, ws, stream);
    if (a.D == 64) return launch_t<false, 64>(a, softcap, geo, ws, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
