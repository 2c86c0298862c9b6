// Generic attention kernel: any element type, any head size up to 256.
//
// One wavefront per query row; lanes own keys while scoring and own head
// dimensions while accumulating P*V.  Only keys inside the row's allowed
// interval [lo, hi] are ever read, so stale or padded slots cannot leak into
// the result.  The streaming recurrence (running max, denominator and
// unnormalized output per row, one key block at a time) is the streaming path
// of "Attention Kernel Design", section "Compute paths"; accumulation is fp32
// and only the final output is narrowed (section "Scheduling, precision, and
// invariants").  It serves fp32, head sizes the MFMA kernels do not cover,
// any row count, and calls with a caller mask (boolean or additive, "Attention
// Kernel Design", sections "Layouts and semantics" and "Compute paths"): each
// lane reads the mask entry of its key, and a 64-key block in which no key is
// left is skipped whole (no K or V reads), the all-false block skipping of
// the streaming path.
#include "kernels.h"

namespace gqa {
namespace {

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
  if constexpr (DT == kF32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    u32x4 r = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = half_to_f32<DT == kBF16>((uint16_t)(r[i] & 0xffffu));
      x[2 * i + 1] = half_to_f32<DT == kBF16>((uint16_t)(r[i] >> 16));
    }
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t off) {
  if constexpr (DT == kF32) return reinterpret_cast<const float*>(base)[off];
  else return half_to_f32<DT == kBF16>(reinterpret_cast<const uint16_t*>(base)[off]);
}

template <int DT>
__device__ __forceinline__ void store1(void* base, int64_t off, float x) {
  if constexpr (DT == kF32) {
    reinterpret_cast<float*>(base)[off] = x;
  } else {
    uint32_t pk = pack2<DT == kBF16>(x, 0.0f);
    reinterpret_cast<uint16_t*>(base)[off] = (uint16_t)(pk & 0xffffu);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + w;  // query row
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  if (i >= a.Lq) return;
  const int g = h / a.G;
  const BatchSpan sp = batch_span(a, b);
  const int p = sp.q_off + i;
  const int lo = row_lo(a, p);
  const int hi = row_hi(a, p, sp.valid);
  const bool capped = a.cap_log2 > 0.0f;

  const int64_t q_off = b * a.q_sb + h * a.q_sh + (int64_t)i * a.q_ss;
  const int64_t k_base = b * a.k_sb + g * a.k_sh;
  const int64_t v_base = b * a.v_sb + g * a.v_sh;

  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // head dims lane + 64 c
  float m = -INFINITY, l = 0.0f;
  bool seen = false;  // some key of the row was kept
  const int64_t m_row = b * a.m_sb + h * a.m_sh + (int64_t)i * a.m_sq;
  for (int kb = lo; kb <= hi; kb += 64) {
    const int j = kb + lane;
    bool keep = j <= hi;
    float bias = 0.0f;
    if (a.mask_kind != 0) {
      if (keep) {
        if (a.mask_kind == 1) {
          keep = reinterpret_cast<const uint8_t*>(a.mask)[m_row + j] != 0;
        } else {
          bias = reinterpret_cast<const float*>(a.mask)[m_row + j];
          keep = bias > -INFINITY;
        }
      }
      if (__ballot(keep) == 0) continue;  // no key left in this block: skip it
    }
    seen = true;
    float t = -INFINITY;
    if (keep) {
      float dot = 0.0f;
      for (int d0 = 0; d0 < a.D; d0 += 8) {
        float kx[8], qx[8];
        load8<DT>(a.k, k_base + (int64_t)slot_of(a, j) * a.k_ss + d0, kx);
        load8<DT>(a.q, q_off + d0, qx);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(qx[e], kx[e], dot);
      }
      t = capped ? a.cap_log2 * tanh_f32(dot * a.scale_over_cap + bias * a.inv_cap)
                 : dot * a.scale_log2 + bias * kLog2e;
    }
    const float m_new = fmaxf(m, wave_max(t));  // finite: the block holds >= 1 key
    const float alpha = fast_exp2(m - m_new);    // 0 on the first block
    const float pj = keep ? fast_exp2(t - m_new) : 0.0f;
    l = l * alpha + wave_sum(pj);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] *= alpha;
    const int nk = min(64, hi - kb + 1);
    for (int jj = 0; jj < nk; ++jj) {
      const float pv = __shfl(pj, jj, 64);
      if (a.mask_kind != 0 && pv == 0.0f) continue;  // a masked key (wave-uniform)
      const int64_t vrow = v_base + (int64_t)slot_of(a, kb + jj) * a.v_ss;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d = lane + 64 * c;
        if (d < a.D) acc[c] = fmaf(pv, load1<DT>(a.v, vrow + d), acc[c]);
      }
    }
    m = m_new;
  }

  float fac;
  if (lo > hi || !seen) {
    fac = 0.0f;  // no allowed key: exactly zero, with or without a sink
  } else if (a.use_sink) {
    const float ts = sink_log2(a, h);
    const float M = fmaxf(m, ts);
    const float e1 = fast_exp2(m - M);
    fac = e1 / (l * e1 + fast_exp2(ts - M));
  } else {
    fac = 1.0f / l;
  }
  const int64_t o_off = b * a.o_sb + h * a.o_sh + (int64_t)i * a.o_ss;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d = lane + 64 * c;
    if (d < a.D) store1<DT>(a.o, o_off + d, acc[c] * fac);
  }
}

}  // namespace

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t stream) {
  dim3 grid((a.Lq + 3) / 4, a.Hq, a.B);
  dim3 block(256);
  switch (dtype) {
    case kF32: hipLaunchKernelGGL(attn_generic_kernel<kF32>, grid, block, 0, stream, a); break;
    case kF16: hipLaunchKernelGGL(attn_generic_kernel<kF16>, grid, block, 0, stream, a); break;
    case kBF16: hipLaunchKernelGGL(attn_generic_kernel<kBF16>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqa
