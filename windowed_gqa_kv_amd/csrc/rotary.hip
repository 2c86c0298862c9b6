// Rotary position embedding of Q and of K before it enters the cache ("onnx:
// import GroupQueryAttention decode steps and its internal rotary", section
// "What changed", do_rotary).
//
// Element i of a row pairs with element i + D/2 (the caller's cos and sin
// tables have D/2 columns and serve both halves) and the pair turns by the
// angle of (position, i): (a, b) -> (a c - b s, b c + a s), in fp32, then
// narrowed to the row's type with round-to-nearest-even.  Positions are
// absolute: the prompt's rows sit at pos0 + l, a decode step's new token t of
// batch b at total_b - curr + t (total_b = seqlens_k[b] + 1), which is also
// its cache slot.
//
// A thread turns P pairs: elements i0 .. i0+P-1 and i0+D/2 .. i0+D/2+P-1, 16
// bytes of each half (P = 8 for half-precision rows whose half is a multiple
// of 8 elements, else P = 4: 8 bytes of a half-precision row, 16 of an fp32
// one), and reads P floats of each table.  The work is a few bytes per
// element and bound by HBM (or by launch latency for a decode step); rows are
// independent and consecutive threads cover consecutive chunks of a row, so
// every access is contiguous across the wave.
#include <algorithm>

#include "kernels.h"

namespace gqa {
namespace {

// P consecutive elements of a row to and from fp32 (P = 4 or 8).
template <int DT>
struct Elem;
template <>
struct Elem<kF32> {
  template <int P>
  __device__ static void load(const void* p, float (&f)[P]) {
#pragma unroll
    for (int i = 0; i < P; i += 4) {
      const f32x4 x = reinterpret_cast<const f32x4*>(p)[i / 4];
      f[i] = x[0]; f[i + 1] = x[1]; f[i + 2] = x[2]; f[i + 3] = x[3];
    }
  }
  template <int P>
  __device__ static void store(void* p, const float (&f)[P]) {
#pragma unroll
    for (int i = 0; i < P; i += 4) reinterpret_cast<f32x4*>(p)[i / 4] = f32x4{f[i], f[i + 1], f[i + 2], f[i + 3]};
  }
  static constexpr int kBytes = 4;
};
template <bool IS_BF16>
struct Half {
  template <int P>
  __device__ static void load(const void* p, float (&f)[P]) {
    uint32_t w[P / 2];
    if constexpr (P == 8) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(p);
      w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
    } else {
      const u32x2 x = *reinterpret_cast<const u32x2*>(p);
      w[0] = x[0]; w[1] = x[1];
    }
#pragma unroll
    for (int i = 0; i < P / 2; ++i) {
      f[2 * i] = half_to_f32<IS_BF16>((uint16_t)(w[i] & 0xffffu));
      f[2 * i + 1] = half_to_f32<IS_BF16>((uint16_t)(w[i] >> 16));
    }
  }
  template <int P>
  __device__ static void store(void* p, const float (&f)[P]) {
    if constexpr (P == 8)
      *reinterpret_cast<u32x4*>(p) = u32x4{pack2<IS_BF16>(f[0], f[1]), pack2<IS_BF16>(f[2], f[3]),
                                           pack2<IS_BF16>(f[4], f[5]), pack2<IS_BF16>(f[6], f[7])};
    else
      *reinterpret_cast<u32x2*>(p) = u32x2{pack2<IS_BF16>(f[0], f[1]), pack2<IS_BF16>(f[2], f[3])};
  }
  static constexpr int kBytes = 2;
};
template <>
struct Elem<kBF16> : Half<true> {};
template <>
struct Elem<kF16> : Half<false> {};

// Job j of the launch (blockIdx.y): rows [B, H_j, L] of src_j turned (or
// copied) into dst_j, row l of batch b going to row l (positions pos0 + l),
// or, in a decode step, to the row of its position.
// I is the index type: 32-bit when every job's thread count fits it.
template <int DT, int P, typename I>
__global__ __launch_bounds__(256) void rotary_kernel(RotaryArgs a) {
  using E = Elem<DT>;
  const int j = blockIdx.y;
  const int cpr = a.D / (2 * P);  // P-pair chunks per row
  const I n = (I)a.B * a.H[j] * a.L * cpr;
  const I idx = (I)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int c = (int)(idx % (I)cpr);
  I r = idx / (I)cpr;
  const int l = (int)(r % (I)a.L);
  r /= (I)a.L;
  const int h = (int)(r % (I)a.H[j]);
  const int b = (int)(r / (I)a.H[j]);
  int64_t pos;
  if (a.seqlens != nullptr) {
    const int64_t total = (int64_t)a.seqlens[b] + 1;
    if (total < a.L || (!a.rolling && total > a.capacity)) return;  // out-of-range length: batch skipped
    pos = total - a.L + l;
  } else {
    pos = a.pos0 + l;
  }
  // A position the tables do not cover happens only in a decode step on a
  // rolling cache (positions pass the capacity, and the host cannot see the
  // lengths): a row to be turned is then left unwritten; a copied row (V)
  // needs no table and is written.
  if (a.turn[j] && (pos < 0 || pos >= a.max_pos)) return;
  const int half = a.D / 2;
  const int i0 = P * c;
  const char* src = reinterpret_cast<const char*>(a.src[j]) +
                    E::kBytes * (b * a.s_sb[j] + h * a.s_sh[j] + (int64_t)l * a.s_ss[j]);
  const int64_t drow = a.to_slot[j] ? (a.rolling ? pos % a.capacity : pos) : l;
  char* dst = reinterpret_cast<char*>(a.dst[j]) +
              E::kBytes * (b * a.d_sb[j] + h * a.d_sh[j] + drow * a.d_ss[j]);
  float x[P], y[P];
  E::template load<P>(src + E::kBytes * i0, x);
  E::template load<P>(src + E::kBytes * (i0 + half), y);
  if (a.turn[j]) {
    float cs[P], sn[P];
    Elem<kF32>::load<P>(a.cos + pos * half + i0, cs);
    Elem<kF32>::load<P>(a.sin + pos * half + i0, sn);
    float u[P], w[P];
#pragma unroll
    for (int e = 0; e < P; ++e) rot_pair(x[e], y[e], cs[e], sn[e], u[e], w[e]);
    E::template store<P>(dst + E::kBytes * i0, u);
    E::template store<P>(dst + E::kBytes * (i0 + half), w);
  } else {
    E::template store<P>(dst + E::kBytes * i0, x);
    E::template store<P>(dst + E::kBytes * (i0 + half), y);
  }
}

template <int DT, int P>
hipError_t launch_dt(const RotaryArgs& a, hipStream_t stream) {
  int64_t most = 0;
  for (int j = 0; j < a.jobs; ++j) most = std::max(most, (int64_t)a.B * a.H[j] * a.L * (a.D / (2 * P)));
  if (most == 0) return hipSuccess;
  const int64_t blocks = (most + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, a.jobs);
  if (blocks * 256 <= (int64_t)UINT32_MAX)
    hipLaunchKernelGGL((rotary_kernel<DT, P, uint32_t>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((rotary_kernel<DT, P, int64_t>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotary(const RotaryArgs& a, int dtype, hipStream_t stream) {
  if (a.jobs < 1 || a.jobs > 3 || a.D % 8 != 0) return hipErrorInvalidValue;
  const bool wide = a.D % 16 == 0;  // halves of whole 16-byte chunks
  if (dtype == kBF16) return wide ? launch_dt<kBF16, 8>(a, stream) : launch_dt<kBF16, 4>(a, stream);
  if (dtype == kF16) return wide ? launch_dt<kF16, 8>(a, stream) : launch_dt<kF16, 4>(a, stream);
  if (dtype == kF32) return launch_dt<kF32, 4>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace gqa
