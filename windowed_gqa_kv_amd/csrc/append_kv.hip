// KV-cache append: present = concat(past, step).
//
// Row t of the step goes to cache slot total_b - curr + t with total_b =
// seqlens_k[b] + 1 (the cache as the concatenation of past and step, "onnx:
// import GroupQueryAttention decode steps and its internal rotary", section
// "What changed"; decode positions (total - curr) + i, "[NPUW] Support GQA
// sliding-window and smooth-softmax in DecomposeGQA", section "Sliding window
// (local_window_size)"); a rolling cache (the same page: sliding_window_cache)
// keeps position p in slot p mod capacity.  One thread moves 16 bytes;
// blockIdx.y selects K or V.
#include "kernels.h"

namespace gqa {
namespace {

// I is the index type: 32-bit when the B * Hkv * curr * chunk count fits it.
template <typename I>
__global__ __launch_bounds__(256) void append_kv_kernel(AppendArgs a) {
  const I chunks = a.row_bytes / 16;
  const I n = (I)a.B * a.Hkv * a.curr * chunks;
  const I idx = (I)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int c = (int)(idx % chunks);
  I r = idx / chunks;
  const int t = (int)(r % (I)a.curr);
  r /= (I)a.curr;
  const int g = (int)(r % (I)a.Hkv);
  const int b = (int)(r / (I)a.Hkv);
  const bool is_v = blockIdx.y == 1;
  // strides are in bytes here (converted by the host launcher)
  const char* src = reinterpret_cast<const char*>(is_v ? a.v_new : a.k_new);
  const int64_t so = is_v ? (b * a.vn_sb + g * a.vn_sh + t * a.vn_ss)
                          : (b * a.kn_sb + g * a.kn_sh + t * a.kn_ss);
  // the new row does not depend on the length: both loads are in flight together
  const u32x4 x = *reinterpret_cast<const u32x4*>(src + so + 16 * c);
  const int64_t total = (int64_t)a.seqlens[b] + 1;
  asm volatile("" ::"v"(x));
  if (total < a.curr || (!a.rolling && total > a.capacity)) return;  // out-of-range length: skip batch
  int64_t slot = total - a.curr + t;
  if (a.rolling) slot %= a.capacity;  // a rolling cache: the position's ring slot
  char* dst = reinterpret_cast<char*>(is_v ? a.v_cache : a.k_cache);
  const int64_t dof = is_v ? (b * a.vc_sb + g * a.vc_sh + slot * a.vc_ss)
                           : (b * a.kc_sb + g * a.kc_sh + slot * a.kc_ss);
  *reinterpret_cast<u32x4*>(dst + dof + 16 * c) = x;
}

// FP8 (E4M3) cache: each thread turns 8 elements of a new row (x * r in fp32,
// r = fp32(1 / scale) from the host) into 8 codes, nearest even, saturating at
// +-448 (the hardware conversion turns overflow into NaN, so the value is
// clamped first; a NaN input gives the code 0x7F).
template <int DT>
__device__ __forceinline__ void load8f(const char* p, float (&f)[8]) {
  if constexpr (DT == kF32) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3]; f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
  } else {
    const u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = half_to_f32<DT == kBF16>((uint16_t)(x[i] & 0xffffu));
      f[2 * i + 1] = half_to_f32<DT == kBF16>((uint16_t)(x[i] >> 16));
    }
  }
}
__device__ __forceinline__ uint32_t e4m3_pack4(const float* t) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(t[i], -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);  // bytes 0, 1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);        // bytes 2, 3
  uint32_t u = (uint32_t)w;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (t[i] != t[i]) u = (u & ~(0xffu << (8 * i))) | (0x7fu << (8 * i));
  return u;
}

// INT8 cache: code = x * r in fp32 (r = fp32(1 / scale[g]), a correctly
// rounded division), rounded to the nearest integer with ties to even,
// clamped to +-127; NaN gives 0.
__device__ __forceinline__ uint32_t i8_pack4(const float* t) {
  uint32_t u = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float c = t[i] != t[i] ? 0.0f : fminf(fmaxf(__builtin_rintf(t[i]), -127.0f), 127.0f);
    u |= ((uint32_t)(int)c & 0xffu) << (8 * i);
  }
  return u;
}

// QK = 1: FP8 (E4M3) codes with per-tensor scales; QK = 2: INT8 codes with
// per-KV-head scales.
template <int DT, int QK, typename I>
__global__ __launch_bounds__(256) void append_kv_q8_kernel(AppendArgs a) {
  constexpr int E = DT == kF32 ? 4 : 2;
  const int chunks = a.row_bytes / (8 * E);  // 8-element chunks per row
  const I n = (I)a.B * a.Hkv * a.curr * chunks;
  const I idx = (I)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int c = (int)(idx % (I)chunks);
  I r = idx / (I)chunks;
  const int t = (int)(r % (I)a.curr);
  r /= (I)a.curr;
  const int g = (int)(r % (I)a.Hkv);
  const int b = (int)(r / (I)a.Hkv);
  const bool is_v = blockIdx.y == 1;
  const char* src = reinterpret_cast<const char*>(is_v ? a.v_new : a.k_new);
  const int64_t so = is_v ? (b * a.vn_sb + g * a.vn_sh + t * a.vn_ss) : (b * a.kn_sb + g * a.kn_sh + t * a.kn_ss);
  float f[8];
  load8f<DT>(src + so + 8 * E * c, f);
  const int64_t total = (int64_t)a.seqlens[b] + 1;
  if (total < a.curr || (!a.rolling && total > a.capacity)) return;  // out-of-range length: skip batch
  int64_t slot = total - a.curr + t;
  if (a.rolling) slot %= a.capacity;
  const float rr = QK == 1 ? (is_v ? a.v_rcp : a.k_rcp) : 1.0f / (is_v ? a.v_scales : a.k_scales)[g];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] *= rr;
  char* dst = reinterpret_cast<char*>(is_v ? a.v_cache : a.k_cache);
  const int64_t dof = is_v ? (b * a.vc_sb + g * a.vc_sh + slot * a.vc_ss) : (b * a.kc_sb + g * a.kc_sh + slot * a.kc_ss);
  if constexpr (QK == 1)
    *reinterpret_cast<u32x2*>(dst + dof + 8 * c) = u32x2{e4m3_pack4(f), e4m3_pack4(f + 4)};
  else
    *reinterpret_cast<u32x2*>(dst + dof + 8 * c) = u32x2{i8_pack4(f), i8_pack4(f + 4)};
}

template <int QK>
hipError_t launch_q8(const AppendArgs& a, int dtype, hipStream_t stream) {
  const int E = dtype == kF32 ? 4 : 2;
  const int64_t n = (int64_t)a.B * a.Hkv * a.curr * (a.row_bytes / (8 * E));
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256), 2);
  const bool small = n + 255 <= (int64_t)UINT32_MAX;
  if (dtype == kBF16) {
    if (small) hipLaunchKernelGGL((append_kv_q8_kernel<kBF16, QK, uint32_t>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((append_kv_q8_kernel<kBF16, QK, int64_t>), grid, dim3(256), 0, stream, a);
  } else if (dtype == kF16) {
    if (small) hipLaunchKernelGGL((append_kv_q8_kernel<kF16, QK, uint32_t>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((append_kv_q8_kernel<kF16, QK, int64_t>), grid, dim3(256), 0, stream, a);
  } else if (dtype == kF32) {
    if (small) hipLaunchKernelGGL((append_kv_q8_kernel<kF32, QK, uint32_t>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((append_kv_q8_kernel<kF32, QK, int64_t>), grid, dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_kv_fp8(const AppendArgs& a, int dtype, hipStream_t stream) {
  return launch_q8<1>(a, dtype, stream);
}

hipError_t launch_append_kv_int8(const AppendArgs& a, int dtype, hipStream_t stream) {
  return launch_q8<2>(a, dtype, stream);
}

hipError_t launch_append_kv(const AppendArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.B * a.Hkv * a.curr * (a.row_bytes / 16);
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256), 2);
  if (n + 255 <= (int64_t)UINT32_MAX)
    hipLaunchKernelGGL(append_kv_kernel<uint32_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kv_kernel<int64_t>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gqa
