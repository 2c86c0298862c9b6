// Device-side building blocks shared by the gfx950 kernels of libgqa_mi355x.
//
// Everything here is written for CDNA4 (gfx950, wave64).  Element types are
// carried as raw 16-bit storage (bf16 / fp16) or float; arithmetic is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// ---------------------------------------------------------------------------
// Vector types matching the MFMA operand registers.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int32_t kMaxPosition = 1 << 30;  // positions stay in 32-bit arithmetic
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Arguments common to every attention kernel (passed by value).
// Strides are in elements; the head dimension is contiguous.
// mode 0 (prompt):  q_offset = Lk - Lq; valid = nonpad[b] (or Lk).
// mode 1 (decode):  total = seqlens[b] + 1; q_offset = total - Lq; valid = total.
// An out-of-range device length turns that batch's rows into zeros.
// ring > 0 (decode on a rolling cache of `ring` = Lk slots): the key at
// position j lives in slot j mod ring and total may pass the capacity.
// ---------------------------------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  const int64_t* nonpad;   // mode 0, may be null
  const int32_t* seqlens;  // mode 1
  const float* head_sink;  // null: sink logit 0 when use_sink
  int32_t B, Hq, Hkv, G, D;
  int32_t Lq;       // prompt rows, or curr for decode
  int32_t Lk;       // keys in K/V, or cache capacity
  int32_t mode;
  int32_t causal;
  int32_t window;   // -1 = off
  int32_t use_sink;
  int32_t ring;         // 0, or the slot count of a rolling cache (decode)
  // Caller mask over [B, Hq, Lq, Lk] (element strides, 0 broadcasts, keys
  // contiguous; the key index is the position): kind 1 boolean (uint8,
  // nonzero attends), kind 2 additive fp32 (added to the scaled logit
  // before softcap; -inf removes the key).
  const void* mask;
  int64_t m_sb, m_sh, m_sq;
  int32_t mask_kind;    // 0 = none
  float inv_cap;        // 1 / softcap (softcap > 0 only)
  float bias_mul;       // 1 / scale: an additive mask value in raw score units
  // Decode on FP8 (E4M3) caches: k and v hold codes (byte strides), the K
  // scale is folded into scale_log2 / scale_over_cap, the V scale multiplies
  // the normalized output.
  int32_t kv_fp8;       // 1: FP8 (E4M3) caches; 2: INT8 caches with per-KV-head scales
  float v_scale;        // 1 unless FP8
  const float* k_scales;  // INT8: device fp32 [Hkv], folded into the scores per KV head
  const float* v_scales;  // INT8: device fp32 [Hkv], multiplies the normalized output
  float scale_log2;     // scale * log2(e)
  float scale_over_cap; // scale / softcap (softcap > 0 only)
  float cap_log2;       // softcap * log2(e)
  // Decode with the step's append fused in (16-bit caches): the curr new K/V
  // rows of every (batch, KV head) are copied from k_new / v_new to their
  // cache slots, and the decode reads those positions from k_new / v_new
  // themselves (no workgroup reads a slot this launch writes).
  int32_t fuse_append;
  const void* k_new;
  const void* v_new;
  int64_t kn_sb, kn_sh, kn_ss;
  int64_t vn_sb, vn_sh, vn_ss;
  // Prompt with rotary on Q (prefill only): when set, query row i is turned
  // at its position q_offset + i with these fp32 [positions, D/2] tables as
  // it is loaded (K arrives turned).
  const float* rot_cos;
  const float* rot_sin;
};

struct BatchSpan {
  int q_off;  // absolute position of query row 0
  int valid;  // keys [0, valid) exist
};

__device__ __forceinline__ BatchSpan batch_span(const AttnArgs& a, int b) {
  BatchSpan s;
  if (a.mode == 0) {
    int64_t n = a.nonpad ? a.nonpad[b] : (int64_t)a.Lk;
    bool ok = n >= 0 && n <= a.Lk;
    s.valid = ok ? (int)n : 0;
    s.q_off = a.Lk - a.Lq;
  } else {
    int64_t total = (int64_t)a.seqlens[b] + 1;
    bool ok = total >= a.Lq && total <= (a.ring ? (int64_t)kMaxPosition : (int64_t)a.Lk);
    s.valid = ok ? (int)total : 0;
    s.q_off = ok ? (int)(total - a.Lq) : 0;
  }
  return s;
}

// Allowed keys of the query at absolute position p form [lo, hi] (empty when
// lo > hi): every constraint is a half-line in the key index.
__device__ __forceinline__ int row_lo(const AttnArgs& a, int p) {
  return a.window < 0 ? 0 : max(0, p - a.window + 1);
}
__device__ __forceinline__ int row_hi(const AttnArgs& a, int p, int valid) {
  return a.causal ? min(p, valid - 1) : valid - 1;
}

// Cache slot of the key at position j (a rolling cache wraps it).
__device__ __forceinline__ int slot_of(const AttnArgs& a, int j) {
  return a.ring ? j % a.ring : j;
}

// Sink logit of query head h in log2 units.
__device__ __forceinline__ float sink_log2(const AttnArgs& a, int h) {
  return a.head_sink ? a.head_sink[h] * kLog2e : 0.0f;
}

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from the identity tanh(y) = 1 - 2 / (e^{2y} + 1) for |y| >= 1/4, and
// its Taylor series through y^9 below that (truncation < 1e-8 relative there).
__device__ __forceinline__ float tanh_f32(float y) {
  float ay = fabsf(y);
  if (ay < 0.25f) {
    float y2 = y * y;
    float poly = 1.0f + y2 * (-1.0f / 3.0f + y2 * (2.0f / 15.0f +
                 y2 * (-17.0f / 315.0f + y2 * (62.0f / 2835.0f))));
    return y * poly;
  }
  float e = fast_exp2(2.0f * kLog2e * ay);
  float r = 1.0f - 2.0f / (e + 1.0f);
  return copysignf(r, y);
}

// tanh for the matrix-core kernels, whose scores go on to 16-bit P: with
// t = e^{-2|y|} (no overflow), tanh|y| = (1 - t) / (1 + t), where 1 - t is
// exact for t >= 1/2, so small |y| keep their relative accuracy; the hardware
// reciprocal (about 1 ulp) replaces the division.  Absolute error a few 1e-7,
// branch-free.
__device__ __forceinline__ float tanh_fast(float y) {
  const float t = fast_exp2(-2.0f * kLog2e * fabsf(y));
  return copysignf((1.0f - t) * fast_rcp(1.0f + t), y);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 x;
  __builtin_memcpy(&x, &h, 2);
  return (float)x;
}
template <bool IS_BF16>
__device__ __forceinline__ float half_to_f32(uint16_t h) {
  if constexpr (IS_BF16) return bf16_to_f32(h); else return f16_to_f32(h);
}

// Round-to-nearest-even narrowing of a pair (one v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <bool IS_BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (IS_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}

// The rotary turn of one pair (a, b) = (element i, element i + D/2) by the
// angle with cosine c and sine s: (a c - b s, b c + a s), in fp32 with the
// products contracted the same way wherever it is computed (so a turn done
// while loading equals the rotary kernel's bit for bit).
__device__ __forceinline__ void rot_pair(float a, float b, float c, float s, float& u, float& w) {
  u = fmaf(a, c, -(b * s));
  w = fmaf(b, c, a * s);
}

// ---------------------------------------------------------------------------
// Wave-level reductions (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Value of lane l ^ 32 (the other half-wave).
// The value of lane i ^ 32, without an LDS round trip: v_permlane32_swap of x
// with itself leaves the low half's values in both halves of one result and
// the high half's in both halves of the other.
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// The value of lane l ^ 16 (v_permlane16_swap exchanges the odd 16-lane rows
// of one operand with the even rows of the other; with both operands x, a
// lane in an odd row finds its partner in the first result, one in an even
// row in the second).
__device__ __forceinline__ float xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

}  // namespace gqa
