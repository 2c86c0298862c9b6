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

}  // namespace

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
