// KV-cache append: present = concat(past, step).
//
// Row t of the step goes to cache slot total_b - curr + t with total_b =
// seqlens_k[b] + 1 (the cache as the concatenation of past and step, "onnx:
// import GroupQueryAttention decode steps and its internal rotary", section
// "What changed"; decode positions (total - curr) + i, "[NPUW] Support GQA
// sliding-window and smooth-softmax in DecomposeGQA", section "Sliding window
// (local_window_size)").  One thread moves 16 bytes; blockIdx.y selects K or V.
#include "kernels.h"

namespace gqa {
namespace {

__global__ __launch_bounds__(256) void append_kv_kernel(AppendArgs a) {
  const int chunks = a.row_bytes / 16;
  const int64_t n = (int64_t)a.B * a.Hkv * a.curr * chunks;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int c = (int)(idx % chunks);
  int64_t r = idx / chunks;
  const int t = (int)(r % a.curr);
  r /= a.curr;
  const int g = (int)(r % a.Hkv);
  const int b = (int)(r / a.Hkv);
  const int64_t total = (int64_t)a.seqlens[b] + 1;
  if (total < a.curr || total > a.capacity) return;  // out-of-range length: skip batch
  const int64_t slot = total - a.curr + t;
  const bool is_v = blockIdx.y == 1;
  const char* src = reinterpret_cast<const char*>(is_v ? a.v_new : a.k_new);
  char* dst = reinterpret_cast<char*>(is_v ? a.v_cache : a.k_cache);
  // strides are in bytes here (converted by the host launcher)
  const int64_t so = is_v ? (b * a.vn_sb + g * a.vn_sh + t * a.vn_ss)
                          : (b * a.kn_sb + g * a.kn_sh + t * a.kn_ss);
  const int64_t dof = is_v ? (b * a.vc_sb + g * a.vc_sh + slot * a.vc_ss)
                           : (b * a.kc_sb + g * a.kc_sh + slot * a.kc_ss);
  const u32x4 x = *reinterpret_cast<const u32x4*>(src + so + 16 * c);
  *reinterpret_cast<u32x4*>(dst + dof + 16 * c) = x;
}

}  // namespace

hipError_t launch_append_kv(const AppendArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.B * a.Hkv * a.curr * (a.row_bytes / 16);
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256), 2);
  hipLaunchKernelGGL(append_kv_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gqa
