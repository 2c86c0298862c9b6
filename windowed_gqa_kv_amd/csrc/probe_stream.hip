// Measurement aid (not part of the attention path): the rate at which the
// decode's own loading scheme streams a set of K/V units with no attention
// work, the ceiling the split-KV decode is measured against.
//
// A unit is 16 key rows of RB bytes (256 at head size 128, 512 at 256, with
// 16-bit elements) of K and the same rows of V, at a byte offset the caller
// lists.  The units are cut evenly over the workgroups; wave w of a
// workgroup takes its slice's units w, w + 4, ...  Each wave streams its
// units through two LDS stages of one K and one V unit by LDS DMA (16 bytes
// a lane, non-temporal, the decode's chunk swizzle), waits for a unit as the
// decode does, reads one word of it and refills the stage.  64 KB of LDS per
// workgroup at 256-byte rows (two workgroups per CU) and 128 KB at 512-byte
// rows (one), as in the decode at those head sizes.
#include "gqa_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

constexpr int kStages = 2;
constexpr int kMaxPerBlock = 256;     // units per workgroup slice

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int RB>
__global__ __launch_bounds__(256) void kv_stream_probe_kernel(const char* __restrict__ K, const char* __restrict__ V,
                                                              int64_t kv_bytes, const int64_t* __restrict__ unit_off,
                                                              int U, float* sink) {
  constexpr int kUnitBytes = 16 * RB;  // one unit of K (or V)
  constexpr int kChunks = RB / 16;     // 16-byte chunks per row
  __shared__ __attribute__((aligned(1024))) unsigned char ring[4][kStages][2 * kUnitBytes];
  __shared__ int64_t offs[kMaxPerBlock];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, k = blockIdx.x;
  const int ua = (int)((int64_t)U * k / G), ub = (int)((int64_t)U * (k + 1) / G);
  const int n = ub - ua;  // <= kMaxPerBlock (checked by the host)
  if (tid < n) {
    int64_t off = unit_off[ua + tid];
    // an offset whose unit would leave either buffer reads the first unit
    offs[tid] = (off < 0 || off > kv_bytes - kUnitBytes) ? 0 : off;
  }
  __syncthreads();
  const int nw = n > w ? (n - w + 3) / 4 : 0;
  auto issue = [&](int s, int j) {
    const int64_t off = offs[w + 4 * j];
    unsigned char* kd = &ring[w][s][0];
#pragma unroll
    for (int i = 0; i < kUnitBytes / 1024; ++i) {
      const int pos = 64 * i + lane, key = pos / kChunks;
      const int cc = (pos % kChunks) ^ ((2 * key + (key >> 3)) & 15);
      const int64_t go = off + key * RB + 16 * cc;
      __builtin_amdgcn_global_load_lds((global_void*)(K + go), (lds_void*)(kd + 1024 * i), 16, 0, 2);
      __builtin_amdgcn_global_load_lds((global_void*)(V + go), (lds_void*)(kd + kUnitBytes + 1024 * i), 16, 0, 2);
    }
  };
  constexpr int kLoadsPerUnit = 2 * (kUnitBytes / 1024);
  float acc = 0.0f;
  const int npro = nw < kStages ? nw : kStages;
  for (int j = 0; j < npro; ++j) issue(j, j);
  for (int j = 0; j < nw; ++j) {
    if (j + 1 < nw)
      wait_vm<kLoadsPerUnit>();  // the next unit may stay in flight
    else
      wait_vm<0>();
    const uint32_t a = (uint32_t)(uintptr_t)(lds_void*)(&ring[w][j % kStages][0]) + 4 * lane;
    float x;
    // the read and its wait in one statement: the register is final when it ends
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(a) : "memory");
    acc += x;
    if (j + kStages < nw) issue(j % kStages, j + kStages);
  }
  if (acc == 1234.5f) sink[0] = acc;  // keeps the reads; practically never true
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int gqa_probe_kv_stream(int grid, int row_bytes, const void* k,
                                                                          const void* v, int64_t kv_bytes,
                                                                          const int64_t* unit_off, int units,
                                                                          void* sink, void* hip_stream) {
  if (grid < 1 || (row_bytes != 256 && row_bytes != 512) || units < 0 || kv_bytes < 16 * row_bytes ||
      k == nullptr || v == nullptr || sink == nullptr || (units > 0 && unit_off == nullptr))
    return 1;
  if (((int64_t)units + grid - 1) / grid > kMaxPerBlock) return 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const char* kp = reinterpret_cast<const char*>(k);
  const char* vp = reinterpret_cast<const char*>(v);
  float* sp = reinterpret_cast<float*>(sink);
  if (row_bytes == 256)
    hipLaunchKernelGGL(kv_stream_probe_kernel<256>, dim3(grid), dim3(256), 0, st, kp, vp, kv_bytes, unit_off, units, sp);
  else
    hipLaunchKernelGGL(kv_stream_probe_kernel<512>, dim3(grid), dim3(256), 0, st, kp, vp, kv_bytes, unit_off, units, sp);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
