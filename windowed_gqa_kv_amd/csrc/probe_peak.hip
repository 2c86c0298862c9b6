// Measurement aid (not part of the attention path): the dense bf16 matrix
// rate and the shader clock of the device, measured rather than quoted.
//
// Every wave issues `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16
// on register operands (no memory traffic), and stamps the shader-clock
// counter (s_memtime) and the fixed 100 MHz counter (s_memrealtime) before
// and after.  The launch's FLOPs over its event time give the rate; the two
// counters' ratio gives the clock the waves ran at.
#include "gqa_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, unsigned long long* stamps, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  // the results are used (kept from being removed), and the stamps wait for them
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][15];
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  const int wave = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (lane == 0) {
    stamps[4 * wave + 0] = t0;
    stamps[4 * wave + 1] = t1;
    stamps[4 * wave + 2] = r0;
    stamps[4 * wave + 3] = r1;
    sink[wave] = s;
  }
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int gqa_probe_mfma_peak(int blocks, int iters, void* stamps,
                                                                          void* sink, void* hip_stream) {
  if (blocks < 1 || iters < 1 || stamps == nullptr || sink == nullptr) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream), iters,
                     reinterpret_cast<unsigned long long*>(stamps), reinterpret_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
