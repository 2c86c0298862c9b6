// Host-side launchers of the gfx950 kernels (internal to libgqa_mi355x).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace gqa {

enum DType { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Any dtype, any head size (multiple of 8, <= 256), prompt or decode mode:
// one wavefront per query row, fp32 throughout.  Writes every output row.
hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t stream);

// Flash-style prompt attention on bf16/fp16 MFMA (32x32x16).  Head sizes 64
// and 128.  Writes every output row.
bool prefill_mfma_supported(int dtype, int head_size);
hipError_t launch_prefill_mfma(const AttnArgs& a, int dtype, bool softcap, hipStream_t stream);

// Split-KV decode on bf16/fp16 MFMA (16x16x32 for QK^T, 16x16x16 for PV):
// one balanced round of workgroups (as many as the device holds at once)
// streams equal slices of the flattened list of 16-key units over all
// (batch, KV head, 16-row tile) row tiles; every piece leaves an fp32
// partial (acc, max, sum) and the last workgroup of each row tile to finish
// merges them, folds the sink and writes O.  Head sizes 64, 128, 256.
// Workspace = per-tile arrival counters (must be zero before the first call;
// every call leaves them zero) followed by the partials.
struct DecodeGeometry {
  int rows;               // G * curr query rows per KV head
  int row_tiles;          // ceil(rows / 16)
  int64_t tiles;          // B * Hkv * row_tiles
  size_t counter_floats;  // leading workspace words holding the arrival counters
  size_t part_floats;     // words of one piece's partial result
  size_t ws_floats;       // workspace words at the largest grid a launch may take
  bool fits;              // tiles within the kernel's per-call limit
};
bool decode_mfma_supported(int dtype, int head_size);
DecodeGeometry decode_geometry(int B, int Hkv, int G, int curr, int head_size);
hipError_t launch_decode_mfma(const AttnArgs& a, int dtype, bool softcap,
                              const DecodeGeometry& geo, float* ws, hipStream_t stream);
// Workspace words the launch above uses on the current device (its resident
// grid instead of the largest one): at most geo.ws_floats.
size_t decode_mfma_scratch_floats(const AttnArgs& a, int dtype, bool softcap, const DecodeGeometry& geo);
constexpr int kDecodeMaxTiles = 2048;  // arrival counters at the front of every decode workspace

// KV-cache append: copy curr rows per (batch, KV head) to slots
// total_b - curr ... total_b - 1 of the cache.
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  int64_t kn_sb, kn_sh, kn_ss;
  int64_t vn_sb, vn_sh, vn_ss;
  int64_t kc_sb, kc_sh, kc_ss;
  int64_t vc_sb, vc_sh, vc_ss;
  const int32_t* seqlens;
  int32_t B, Hkv, curr, row_bytes;
  int32_t capacity;
  int32_t rolling;  // 1: slot = position mod capacity, positions may pass it
  float k_rcp, v_rcp;  // FP8 caches: fp32(1 / scale) of K and V
  const float* k_scales;  // INT8 caches: per-KV-head scales of K and V (device fp32 [Hkv])
  const float* v_scales;
};
hipError_t launch_append_kv(const AppendArgs& a, hipStream_t stream);
// The same into FP8 (E4M3) caches (byte strides for the caches, element
// strides times the element size for the new rows; row_bytes of the new rows).
hipError_t launch_append_kv_fp8(const AppendArgs& a, int dtype, hipStream_t stream);
// The same into INT8 caches with per-KV-head scales (a.k_scales / a.v_scales).
hipError_t launch_append_kv_int8(const AppendArgs& a, int dtype, hipStream_t stream);

// Rotary position embedding: up to three jobs in one launch (blockIdx.y),
// each turning (turn = 1) or copying (turn = 0) rows [B, H[j], L, D] of
// src[j] into dst[j].  Row l of batch b sits at position pos0 + l, or, when
// seqlens is set (a decode step of L = curr tokens), at seqlens[b] + 1 - L + l,
// batches whose length falls outside [L, capacity] being skipped; to_slot[j]
// writes it to the row of its position instead of row l.  Strides are in
// elements; tables are fp32 [max_pos, D/2].
struct RotaryArgs {
  const void* src[3];
  void* dst[3];
  int64_t s_sb[3], s_sh[3], s_ss[3];
  int64_t d_sb[3], d_sh[3], d_ss[3];
  int32_t H[3];
  int32_t turn[3];
  int32_t to_slot[3];
  int32_t jobs;
  int32_t B, L, D;
  int64_t pos0;
  const int32_t* seqlens;
  int32_t capacity;
  int32_t rolling;            // step mode: slot = position mod capacity, positions may pass it
  const float* cos;
  const float* sin;
  int64_t max_pos;
};
hipError_t launch_rotary(const RotaryArgs& a, int dtype, hipStream_t stream);

}  // namespace gqa
