// Flash-style prompt attention on CDNA4 matrix cores (bf16 / fp16 inputs,
// fp32 accumulation), head sizes 32, 64, 128 and 256.
//
// What it computes is the definition in include/gqa.h; the method is the
// streaming path of "Attention Kernel Design" (section "Compute paths": visit
// KV blocks with an online softmax, keep one score tile and per-row running
// max / denominator / unnormalized output; causal and padding frontiers skip
// whole blocks), with the absolute-position window of "[NPUW] Support GQA
// sliding-window and smooth-softmax in DecomposeGQA" (section "Sliding window
// (local_window_size)") as one more frontier and the sink folded into the
// final denominator (same page, section "smooth_softmax / head_sink").
//
// Layout of the work.
//   * Workgroup = 4 waves.  It holds hw query heads of one KV head (hw = the
//     largest power of two dividing G, at most 4) and 4 / hw groups of 32
//     rows of each; wave w owns 32 rows of one head.  All of them read the
//     same keys, so K and V tiles of 64 rows are loaded once per workgroup:
//     from global memory straight into LDS by LDS DMA (global_load_lds_dwordx4,
//     no registers held by loads in flight), double buffered, one barrier per
//     tile.  Two workgroups fit on a CU (one at head size 256, whose tiles
//     take 128 KB of LDS and whose waves use up to 512 registers).
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q held in
//     registers for the whole kernel), so each lane ends up owning one query
//     row and 16 keys of every 32-key sub-tile.  The K rows fed to the MFMA M
//     index are permuted (key_of_m) so that those 16 keys come as two runs of
//     8 consecutive keys -- exactly the B-operand layout the P*V MFMA needs.
//     P therefore goes from the score accumulators to the next MFMA without
//     an LDS round trip.
//   * O^T += V^T P^T on the same MFMA: the A operand (8 consecutive keys of one
//     head-dim column per lane) comes out of the row-major V tile through two
//     transposing LDS reads (ds_read_b64_tr_b16), addressed by per-lane
//     offsets fixed for the whole kernel plus immediates.  K and V rows are
//     stored with XOR-swizzled 16-byte chunks (chosen per lane in the DMA
//     source address), which keeps both read patterns free of bank conflicts.
//   * Operand reads are batched (four K operands, or the four V operands of one
//     16-key step, per wait) and issued one batch ahead of the MFMAs that use
//     them; the next tile's DMA loads are spread over the K batches.  Every
//     tile a wave can see takes one branch-free path; sub-tiles outside all of
//     its rows' bands are masked like any other excluded key.
//   * Online softmax in fp32 with exp2, the scale folded into one FMA, a lazy
//     rescale (the running max only moves when it grows by more than 2^8, on
//     a real branch), masks evaluated only on boundary sub-tiles, and pairs
//     narrowed by one conversion each.  The vector work per tile is the floor
//     of the method: the two contractions and their softmax take about the
//     same issue time per wave.
//   * Work items are ordered (batch, KV head)-major so that the workgroups of
//     one KV head land on the same XCD (its own L2), heaviest row blocks
//     first within each KV head.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace gqa {
namespace {

constexpr int kWaves = 4;   // waves per workgroup (two workgroups per CU)
constexpr int NSTAGE = 2;   // K/V tiles in LDS: the current one and the next
constexpr int BN = 64;   // keys per LDS tile
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

template <bool IS_BF16>
__device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (IS_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// MFMA M index -> key within a 32-key sub-tile.  With m = 8a + 4h + c the
// accumulator register r = 4a + c of lane half h then holds key
// 16*(r/8) + 8h + r%8: two runs of 8 consecutive keys per lane.
__device__ __forceinline__ int key_of_m(int m) {
  const int a = m >> 3, hh = (m >> 2) & 1, c = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + c;
}
// XOR swizzle of the 16-byte chunks of K row r: the 16 rows one operand read
// touches per 16 lanes land on 16 different bank groups.
template <int D>
__host__ __device__ constexpr int k_swz(int r) {
  if constexpr (D >= 128)
    return r & 15;  // 16 (or 32) chunks per row
  else if constexpr (D == 64)
    return (r >> 1) & 7;
  else
    return (r >> 2) & 3;  // 4 chunks per row: rows r and r + 4 share banks
}
// V tile rows (row-major, 16-byte chunks XOR-swizzled by key): the
// transposing reads of the P*V operand then hit every bank equally.
template <int D>
__host__ __device__ constexpr int vrow_swz(int key) {
  if constexpr (D >= 128)
    return 4 * (key & 3);
  else if constexpr (D == 64)
    return 4 * ((key >> 1) & 1);
  else
    return 0;  // one 32-column block: the four rows of a read are 256 contiguous bytes
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Operand reads of the DMA-filled tiles are ordinary LDS loads, tracked by
// the compiler: it places the lgkmcnt wait in front of each value's first use
// and may keep, copy or spill the results like any other value.  All DMA
// loads are inline assembly, which the compiler does not see as LDS writes,
// so it puts no wait for them in front of these reads; a tile's DMA is waited
// for explicitly (wait_vm, then the workgroup barrier) before its stage is
// read, and the barrier is a compiler memory barrier, so no read moves across
// it.  The reads are issued one batch ahead of the MFMAs that use them (the
// source order is the pipeline).
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(const lds_u8* base, uint32_t off) {
  return *reinterpret_cast<const lds_u32x4*>(base + off + OFF);
}
// One transposing read (ds_read_b64_tr_b16): 4 16-bit values of one column,
// from the 4 rows whose addresses the lanes of each group of four hold.
template <int OFF>
__device__ __forceinline__ uint64_t lds_tr16(const lds_u8* base, uint32_t off) {
  return __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                          const_cast<lds_i16x4*>(reinterpret_cast<const lds_i16x4*>(base + off + OFF))));
}
// One wave-wide LDS DMA load (16 bytes per lane, 1 KB in all) from the
// uniform base sbase plus this lane's 32-bit byte offset voff, to the LDS
// bytes at lds_addr + 16 * lane.  The scalar-base form keeps the tile's base
// address off the vector ALU.  The compiler does not see it as a memory
// load: the callers wait for it with explicit vmcnt waits.
__device__ __forceinline__ void dma_saddr(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  // M0 (the LDS destination) is an input operand, so the compiler sets it
  // and knows its value afterwards
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
// The same from a per-lane 64-bit address (rows clamped per lane).
__device__ __forceinline__ void dma_vaddr(const void* addr, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(addr), "{m0}"(lds_addr) : "memory");
}
// Barrier between tiles: wait for this wave's LDS operations, then meet.  A
// fenced barrier would also wait for the next tile's DMA loads, which count as
// LDS writes; the empty asm statements keep the compiler from moving LDS
// reads across the barrier instead.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Caller-mask bytes are read through global-address-space pointers: generic
// (flat) loads would also count against lgkmcnt, which the LDS operand reads
// wait on by count.
typedef __attribute__((address_space(1))) const uint64_t global_u64;
typedef __attribute__((address_space(1))) const unsigned char global_u8;
typedef __attribute__((address_space(1))) const f32x4 global_f32x4;
typedef __attribute__((address_space(1))) const float global_f32;

// Two waves per SIMD (two workgroups per CU): the register budget is 256;
// at head size 256 one wave per SIMD with up to 512.
// MASK = 1: a caller boolean mask (uint8, nonzero attends) over [B, Hq, Lq, Lk];
// MASK = 2: a caller additive mask (fp32, added to the scaled logit).
template <bool IS_BF16, int D, bool SOFTCAP, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2))) void prefill_mfma_kernel(
    AttnArgs a, int nrb, int items, int per_xcd, int hw) {
  constexpr int KS = D / 16;    // k-steps of the QK^T contraction
  constexpr int DB = D / 32;    // 32-wide output blocks
  constexpr int CPR = D / 8;    // 16-byte chunks per K row
  constexpr int TILE = BN * D;  // elements of one K (or V) tile
  // K tiles of both stages, then V tiles of both stages: every operand read of
  // either stage is a per-lane base register plus an immediate below 64 KB
  // (with K and V interleaved per stage, stage 1 of head size 256 starts
  // 64 KB in, past the offset field, and each read needed an address add).
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][NSTAGE][TILE];

  // ---- work item: XCD-major, KV-head-major, heavy row blocks first ----
  // A workgroup holds hw query heads of one KV head (hw divides G, at most 4)
  // and 4 / hw groups of 32 rows of each: all its waves share every K/V tile.
  const int id = blockIdx.x;
  const int item = (id & 7) * per_xcd + (id >> 3);
  if (item >= items) return;
  const int ngrp = a.G / hw;  // head groups per KV head
  const int per_bg = ngrp * nrb;
  const int bg = item / per_bg;
  const int rem = item - bg * per_bg;
  const int rb = nrb - 1 - rem / ngrp;
  const int hg = rem % ngrp;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 31;
  const int h2 = lane >> 5;
  const int h = g * a.G + hg * hw + w % hw;  // this wave's query head
  const int rpw = 32 * (kWaves / hw);        // rows of each head in this workgroup

  const BatchSpan sp = batch_span(a, b);
  const int row0 = rb * rpw;
  const int rows_here = min(rpw, a.Lq - row0);
  // With a caller mask the first tile starts at a multiple of 64 keys, so that
  // the mask runs below are aligned (keys before the band are masked like any
  // other excluded key).
  const int kv_lo = MASK ? (row_lo(a, sp.q_off + row0) & ~(BN - 1)) : row_lo(a, sp.q_off + row0);
  const int kv_hi = row_hi(a, sp.q_off + row0 + rows_here - 1, sp.valid);

  const int wrow0 = row0 + 32 * (w / hw);
  const int wrows = min(32, a.Lq - wrow0);  // may be <= 0
  const int pw0 = sp.q_off + wrow0;
  const int pw1 = pw0 + max(wrows, 1) - 1;
  const int w_lo = row_lo(a, pw0);
  const int w_hi = row_hi(a, pw1, sp.valid);
  const int my_row = wrow0 + n;
  const int my_p = sp.q_off + my_row;
  const int my_lo = row_lo(a, my_p);
  const int my_hi = row_hi(a, my_p, sp.valid);

  const uint16_t* __restrict__ Kg = reinterpret_cast<const uint16_t*>(a.k) + b * a.k_sb + g * a.k_sh;
  const uint16_t* __restrict__ Vg = reinterpret_cast<const uint16_t*>(a.v) + b * a.v_sb + g * a.v_sh;

  // Q rows stay in registers (B operand of S^T = K Q^T).
  u32x4 qf[KS];
  const bool rot = a.rot_cos != nullptr;
  f32x4 rc[KS / 2][2], rs[KS / 2][2];  // rotary angles of the row (cos, sin), when rot
  {
    const bool ok = my_row < a.Lq;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + b * a.q_sb + h * a.q_sh +
                         (int64_t)(ok ? my_row : 0) * a.q_ss + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[ks] = ok ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : z;
    }
    // Rotary on Q: the lane's elements i of k-step ks < KS/2 and their
    // partners i + D/2 of k-step ks + KS/2 turn by the angles of the row's
    // position (the rotary kernel's arithmetic, then RNE to the input type).
    // The angles are loaded with Q; the turn waits until the first tile's
    // DMA is on its way.
    if (rot && ok && my_p >= 0) {
      const float* cr = a.rot_cos + (int64_t)my_p * (D / 2) + 8 * h2;
      const float* sr = a.rot_sin + (int64_t)my_p * (D / 2) + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) {
        rc[ks][0] = *reinterpret_cast<const f32x4*>(cr + 16 * ks);
        rc[ks][1] = *reinterpret_cast<const f32x4*>(cr + 16 * ks + 4);
        rs[ks][0] = *reinterpret_cast<const f32x4*>(sr + 16 * ks);
        rs[ks][1] = *reinterpret_cast<const f32x4*>(sr + 16 * ks + 4);
      }
    }
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // raw-score units (log2 units with a softcap)
  float l_run = 0.0f;       // partial sum over this lane's keys

  const int nblk = kv_lo <= kv_hi ? (kv_hi - kv_lo + BN) / BN : 0;

  // K and V tiles go from global memory straight into LDS (LDS DMA, 1 KB per
  // wave-wide instruction).  Both are row-major with XOR-swizzled 16-byte
  // chunks; lane L of instruction i writes position 64 i + L, so it loads the
  // global chunk that the swizzle puts there.  The per-lane source offsets
  // within a tile are the same for every tile; only the tile's base address
  // (wave-uniform) moves.  In the last tile, rows past kv_hi are clamped to
  // kv_hi: real, finite keys that the masks remove for every row.
  constexpr int NDMA = TILE * 2 / 1024 / kWaves;  // per wave, per tile, per tensor
  constexpr int RPI = 64 / CPR;              // tile rows per DMA instruction
  const int64_t krow_b = a.k_ss * 2, vrow_b = a.v_ss * 2;
  uint32_t koff[NDMA], voff[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = RPI * (NDMA * w + i) + lane / CPR, slot = lane % CPR;
    koff[i] = (uint32_t)(r * krow_b) + 16 * (slot ^ k_swz<D>(r));
    voff[i] = (uint32_t)(r * vrow_b) + 16 * (slot ^ vrow_swz<D>(r));
  }
  // instruction pair i (one K and one V load) of this wave's share of a tile
  auto dma_part = [&](int kb, int buf, int i) {
    uint16_t* kdst = &lds[0][buf][0] + 512 * (NDMA * w + i);
    uint16_t* vdst = &lds[1][buf][0] + 512 * (NDMA * w + i);
    if (kb + BN - 1 <= kv_hi) {
      const char* kbase = reinterpret_cast<const char*>(Kg) + kb * krow_b;
      const char* vbase = reinterpret_cast<const char*>(Vg) + kb * vrow_b;
      dma_saddr(kbase, koff[i], (uint32_t)(uintptr_t)(lds_void*)kdst);
      dma_saddr(vbase, voff[i], (uint32_t)(uintptr_t)(lds_void*)vdst);
    } else {
      const int r = RPI * (NDMA * w + i) + lane / CPR, slot = lane % CPR;
      const int j = min(kb + r, kv_hi);
      dma_vaddr(Kg + (int64_t)j * a.k_ss + 8 * (slot ^ k_swz<D>(r)), (uint32_t)(uintptr_t)(lds_void*)kdst);
      dma_vaddr(Vg + (int64_t)j * a.v_ss + 8 * (slot ^ vrow_swz<D>(r)), (uint32_t)(uintptr_t)(lds_void*)vdst);
    }
  };
  auto dma_tile = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma_part(kb, buf, i);
  };
  static_assert(NDMA >= 1 && NDMA <= KS / 2, "at most one DMA pair per batch of QK operand reads");

  const float c_l2 = SOFTCAP ? 1.0f : a.scale_log2;  // raw units -> log2 units

  // ---- caller mask, one tile ahead ----
  // Per tile, this lane's row holds four runs of 8 keys: run x = 2 s + r is
  // keys kb + 16 x + 8 h2 .. + 7, the keys of sc[s][8 r .. 8 r + 7].  Masked
  // tiles start at multiples of 64 keys and the host checks the mask's
  // alignment, so a run is one aligned 8-byte load; a run that crosses Lk is
  // read byte by byte.  Rows past Lq read the last row (never stored).
  global_u8* mrow = nullptr;
  if constexpr (MASK == 1)
    mrow = (global_u8*)(reinterpret_cast<const unsigned char*>(a.mask) + b * a.m_sb + h * a.m_sh +
                        (int64_t)min(my_row, a.Lq - 1) * a.m_sq);
  auto mask_load = [&](int kb, uint64_t (&mk)[4]) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int s0 = kb + 16 * x + 8 * h2;
      if (s0 + 8 <= a.Lk) {
        mk[x] = *(global_u64*)(mrow + s0);
      } else {
        uint64_t v = 0;
        for (int e = 0; e < 8; ++e)
          if (s0 + e < a.Lk) v |= (uint64_t)mrow[s0 + e] << (8 * e);
        mk[x] = v;
      }
    }
  };
  // mk_cur: this tile's runs; mk_nxt: those of the next tile computed, loaded
  // one computed tile ahead (only for tiles the mask does not keep whole).
  uint64_t mk_cur[4] = {0, 0, 0, 0}, mk_nxt[4] = {0, 0, 0, 0};
  bool mk_full = false;  // the current tile's mask keeps every key of this wave's rows
  // Tile maps of the boolean mask, filled by a first pass over the mask
  // before any K/V is loaded: bit t of need_map is set when some wave of the
  // workgroup needs tile t (its band reaches the tile and the mask leaves one
  // of its rows a key there), bit t of full_map[w] when the mask keeps every
  // key of tile t for wave w's rows.  A tile no wave needs is neither loaded
  // nor computed, and a tile kept whole reads no mask in the main loop.
  // Tiles past the map (rows of more than 2048 tiles) are taken as needed and
  // not whole.
  constexpr int kMapWords = MASK == 1 ? 64 : 1;
  __shared__ uint32_t need_map[kMapWords];
  __shared__ uint32_t full_map[kWaves][kMapWords];
  const int mapped = MASK == 1 ? min(nblk, 32 * kMapWords) : 0;
  auto full_at = [&](int t) -> bool {
    return t < mapped && ((full_map[w][t >> 5] >> (t & 31)) & 1u) != 0;
  };
  // Additive mask: the same runs as fp32 (two aligned 16-byte loads each),
  // loaded at the start of the tile that uses them: the K Q^T MFMAs cover the
  // latency, and every tile is evaluated in full.  bias / scale in raw score
  // units, so that the log2 scaling adds bias * log2(e).
  global_f32* frow = nullptr;
  if constexpr (MASK == 2)
    frow = (global_f32*)(reinterpret_cast<const float*>(a.mask) + b * a.m_sb + h * a.m_sh +
                         (int64_t)min(my_row, a.Lq - 1) * a.m_sq);
  f32x4 bias[4][2];
  auto bias_load = [&](int kb) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int s0 = kb + 16 * x + 8 * h2;
      if (s0 + 8 <= a.Lk) {
        bias[x][0] = *(global_f32x4*)(frow + s0);
        bias[x][1] = *(global_f32x4*)(frow + s0 + 4);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bias[x][e >> 2][e & 3] = s0 + e < a.Lk ? frow[s0 + e] : 0.0f;
      }
    }
  };
  const int kr0 = key_of_m(n);                        // this lane's K row in a sub-tile

  const lds_u8* const lbase = (const lds_u8*)(lds_void*)&lds[0][0][0];
  constexpr int kStage = TILE * 2;             // bytes of one K (or V) tile
  constexpr int kVBase = NSTAGE * TILE * 2;    // byte offset of the V tiles
  constexpr int kSubBytes = 2 * 32 * D;  // bytes of one 32-key sub-tile of K
  // Per-lane LDS byte offsets of the K operand reads of stage 0, sub-tile 0, one
  // per k-step (chunk 2 ks + h2 of row kr0); the other sub-tile and stage are
  // immediate offsets, since row 32 + r has the same swizzle as row r.
  static_assert(k_swz<D>(32) == k_swz<D>(0) && k_swz<D>(33) == k_swz<D>(1) && k_swz<D>(63) == k_swz<D>(31),
                "sub-tiles share the K swizzle");
  uint32_t kra[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kra[ks] = 2 * kr0 * D + 16 * ((2 * ks + h2) ^ k_swz<D>(kr0));
  // Per-lane byte offsets (from the first stage) of the transposing V reads of
  // 16-key step 0: rows 8 (g >> 1) + j (+ 4) of the step, columns
  // 16 (g & 1) + 4 c .. + 3 of each 32-column block.  Step st adds 32 D st
  // bytes and the second row 8 D; the swizzle is the same for all of them.
  uint32_t vrd[DB];
  {
    const int tg = lane >> 4, tj = (lane >> 2) & 3, tc = lane & 3;
    const int key0 = 8 * (tg >> 1) + tj;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk = 4 * db + 2 * (tg & 1) + (tc >> 1);
      vrd[db] = kVBase + 2 * D * key0 + 16 * (chunk ^ vrow_swz<D>(key0)) + 8 * (tc & 1);
    }
  }

  // Sub-tiles (32 keys) of the tile at kb that this wave can see; a tile with
  // at least one is computed whole, and a sub-tile outside every row's band
  // is masked out like any other excluded key.
  auto active = [&](int kb, bool& a0, bool& a1) {
    a0 = wrows > 0 && kb <= w_hi && kb + 31 >= w_lo;
    a1 = wrows > 0 && kb + 32 <= w_hi && kb + 63 >= w_lo;
  };

  // ---- S^T = K Q^T for both sub-tiles, two k-steps per batch of reads (the
  // next batch's reads in flight during the current batch's MFMAs); the DMA
  // pairs of a later tile ride along, one per batch ----
  auto qk = [&](auto st_tag, f32x16 (&sc)[2], auto&& dma_at) {
    constexpr int ST = decltype(st_tag)::value;
    sc[0] = f32x16{};
    sc[1] = f32x16{};
    u32x4 kf[2][4];
    auto issue = [&](int ks, u32x4 (&d)[4]) {
      d[0] = lds_b128<ST * kStage>(lbase, kra[ks]);
      d[1] = lds_b128<ST * kStage + kSubBytes>(lbase, kra[ks]);
      d[2] = lds_b128<ST * kStage>(lbase, kra[ks + 1]);
      d[3] = lds_b128<ST * kStage + kSubBytes>(lbase, kra[ks + 1]);
    };
    issue(0, kf[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      u32x4 (&cur)[4] = kf[(ks >> 1) & 1];
      if (ks + 2 < KS) issue(ks + 2, kf[((ks >> 1) + 1) & 1]);
      if ((ks >> 1) < NDMA) dma_at(ks >> 1);
      sc[0] = mma32<IS_BF16>(cur[0], qf[ks], sc[0]);
      sc[1] = mma32<IS_BF16>(cur[1], qf[ks], sc[1]);
      sc[0] = mma32<IS_BF16>(cur[2], qf[ks + 1], sc[0]);
      sc[1] = mma32<IS_BF16>(cur[3], qf[ks + 1], sc[1]);
    }
  };

  // ---- softmax of one tile's scores, in pieces that can sit between the
  // MFMAs of the previous tile's P V ----
  // (1) masks and the row max; when the running max has to move, m and l move
  // now and the factor for O is returned (O is rescaled only after all of the
  // previous tile's P V has been added to it).
  auto softmax_max = [&](f32x16 (&sc)[2], int kb, bool a0, bool a1, float& alpha) -> bool {
    float bm = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int k0 = kb + 32 * sub;
      f32x16& acc = sc[sub];
      if constexpr (SOFTCAP) {  // an additive mask value enters the cap with the logit
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) {
          float x = acc[r2];
          if constexpr (MASK == 2) x = fmaf(bias[2 * sub + (r2 >> 3)][(r2 >> 2) & 1][r2 & 3], a.bias_mul, x);
          acc[r2] = a.cap_log2 * tanh_fast(x * a.scale_over_cap);
        }
      }
      // masks only where the sub-tile crosses a frontier of some row of this
      // wave (or is outside all of them)
      const bool interior = (sub ? a1 : a0) && (a.window < 0 || k0 >= pw1 - a.window + 1) &&
                            (!a.causal || k0 + 31 <= pw0) && (k0 + 31 < sp.valid);
      if (!interior) {
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) {
          const int j = k0 + 16 * (r2 >> 3) + 8 * h2 + (r2 & 7);
          acc[r2] = (j < my_lo || j > my_hi) ? -INFINITY : acc[r2];
        }
      }
      if constexpr (MASK == 1) {  // the caller mask, unless it keeps every key of the wave's tile
        if (!mk_full) {
#pragma unroll
          for (int r2 = 0; r2 < 16; ++r2) {
            const uint64_t run = mk_cur[2 * sub + (r2 >> 3)];
            acc[r2] = ((run >> (8 * (r2 & 7))) & 0xffu) ? acc[r2] : -INFINITY;
          }
        }
      }
      if constexpr (MASK == 2) {  // -inf (or NaN) removes the key
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) {
          const float bv = bias[2 * sub + (r2 >> 3)][(r2 >> 2) & 1][r2 & 3];
          acc[r2] = bv > -INFINITY ? (SOFTCAP ? acc[r2] : fmaf(bv, a.bias_mul, acc[r2])) : -INFINITY;
        }
      }
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) bm = fmaxf(bm, acc[r2]);
    }
    // lane owns row n; lanes n and n+32 share the row
    bm = fmaxf(bm, xor32(bm));
    const float m_new = fmaxf(m_run, bm);
    const bool need = (m_new - m_run) * c_l2 > kRescaleLog2;  // false while both are -inf
    alpha = 1.0f;
    const bool any = __any(need);
    if (any) {
      // a real branch: moving the running max is rare
      asm volatile("" ::: "memory");
      alpha = need ? fast_exp2((m_run - m_new) * c_l2) : 1.0f;
      m_run = need ? m_new : m_run;
      l_run *= alpha;
    }
    return any;
  };
  // (2) P = exp2(x - m) for keys 8 half .. 8 half + 7 of each row's two runs
  // in sub-tile sub, packed to the input type; l += sum P
  auto softmax_exp = [&](const f32x16& acc, int half, u32x4& pk) {
    const float mb = m_run == -INFINITY ? 0.0f : m_run * c_l2;
    float pv[8];
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) {
      pv[r2] = fast_exp2(fmaf(acc[8 * half + r2], c_l2, -mb));
      l_run += pv[r2];
    }
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) pk[q2] = pack2<IS_BF16>(pv[2 * q2], pv[2 * q2 + 1]);
  };
  auto rescale_o = [&](float alpha) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) o[db][r2] *= alpha;
    // the scaled accumulators pass through an asm statement that cannot be
    // speculated, so the (rare) multiplies stay behind the branch instead of
    // being hoisted out of it as o * (cond ? alpha : 1)
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(o[db]));
  };

  // ---- O^T += V^T P^T: four 16-key steps, the reads of the next step in
  // flight during the MFMAs of the current one; consecutive MFMAs update
  // different accumulators ----
  auto pv = [&](auto stage_tag, const u32x4 (&pb)[2][2], auto&& before, auto&& after) {
    constexpr int SO = decltype(stage_tag)::value * kStage;
    uint64_t vr[2][2 * DB];
    // the V operands of 16-key step ST: for each 32-wide output block, rows
    // key0 and key0 + 4 (immediate offsets from the block's per-lane offset)
    auto vissue = [&](auto st_tag, uint64_t (&d)[2 * DB]) {
      constexpr int O0 = SO + 32 * D * decltype(st_tag)::value;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        d[2 * db] = lds_tr16<O0>(lbase, vrd[db]);
        d[2 * db + 1] = lds_tr16<O0 + 8 * D>(lbase, vrd[db]);
      }
    };
    auto vstep = [&](auto st_tag) {
      constexpr int ST = decltype(st_tag)::value;
      uint64_t (&cur)[2 * DB] = vr[ST & 1];
      if constexpr (ST + 1 < 4) vissue(std::integral_constant<int, ST + 1>{}, vr[(ST + 1) & 1]);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = mma32<IS_BF16>(__builtin_bit_cast(u32x4, u64x2{cur[2 * db], cur[2 * db + 1]}),
                               pb[ST >> 1][ST & 1], o[db]);
    };
    vissue(std::integral_constant<int, 0>{}, vr[0]);
    before();
    vstep(std::integral_constant<int, 0>{});
    after(0);
    vstep(std::integral_constant<int, 1>{});
    after(1);
    vstep(std::integral_constant<int, 2>{});
    after(2);
    vstep(std::integral_constant<int, 3>{});
    after(3);
  };

  // ---- schedule: per tile, K Q^T (the next tile's loads riding along), the
  // softmax, P V; then wait for the next tile and meet ----
  // the first tile at or after t that the workgroup computes (nblk if none)
  auto next_tile = [&](int t) -> int {
    if constexpr (MASK == 1) {
      while (t < mapped) {
        const uint32_t word = need_map[t >> 5] >> (t & 31);
        if (word != 0) return t + __builtin_ctz(word);
        t = min((t | 31) + 1, mapped);
      }
    }
    return min(t, nblk);
  };
  if constexpr (MASK == 1) {
    // ---- the first pass over the boolean mask: fill the tile maps ----
    // When the mask does not vary over heads, the waves that share their
    // rows (the hw heads of one row group) split the tiles and each writes
    // the bits of the whole group, so the workgroup reads each mask byte once.
    for (int i = tid; i < kMapWords; i += 256) need_map[i] = 0;
    for (int i = tid; i < kWaves * kMapWords; i += 256) (&full_map[0][0])[i] = 0;
    __syncthreads();
    const bool shared_rows = a.m_sh == 0;
    const int step = shared_rows ? hw : 1;
    const int g0 = shared_rows ? w - w % hw : w;
    constexpr int PB = 4;  // tiles in flight per wave (more made no run faster)
    for (int t0 = shared_rows ? w % hw : 0; t0 < mapped; t0 += PB * step) {
      // A tile that reaches past Lk is taken as needed (if the band reaches
      // it) and not whole, without reading it: the main loop reads its runs
      // byte by byte.
      uint64_t mk[PB][4];
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        const int kbp = kv_lo + (t0 + p * step) * BN;
        if (t0 + p * step < mapped && kbp + BN <= a.Lk)
#pragma unroll
          for (int x = 0; x < 4; ++x) mk[p][x] = *(global_u64*)(mrow + kbp + 16 * x + 8 * h2);
      }
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        const int t = t0 + p * step;
        if (t < mapped) {
          const int kbp = kv_lo + t * BN;
          bool b0, b1;
          active(kbp, b0, b1);
          bool need = b0 || b1, full = false;
          if (kbp + BN <= a.Lk) {
            const bool n0 = __any((mk[p][0] | mk[p][1]) != 0), n1 = __any((mk[p][2] | mk[p][3]) != 0);
            need = (b0 && n0) || (b1 && n1);
            // every byte of every run nonzero in every lane (the
            // has-zero-byte bit trick on each run): the tile keeps all keys
            constexpr uint64_t kOnes = 0x0101010101010101ull, kHigh = 0x8080808080808080ull;
            uint64_t zero = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) zero |= (mk[p][x] - kOnes) & ~mk[p][x] & kHigh;
            full = __all(zero == 0);
          }
          const uint32_t bit = 1u << (t & 31);
          if (lane == 0) {
            if (need) atomicOr(&need_map[t >> 5], bit);
            if (full)
              for (int j = 0; j < step; ++j) atomicOr(&full_map[g0 + j][t >> 5], bit);
          }
        }
      }
    }
    __syncthreads();
  }
  const int t_first = next_tile(0);
  if (t_first < nblk) dma_tile(kv_lo + t_first * BN, 0);
  if constexpr (MASK == 1)
    if (t_first < nblk && !full_at(t_first)) mask_load(kv_lo + t_first * BN, mk_nxt);
  __builtin_amdgcn_s_waitcnt(0);  // Q registers, the first tile (and its mask)
  tile_barrier();
  if (rot && my_row < a.Lq && my_p >= 0) {
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      u32x4 lo = qf[ks], hi = qf[ks + KS / 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4& c = rc[ks][e >> 1];
        const f32x4& sn = rs[ks][e >> 1];
        float u0, w0, u1, w1;
        rot_pair(half_to_f32<IS_BF16>((uint16_t)(lo[e] & 0xffffu)), half_to_f32<IS_BF16>((uint16_t)(hi[e] & 0xffffu)),
                 c[2 * (e & 1)], sn[2 * (e & 1)], u0, w0);
        rot_pair(half_to_f32<IS_BF16>((uint16_t)(lo[e] >> 16)), half_to_f32<IS_BF16>((uint16_t)(hi[e] >> 16)),
                 c[2 * (e & 1) + 1], sn[2 * (e & 1) + 1], u1, w1);
        lo[e] = pack2<IS_BF16>(u0, u1);
        hi[e] = pack2<IS_BF16>(w0, w1);
      }
      qf[ks] = lo;
      qf[ks + KS / 2] = hi;
    }
  }

  if constexpr (D >= 256) {
    // One wave per SIMD: Q lives in accumulation registers (the MFMA reads
    // its operands from them), which leaves the vector registers to the K and
    // V operands and the softmax instead of spilling them there.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qf[ks]));
  }
  f32x16 sc[2];
  u32x4 pb[2][2];
  // One tile; its stage (it & 1) is a compile-time constant, so that every
  // LDS address of the tile is a per-lane register plus an immediate.
  auto tile = [&](int t, int tn, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    const int kb = kv_lo + t * BN;
    const int kbn = kv_lo + tn * BN;  // the next tile computed
    // The next tile's loads are spread over the K operand batches (or issued
    // at once by a wave with nothing to compute here): a wave that issued all
    // of them back to back would stall behind the other waves' loads.
    const bool load_next = tn < nblk;
    bool a0, a1;
    active(kb, a0, a1);
    if constexpr (MASK == 1) {
      // this tile's runs landed with the previous tile's loads (none if the
      // mask keeps it whole); fetch those of the next tile computed unless
      // the mask keeps that one whole; skip sub-tiles whose keys the mask
      // clears for all 32 rows
      mk_full = full_at(t);
#pragma unroll
      for (int x = 0; x < 4; ++x) mk_cur[x] = mk_nxt[x];
      if (load_next && !full_at(tn)) mask_load(kbn, mk_nxt);
      if (!mk_full) {
        a0 = a0 && __any((mk_cur[0] | mk_cur[1]) != 0);
        a1 = a1 && __any((mk_cur[2] | mk_cur[3]) != 0);
      }
    }
    auto dma_at = [&](int i) {
      if (load_next) dma_part(kbn, ST ^ 1, i);
    };
    if constexpr (MASK == 2)
      if (a0 || a1) bias_load(kb);
    if (a0 || a1) {
      qk(stage_tag, sc, dma_at);
      float alpha;
      if (softmax_max(sc, kb, a0, a1, alpha)) rescale_o(alpha);
#pragma unroll
      for (int q = 0; q < 4; ++q) softmax_exp(sc[q >> 1], q & 1, pb[q >> 1][q & 1]);
      pv(stage_tag, pb, [] {}, [](int) {});
    } else if (load_next) {
      dma_tile(kbn, ST ^ 1);
    }
    // this wave's loads of the next tile have landed; after the barrier every
    // wave's have, and nobody reads this tile's stage any more
    wait_vm<0>();
    tile_barrier();
  };
  if constexpr (MASK == 1) {
    // from needed tile to needed tile
    for (int t = t_first; t < nblk;) {
      int tn = next_tile(t + 1);
      tile(t, tn, std::integral_constant<int, 0>{});
      t = tn;
      if (t >= nblk) break;
      tn = next_tile(t + 1);
      tile(t, tn, std::integral_constant<int, 1>{});
      t = tn;
    }
  } else {
    for (int it = 0; it < nblk; it += 2) {
      tile(it, it + 1, std::integral_constant<int, 0>{});
      if (it + 1 < nblk) tile(it + 1, it + 2, std::integral_constant<int, 1>{});
    }
  }

  // ---- epilogue: fold the sink, normalize, narrow, store ----
  if (my_row >= a.Lq) return;
  const float l_row = l_run + xor32(l_run);
  float fac;
  if (my_lo > my_hi || (MASK != 0 && m_run == -INFINITY)) {
    fac = 0.0f;  // no key left for the row: exactly zero
  } else if (a.use_sink) {
    const float mt = m_run * c_l2;
    const float ts = sink_log2(a, h);
    const float M = fmaxf(mt, ts);
    const float e1 = fast_exp2(mt - M);
    fac = e1 / (l_row * e1 + fast_exp2(ts - M));
  } else {
    fac = 1.0f / l_row;
  }
  uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)my_row * a.o_ss;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 pk;
      pk[0] = pack2<IS_BF16>(o[db][4 * q4] * fac, o[db][4 * q4 + 1] * fac);
      pk[1] = pack2<IS_BF16>(o[db][4 * q4 + 2] * fac, o[db][4 * q4 + 3] * fac);
      *reinterpret_cast<u32x2*>(op + 32 * db + 8 * q4 + 4 * h2) = pk;
    }
}

template <bool IS_BF16, int D>
hipError_t launch_t(const AttnArgs& a, bool softcap, hipStream_t stream) {
  // heads per workgroup: the largest power of two that divides G, at most 4 (one per wave)
  const int hw = std::min(a.G & -a.G, kWaves);
  const int rpw = 32 * (kWaves / hw);
  const int nrb = (a.Lq + rpw - 1) / rpw;
  const int items = a.B * a.Hkv * (a.G / hw) * nrb;
  const int per_xcd = (items + 7) / 8;
  dim3 grid(8 * per_xcd), block(64 * kWaves);
  if (a.mask_kind == 1 && softcap)
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, true, 1>), grid, block, 0, stream, a, nrb, items, per_xcd, hw);
  else if (a.mask_kind == 1)
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, false, 1>), grid, block, 0, stream, a, nrb, items, per_xcd, hw);
  else if (a.mask_kind == 2 && softcap)
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, true, 2>), grid, block, 0, stream, a, nrb, items, per_xcd, hw);
  else if (a.mask_kind == 2)
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, false, 2>), grid, block, 0, stream, a, nrb, items, per_xcd, hw);
  else if (softcap)
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, true, 0>), grid, block, 0, stream, a, nrb, items, per_xcd, hw);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<IS_BF16, D, false, 0>), grid, block, 0, stream, a, nrb, items, per_xcd, hw);
  return hipGetLastError();
}

}  // namespace

bool prefill_mfma_supported(int dtype, int head_size) {
  return (dtype == kBF16 || dtype == kF16) &&
         (head_size == 32 || head_size == 64 || head_size == 128 || head_size == 256);
}

hipError_t launch_prefill_mfma(const AttnArgs& a, int dtype, bool softcap, hipStream_t stream) {
  if (a.B == 0 || a.Lq == 0) return hipSuccess;
  if (dtype == kBF16) {
    if (a.D == 128) return launch_t<true, 128>(a, softcap, stream);
    if (a.D == 64) return launch_t<true, 64>(a, softcap, stream);
    if (a.D == 256) return launch_t<true, 256>(a, softcap, stream);
    if (a.D == 32) return launch_t<true, 32>(a, softcap, stream);
  } else if (dtype == kF16) {
    if (a.D == 128) return launch_t<false, 128>(a, softcap, stream);
    if (a.D == 64) return launch_t<false, 64>(a, softcap, stream);
    if (a.D == 256) return launch_t<false, 256>(a, softcap, stream);
    if (a.D == 32) return launch_t<false, 32>(a, softcap, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
