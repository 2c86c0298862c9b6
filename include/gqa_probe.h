/*
 * gqa_probe.h -- measurement aids of libgqa_mi355x (not part of the attention
 * path): the device's dense bf16 matrix rate and shader clock, and the rate
 * at which the decode's loading scheme streams K/V units, measured.
 */
#ifndef GQA_MI355X_PROBE_H
#define GQA_MI355X_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `blocks` workgroups of 4 waves; every wave issues `iters` rounds
 * of 8 independent v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on register
 * operands and records its shader-clock counter (s_memtime) and 100 MHz
 * counter (s_memrealtime) before and after: stamps is device uint64
 * [blocks * 4][4] = (clock start, clock end, 100 MHz start, 100 MHz end),
 * sink device fp32 [blocks * 4] (keeps the results alive).  Both buffers are
 * the caller's.  The caller times the launch (events on hip_stream) for the
 * rate; clock = d(clock) / d(100 MHz) * 100 MHz.  Returns 0, 1 for a bad
 * argument, 4 for a launch error. */
int gqa_probe_mfma_peak(int blocks, int iters, void* stamps, void* sink, void* hip_stream);

/* Streams `units` K/V units through the split-KV decode's loading scheme with
 * no attention work: the ceiling its HBM rate is read against.  A unit is 16
 * key rows of row_bytes bytes (256: head size 128, 512: head size 256, with
 * 16-bit elements) of k and the same bytes of v, at byte offset unit_off[u]
 * (device int64 [units]) in both; the
 * units are cut evenly over `grid` workgroups of 4 waves, and each wave
 * streams its share through two LDS stages by LDS DMA (non-temporal, the
 * decode's chunk swizzle), waiting for each unit as the decode does.
 * kv_bytes is the size of the smaller of the two buffers; an offset whose
 * unit would leave it reads the first unit instead.  sink is a device fp32
 * [1] that keeps the reads (practically never written).  The caller times
 * the launch (events on hip_stream).  Returns 0, 1 for a bad argument (grid
 * < 1, row_bytes other than 256 or 512, a NULL buffer, kv_bytes below one
 * unit, or more than 256 units per workgroup), 4 for a launch error. */
int gqa_probe_kv_stream(int grid, int row_bytes, const void* k, const void* v, int64_t kv_bytes,
                        const int64_t* unit_off, int units, void* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_MI355X_PROBE_H */
