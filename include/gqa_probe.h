/*
 * gqa_probe.h -- measurement aid of libgqa_mi355x (not part of the attention
 * path): the device's dense bf16 matrix rate and shader clock, measured.
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

#ifdef __cplusplus
}
#endif

#endif /* GQA_MI355X_PROBE_H */
