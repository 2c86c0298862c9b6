/*
 * gqa.h -- C ABI of the MI355X (gfx950) windowed grouped-query attention library.
 *
 * Library: libgqa_mi355x.so (hand-written HIP kernels; no host fallback).
 *
 * What is computed.  For batch b, query head h (K/V head g = h / G, G =
 * num_heads / kv_num_heads, K/V never copied per query head), query row i at
 * absolute position p = q_offset_b + i, and key slot j at position j, key j is
 * ALLOWED iff
 *     j < valid_b  and  (not causal or j <= p)  and  (W == -1 or p - j < W).
 * x_ij = scale * <q_i, k_j>, then x_ij = c * tanh(x_ij / c) when softcap c > 0.
 *     O_i = sum_{j allowed} e^{x_ij} v_j / (sum_{j allowed} e^{x_ij} + [sink] e^{s_h})
 * and O_i = 0 exactly when no key is allowed.  Sources (page, section):
 *   - head sharing without copies, [B,H,L,D] / [B,L,H*D] layouts, softcap,
 *     nonpad_kv_seqlen, zero rows, fp32 accumulation: "Attention Kernel
 *     Design" (onnx-light-cpu), sections "Layouts and semantics" and
 *     "Scheduling, precision, and invariants";
 *   - window in absolute positions, decode rows at (total - curr) + i, sink
 *     in the denominator only: "[NPUW] Support GQA sliding-window and
 *     smooth-softmax in DecomposeGQA", sections "Sliding window
 *     (local_window_size)" and "smooth_softmax / head_sink";
 *   - bottom-right causal alignment and the KV cache as concatenation of past
 *     and step: "onnx: import GroupQueryAttention decode steps and its
 *     internal rotary", section "What changed".
 *
 * Conventions shared by every entry point.
 *   Ownership:  every device buffer belongs to the caller.  The library never
 *               allocates device memory; it owns only the host-side plan and
 *               the static decode scratch array of gqa_decode_noalloc (part of
 *               its code object, one per GPU).
 *   Asynchrony: calls enqueue work on `hip_stream` (a hipStream_t; NULL = the
 *               default stream) and return; GQA_OK means "enqueued".
 *   Validation: everything checkable on the host is checked before any launch.
 *               On error nothing is enqueued, the status says which class of
 *               error, and gqa_last_error() returns a message naming the
 *               argument (thread-local; valid until the next failing call on
 *               the same thread).
 *   Tensors:    gqa_tensor = base pointer + element strides for batch, head and
 *               sequence; the head dimension is contiguous.  [B,H,L,D] and
 *               [B,L,H*D] are both expressible.  Base pointers must be 16-byte
 *               aligned and strides multiples of 16 bytes / element size.
 *   Device-side lengths: seqlens_k / nonpad_kv_seqlen live in device memory
 *               and cannot be checked on the host.  A value out of range makes
 *               every output row of that batch exactly zero (and append_kv
 *               skip that batch); no access leaves the tensors' extents.
 *   Threads:    a plan is immutable after gqa_plan(); it may be used from
 *               several threads/streams at once if each call gets its own
 *               workspace.
 */
#ifndef GQA_MI355X_H
#define GQA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gqa_plan_s* gqa_plan_t;

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1, /* malformed argument or attribute combination */
  GQA_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels cover */
  GQA_ERR_CAPACITY = 3,    /* a size exceeds the plan's maxima or the cache */
  GQA_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} gqa_status;

/* Element type of Q, K, V, O and the cache (all equal).  Mirrors the
 * FLOAT / FLOAT16 / BFLOAT16 type set of "Attention Kernel Design". */
typedef enum { GQA_F32 = 0, GQA_F16 = 1, GQA_BF16 = 2 } gqa_dtype;

/* Node attributes.  Mirrors GroupQueryAttention's attribute set as the pages
 * describe it (num_heads, kv_num_heads, scale, local_window_size, softcap,
 * smooth_softmax, head_sink) plus the causal flag of ONNX Attention. */
typedef struct {
  int32_t num_heads;         /* Hq > 0 */
  int32_t kv_num_heads;      /* Hkv > 0, Hq % Hkv == 0 */
  int32_t head_size;         /* D: multiple of 8, 8..256 (V has the same D) */
  float scale;               /* > 0; 0 selects 1/sqrt(D) */
  int32_t local_window_size; /* -1 = off; W >= 1 = keys kept per query, self included */
  float softcap;             /* 0 = off; c > 0 applies c*tanh(x/c) to scaled logits */
  int32_t smooth_softmax;    /* 0/1: extra logit 0 in the denominator when no head_sink */
  int32_t use_head_sink;     /* 0/1: a per-query-head fp32 sink logit array is passed */
  int32_t is_causal;         /* 1 = bottom-right causal band; 0 only with W == -1 */
  gqa_dtype dtype;           /* element type of every tensor argument */
  int32_t rolling_cache;     /* 0/1: the KV cache is a ring (sliding_window_cache, "[NPUW]
                              * Support GQA sliding-window ...", section "Sliding window
                              * (local_window_size)"): the token at position p lives in slot
                              * p mod capacity, positions may pass the capacity, and every
                              * call needs capacity >= W + curr - 1 (so every key a step may
                              * see is still held).  Needs W >= 1.  Affects gqa_append_kv,
                              * gqa_append_kv_rotary and gqa_decode only. */
} gqa_attrs;

/* A strided 4-D view [B][H][L][D] with a contiguous last dimension.  Strides
 * are in elements.  [B,L,H*D] is stride_b = L*H*D, stride_h = D, stride_s = H*D. */
typedef struct {
  void* data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_s;
} gqa_tensor;

/* Validate attributes and size limits; build an immutable plan.
 * max_batch, max_q_len (prefill Lq / decode curr) and max_kv_len (prefill Lk /
 * decode capacity) bound every later call and size the workspace.
 * Following the descriptor/plan split of "Attention Kernel Design", section
 * "Descriptor and invocation plan".  Host only; touches no device.
 * Errors: INVALID_ARG (bad attribute or pairing), UNSUPPORTED (head_size). */
gqa_status gqa_plan(const gqa_attrs* attrs, int32_t max_batch, int32_t max_q_len,
                    int64_t max_kv_len, gqa_plan_t* out_plan);

/* Release a plan (NULL is ignored).  Must not race with calls using it.
 * The plan is the host-side descriptor of "Attention Kernel Design", section
 * "Descriptor and invocation plan"; it owns no device memory. */
void gqa_plan_destroy(gqa_plan_t plan);

/* Bytes of device workspace gqa_decode needs at the plan's maxima: per-row-
 * tile arrival counters (a fixed region of 2048 32-bit words at the front)
 * followed by the split-KV partial results (running max, denominator and
 * unnormalized output of each piece of the key range, merged by log-sum-exp:
 * the streaming recurrence of "Attention Kernel Design", section "Compute
 * paths", cut into independent key ranges).  The workspace must be
 * zero-filled once before its first gqa_decode call; every completed call
 * leaves the counters at zero again, so it can be reused by later calls (of
 * any plan and shape) without clearing.  gqa_prefill and gqa_append_kv need
 * none.  0 for NULL. */
size_t gqa_workspace_size(gqa_plan_t plan);

/* Prompt attention on an empty past ("Attention Kernel Design", sections
 * "Layouts and semantics" and "Compute paths"; bottom-right band of "onnx:
 * import GroupQueryAttention decode steps ...", section "What changed").
 *   q   [B, Hq,  Lq, D]   k, v [B, Hkv, Lk, D]   out [B, Hq, Lq, D]
 *   q_offset = Lk - Lq (rows with negative positions see nothing -> 0).
 *   nonpad_kv_seqlen: device int64 [B] or NULL (NULL = Lk for every batch);
 *     keys j >= nonpad_b are masked; the causal offset is unchanged.
 *   head_sink: device fp32 [Hq]; non-NULL iff attrs.use_head_sink.
 *   workspace/ws_bytes: unused (may be NULL/0).
 * B == 0 or Lq == 0 is a no-op.  Lk == 0 writes zeros.
 * Errors: INVALID_ARG (NULL/misaligned/negative sizes, sink pairing),
 *   CAPACITY (B, Lq or Lk above the plan maxima), UNSUPPORTED (stride
 *   alignment), HIP (launch failure). */
gqa_status gqa_prefill(gqa_plan_t plan, int32_t B, int32_t Lq, int64_t Lk,
                       gqa_tensor q, gqa_tensor k, gqa_tensor v, gqa_tensor out,
                       const int64_t* nonpad_kv_seqlen, const float* head_sink,
                       void* workspace, size_t ws_bytes, void* hip_stream);

/* Append curr new K/V rows per (batch, KV head) to the cache: row t goes to
 * slot total_b - curr + t, total_b = seqlens_k[b] + 1 (present =
 * concat(past, step), "onnx: import GroupQueryAttention decode steps ...",
 * section "What changed"); with attrs.rolling_cache, to slot
 * (total_b - curr + t) mod capacity.
 *   k_new, v_new [B, Hkv, curr, D]   k_cache, v_cache [B, Hkv, capacity, D]
 *   seqlens_k: device int32 [B] (a [B,1] array is the same memory).
 * A batch with total_b < curr, or (without rolling_cache) total_b > capacity,
 * is skipped.
 * Errors: INVALID_ARG, CAPACITY (curr > capacity or above plan maxima),
 *   UNSUPPORTED, HIP. */
gqa_status gqa_append_kv(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                         gqa_tensor k_new, gqa_tensor v_new,
                         gqa_tensor k_cache, gqa_tensor v_cache,
                         const int32_t* seqlens_k, void* hip_stream);

/* Single- or multi-token decode of curr new tokens against a cache that
 * already holds them (call gqa_append_kv first).  Query row t of batch b sits
 * at position total_b - curr + t; keys are the slots [0, total_b) ("[NPUW]
 * Support GQA sliding-window ...", section "Sliding window
 * (local_window_size)"; causal inside the step: row t sees new tokens <= t).
 * With attrs.rolling_cache the key at position j is read from slot
 * j mod capacity; the result is the windowed attention over the whole
 * history (the same page: the window as a mask over the full cache and the
 * rolling buffer give the same result), which needs capacity >= W + curr - 1.
 *   q, out [B, Hq, curr, D]   k_cache, v_cache [B, Hkv, capacity, D]
 *   seqlens_k: device int32 [B]; head_sink as in gqa_prefill.
 *   workspace: device, >= gqa_workspace_size(plan) bytes, 16-byte aligned,
 *     zero-filled before its first use (see gqa_workspace_size), owned by
 *     this call until it completes on the stream; calls that overlap in time
 *     must use different workspaces.
 * Errors: INVALID_ARG (incl. workspace too small), CAPACITY, UNSUPPORTED, HIP. */
gqa_status gqa_decode(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                      gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                      const int32_t* seqlens_k, const float* head_sink,
                      void* workspace, size_t ws_bytes, void* hip_stream);

/* One decode step in one call: gqa_append_kv of the step's curr new K/V rows
 * followed by gqa_decode of its curr query rows (the cache as the
 * concatenation of past and step, "onnx: import GroupQueryAttention decode
 * steps and its internal rotary", section "What changed"; the rows' positions
 * and window of "[NPUW] Support GQA sliding-window and smooth-softmax in
 * DecomposeGQA", section "Sliding window (local_window_size)").  Arguments
 * as the two calls; the results (out and the cache contents) are those of the
 * two calls.  On the matrix-core decode (bf16/fp16, head size 64/128/256) it
 * is one launch: the new rows are copied to their slots while the attention
 * reads those positions from k_new / v_new directly; otherwise the append
 * kernel runs first.
 *   k_new, v_new [B, Hkv, curr, D]; the rest as gqa_decode.
 * Errors: as gqa_append_kv and gqa_decode. */
gqa_status gqa_append_decode(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                             gqa_tensor q, gqa_tensor k_new, gqa_tensor v_new,
                             gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                             const int32_t* seqlens_k, const float* head_sink,
                             void* workspace, size_t ws_bytes, void* hip_stream);

/* gqa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The split-KV partials and arrival counters live
 * in a static device array of the library, 16 MiB per GPU, held by each GPU
 * the library runs on until the process ends; its address is looked up on
 * the first call on a device, which also clears the counters with a small
 * kernel on `hip_stream`.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library call.  All calls on one GPU share that array, so calls
 * that overlap in time on one GPU (other streams, other threads) race and
 * must not be issued; consecutive calls on one stream are fine.  Arguments,
 * results and the other errors are those of gqa_decode.
 * Errors: as gqa_decode, and CAPACITY when a call needs more scratch than the
 *   array holds (about 1500 row tiles of 16 query rows at head size 128, 760
 *   at 256; such calls need gqa_decode with a workspace). */
gqa_status gqa_decode_noalloc(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                              gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                              const int32_t* seqlens_k, const float* head_sink, void* hip_stream);

/* Rotary position tables supplied by the caller ("onnx: import
 * GroupQueryAttention decode steps and its internal rotary", section "What
 * changed": cos/sin caches with half the head size).  Device fp32, row-major
 * [max_pos, head_size / 2], 16-byte aligned; row p holds the cosines
 * (sines) of position p's angles, column i the angle of the pair
 * (i, i + head_size/2).  Owned by the caller. */
typedef struct {
  const float* cos;
  const float* sin;
  int64_t max_pos;
} gqa_rotary_tables;

/* Rotary position embedding of rows [B, H, L, head_size] (do_rotary of the
 * page above): element i pairs with i + head_size/2 and the pair turns by the
 * angle of its row's position, (a, b) -> (a c - b s, b c + a s), computed in
 * fp32 and rounded to the plan's dtype (nearest even).  Row l sits at
 * position pos0 + l: a prompt on an empty past passes pos0 = Lk - Lq for Q
 * and 0 for K (positions 0 .. S-1 when Lq = Lk = S), then calls gqa_prefill
 * on the results.
 *   x, y: [B, H, L, head_size] of the plan's dtype; y may be x itself (in
 *     place) but must not otherwise overlap it.
 * B, H or L == 0 is a no-op.
 * Errors: INVALID_ARG (NULL or negative arguments), CAPACITY (pos0 + L >
 *   tables->max_pos), UNSUPPORTED (alignment, sizes above 65535 / 2^30), HIP. */
gqa_status gqa_apply_rotary(gqa_plan_t plan, int32_t B, int32_t H, int32_t L, int64_t pos0,
                            gqa_tensor x, gqa_tensor y, const gqa_rotary_tables* tables,
                            void* hip_stream);

/* gqa_prefill with the rotary embedding of Q fused into the prefill's load
 * of Q (do_rotary of the page above: a prompt's rows take positions 0 .. S-1,
 * bottom-right aligned): query row i is turned at position Lk - Lq + i
 * exactly as gqa_apply_rotary would turn it (fp32, then RNE to the plan's
 * type), and the result equals gqa_apply_rotary on q followed by
 * gqa_prefill, bit for bit.  K arrives turned (gqa_apply_rotary with pos0 =
 * 0, or a cache filled by gqa_append_kv_rotary); V is not turned.
 * Arguments as gqa_prefill; tables as gqa_apply_rotary, covering positions
 * 0 .. Lk - 1.  Needs a bf16 or fp16 plan of head size 32, 64, 128 or 256
 * (the matrix-core prefill).
 * Errors: as gqa_prefill; CAPACITY when tables->max_pos < Lk; UNSUPPORTED for
 *   other plans and for K/V row strides of 2^24 elements or more. */
gqa_status gqa_prefill_rotary(gqa_plan_t plan, int32_t B, int32_t Lq, int64_t Lk,
                              gqa_tensor q, gqa_tensor k, gqa_tensor v, gqa_tensor out,
                              const int64_t* nonpad_kv_seqlen, const float* head_sink,
                              const gqa_rotary_tables* tables, void* hip_stream);

/* gqa_append_kv with rotary, in one launch: the curr new K rows are turned at
 * their positions before they enter the cache (K is cached rotated, the page
 * above), the new V rows are copied, and the curr query rows are turned into
 * q_rot for the gqa_decode call that follows.  New token t of batch b sits at
 * position total_b - curr + t, total_b = seqlens_k[b] + 1, which is also its
 * cache slot (a single generated token: position seqlens_k[b]); with
 * attrs.rolling_cache the slot is that position mod capacity, positions may
 * pass the capacity, and K and q_rot rows whose position is at or past
 * tables->max_pos are left unwritten (the host cannot see the lengths; the
 * V rows are still copied).
 *   q, q_rot [B, Hq, curr, D] (q_rot may be q itself); k_new, v_new, k_cache,
 *   v_cache and seqlens_k as in gqa_append_kv; tables as above.
 * A batch with total_b < curr, or (without rolling_cache) total_b > capacity,
 * is skipped (its cache
 * slots and q_rot rows are left as they are).
 * Errors: as gqa_append_kv, and CAPACITY when tables->max_pos < capacity. */
gqa_status gqa_append_kv_rotary(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                gqa_tensor q, gqa_tensor q_rot,
                                gqa_tensor k_new, gqa_tensor v_new,
                                gqa_tensor k_cache, gqa_tensor v_cache,
                                const int32_t* seqlens_k, const gqa_rotary_tables* tables,
                                void* hip_stream);

/* A caller mask over [B, Hq, Lq, Lk] (decode: [B, Hq, curr, capacity], the
 * key index being the position), broadcast by zero strides ("Attention
 * Kernel Design", section "Layouts and semantics": boolean and float
 * additive broadcast masks; "onnx: import GroupQueryAttention decode steps
 * ...", section "What changed": attention_bias summed with the band).
 *   GQA_MASK_BOOL: uint8, nonzero = the query may attend the key; the keys it
 *     clears leave the allowed set.
 *   GQA_MASK_ADDITIVE: fp32, added to the scaled logit before softcap; -inf
 *     (or NaN) removes the key; +inf is not allowed.  The sink gets no bias.
 * A row left with no key is exactly 0.  Device memory, caller-owned; the
 * key dimension is contiguous, strides are in elements and >= 0. */
typedef enum { GQA_MASK_BOOL = 1, GQA_MASK_ADDITIVE = 2 } gqa_mask_kind;
typedef struct {
  const void* data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_q;
  gqa_mask_kind kind;
} gqa_mask;

/* gqa_prefill with a caller mask (arguments otherwise as gqa_prefill).  On a
 * bf16 or fp16 plan of head size 32, 64, 128 or 256 (with or without softcap), a boolean mask
 * whose data and strides are multiples of 8 bytes, or an additive one whose
 * data is 16-byte aligned and strides multiples of 4 elements, runs on the
 * matrix-core prefill: each wave reads its rows' entries of a 64-key tile (a
 * boolean mask one tile ahead, skipping a tile it clears for all 32 rows; an
 * additive mask at the start of the tile, evaluated in full).  Other masks run
 * on the streaming one-wavefront-per-row kernel, which skips a 64-key block
 * with no key left (the all-false block skipping of "Attention Kernel
 * Design", section "Compute paths").
 * Errors: as gqa_prefill, and INVALID_ARG for a NULL mask, an unknown kind or
 *   a negative stride, UNSUPPORTED for a misaligned additive mask. */
gqa_status gqa_prefill_masked(gqa_plan_t plan, int32_t B, int32_t Lq, int64_t Lk,
                              gqa_tensor q, gqa_tensor k, gqa_tensor v, gqa_tensor out,
                              const int64_t* nonpad_kv_seqlen, const float* head_sink,
                              const gqa_mask* mask, void* hip_stream);

/* gqa_decode with a caller mask over [B, Hq, curr, capacity] (arguments
 * otherwise as gqa_decode).  With a workspace (as gqa_decode's), a bf16/fp16
 * plan of head size 64, 128 or 256 (with or without softcap), and a mask whose data and
 * strides are multiples of 4 bytes (boolean) or 16 bytes and 4 elements
 * (additive), it runs on the matrix-core split-KV decode, each lane reading
 * its 4 entries of a 16-key unit one unit ahead.  Otherwise (or with a NULL
 * workspace) it runs on the streaming kernel of gqa_prefill_masked.
 * Errors: as gqa_decode and gqa_prefill_masked, and UNSUPPORTED with a
 *   rolling cache (positions pass the mask's width). */
gqa_status gqa_decode_masked(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                             gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache,
                             gqa_tensor out, const int32_t* seqlens_k, const float* head_sink,
                             const gqa_mask* mask, void* workspace, size_t ws_bytes,
                             void* hip_stream);

/* FP8 (E4M3) KV cache (the pages name quantized KV caches only as outside
 * their scope: "[NPUW] Support GQA sliding-window ...", section
 * "smooth_softmax / head_sink"; every rule here is this library's reading).
 * The caches are uint8 [B, Hkv, capacity, D] of OCP E4M3 codes (sign, 4
 * exponent bits with bias 7, 3 mantissa bits; largest finite 448; no
 * infinities), with one fp32 scale for K and one for V: K = decode(code) *
 * k_scale.  Strides of the caches are in bytes (= elements), multiples of 16.
 *
 * gqa_append_kv_fp8: gqa_append_kv that quantizes the new rows (the plan's
 * dtype): code = nearest E4M3 value of x * fp32(1 / scale) computed in fp32,
 * ties to even, magnitudes beyond 448 saturated to 448, NaN to 0x7F.
 * Errors: as gqa_append_kv, and INVALID_ARG for a scale that is not finite
 * and positive. */
gqa_status gqa_append_kv_fp8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                             gqa_tensor k_new, gqa_tensor v_new,
                             gqa_tensor k_cache, gqa_tensor v_cache,
                             const int32_t* seqlens_k, float k_scale, float v_scale,
                             void* hip_stream);

/* gqa_decode against FP8 caches (arguments otherwise as gqa_decode).  The
 * matrix-core split-KV decode streams the codes (half the bytes of a 16-bit
 * cache), turns each 16-key unit into the plan's 16-bit type in LDS (exact),
 * folds k_scale into the softmax scale and v_scale into the normalization.
 * Needs a bf16 or fp16 plan of head size 64, 128 or 256 (UNSUPPORTED
 * otherwise).  Errors: as gqa_decode, and INVALID_ARG for a bad scale. */
gqa_status gqa_decode_fp8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                          gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                          const int32_t* seqlens_k, const float* head_sink,
                          float k_scale, float v_scale,
                          void* workspace, size_t ws_bytes, void* hip_stream);

/* INT8 KV cache with per-KV-head scales (the same pages name quantized
 * caches only as outside their scope; every rule here is this library's
 * reading).  The caches are int8 [B, Hkv, capacity, D] of symmetric codes in
 * -127 .. 127 with one fp32 scale per KV head for K and one for V, device
 * arrays [Hkv] (the same for every batch): K[b, g] = code * k_scales[g].
 * Strides of the caches are in bytes (= elements), multiples of 16.  The
 * scales must be finite and > 0 (device memory: not checked).
 *
 * gqa_append_kv_int8: gqa_append_kv that quantizes the new rows (the plan's
 * dtype): code = x * fp32(1 / scale[g]) computed in fp32, rounded to the
 * nearest integer with ties to even, clamped to +-127; NaN gives 0.
 * Errors: as gqa_append_kv, and INVALID_ARG for NULL scales. */
gqa_status gqa_append_kv_int8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                              gqa_tensor k_new, gqa_tensor v_new,
                              gqa_tensor k_cache, gqa_tensor v_cache,
                              const int32_t* seqlens_k, const float* k_scales, const float* v_scales,
                              void* hip_stream);

/* gqa_decode against INT8 caches (arguments otherwise as gqa_decode).  The
 * matrix-core split-KV decode streams the codes (half the bytes of a 16-bit
 * cache), turns each 16-key unit into the plan's 16-bit type in LDS (exact),
 * folds each KV head's k_scale into the softmax scale and its v_scale into
 * the normalization.  Needs a bf16 or fp16 plan of head size 64, 128 or 256
 * (UNSUPPORTED otherwise); a caller mask goes through gqa_decode_int8_masked.
 * Errors: as gqa_decode, INVALID_ARG for NULL scales, UNSUPPORTED for other
 *   plans or more than 2048 row tiles. */
gqa_status gqa_decode_int8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                           gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                           const int32_t* seqlens_k, const float* head_sink,
                           const float* k_scales, const float* v_scales,
                           void* workspace, size_t ws_bytes, void* hip_stream);

/* gqa_decode_fp8 with a caller mask over [B, Hq, curr, capacity], as for
 * gqa_decode_masked ("Attention Kernel Design", section "Layouts and
 * semantics": boolean or additive attention_bias broadcast over batch and
 * heads).  An additive value is added to the scaled logit of the dequantized
 * K (before softcap).  FP8 caches run only on the matrix-core decode, so the
 * mask's data and strides must be multiples of 4 bytes (boolean) or 16 bytes
 * and 4 elements (additive).
 * Errors: as gqa_decode_fp8 and gqa_decode_masked; UNSUPPORTED for another
 *   mask layout or a rolling cache. */
gqa_status gqa_decode_fp8_masked(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                 gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                 const int32_t* seqlens_k, const float* head_sink,
                                 float k_scale, float v_scale, const gqa_mask* mask,
                                 void* workspace, size_t ws_bytes, void* hip_stream);

/* gqa_decode_int8 with a caller mask over [B, Hq, curr, capacity], as for
 * gqa_decode_masked ("Attention Kernel Design", section "Layouts and
 * semantics": boolean or additive attention_bias broadcast over batch and
 * heads).  An additive value is added to the scaled logit of the dequantized
 * K (before softcap), whatever the head's k_scale.  The mask's data and
 * strides must be multiples of 4 bytes (boolean) or 16 bytes and 4 elements
 * (additive), as for gqa_decode_fp8_masked.
 * Errors: as gqa_decode_int8 and gqa_decode_masked; INVALID_ARG for a NULL
 *   mask; UNSUPPORTED for another mask layout or a rolling cache. */
gqa_status gqa_decode_int8_masked(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                  gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                  const int32_t* seqlens_k, const float* head_sink,
                                  const float* k_scales, const float* v_scales, const gqa_mask* mask,
                                  void* workspace, size_t ws_bytes, void* hip_stream);

/* The kernel that computed the attention of this thread's last call, so a
 * caller can tell a fast path from the slow one (the pages' streaming path
 * serves every accepted type, "Attention Kernel Design", section "Compute
 * paths"; here it is the fallback):
 *   GQA_PATH_NONE            no attention ran: a failed or empty call, or a
 *                            call without attention (append, rotary);
 *   GQA_PATH_MATRIX_PREFILL  the matrix-core prefill (bf16/fp16, head size
 *                            32/64/128/256);
 *   GQA_PATH_MATRIX_DECODE   the matrix-core split-KV decode (bf16/fp16, head
 *                            size 64/128/256, at most 2048 row tiles of 16
 *                            query rows per call);
 *   GQA_PATH_STREAMING       the one-wavefront-per-row fp32 kernel: fp32
 *                            plans, other head sizes, K/V row strides of 2^24
 *                            elements or more, masks whose layout the matrix
 *                            cores cannot read, decode calls with more row
 *                            tiles -- correct, and tens of times slower.
 * Set when the call enqueues its launch; thread-local. */
typedef enum {
  GQA_PATH_NONE = 0,
  GQA_PATH_MATRIX_PREFILL = 1,
  GQA_PATH_MATRIX_DECODE = 2,
  GQA_PATH_STREAMING = 3
} gqa_path;
gqa_path gqa_last_path(void);

/* Message for the last non-OK status returned on this thread ("" if none).
 * Every rejection names the argument and the rule it breaks: the "rejected
 * with specific messages" convention of "onnx: import GroupQueryAttention
 * decode steps and its internal rotary", section "What changed", and the
 * explicit failure of invalid pairings of "Attention Kernel Design", section
 * "Scheduling, precision, and invariants". */
const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_MI355X_H */
