// C ABI of libgqa_mi355x: attribute validation, the immutable plan, per-call
// argument checks and kernel dispatch.
//
// The split between a validated descriptor (built once) and a per-call plan
// (layout and strides, head mapping, lengths) follows "Attention Kernel
// Design", section "Descriptor and invocation plan"; explicit failure with a
// specific message for every unsupported or inconsistent input follows the
// same page, section "Scheduling, precision, and invariants", and the
// "rejected with specific messages" convention of "onnx: import
// GroupQueryAttention decode steps and its internal rotary", section "What
// changed".  Nothing here touches the device except the kernel launches.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "gqa.h"
#include "kernels.h"

#define GQA_API extern "C" __attribute__((visibility("default")))

struct gqa_plan_s {
  gqa_attrs attrs;
  float scale;  // resolved (0 -> 1/sqrt(D))
  int G;
  int32_t max_batch;
  int32_t max_q_len;
  int64_t max_kv_len;
  size_t ws_bytes;
};

namespace {

constexpr int64_t kMaxLen = int64_t(1) << 30;  // keeps every position in int32 arithmetic

thread_local std::string g_err;
// The kernel that computed the attention of this thread's last call (a
// gqa_path value): set when a launch is enqueued, reset at every entry.
thread_local int g_path = GQA_PATH_NONE;

gqa_status fail(gqa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

int elem_size(gqa_dtype t) { return t == GQA_F32 ? 4 : 2; }

gqa_status check_tensor(const char* name, const gqa_tensor& t, int esz) {
  if (t.data == nullptr) return fail(GQA_ERR_INVALID_ARG, "%s.data is NULL", name);
  if (reinterpret_cast<uintptr_t>(t.data) % 16 != 0)
    return fail(GQA_ERR_UNSUPPORTED, "%s.data must be 16-byte aligned", name);
  if (t.stride_b < 0 || t.stride_h < 0 || t.stride_s < 0)
    return fail(GQA_ERR_INVALID_ARG, "%s has a negative stride", name);
  const int64_t q = 16 / esz;
  if (t.stride_b % q || t.stride_h % q || t.stride_s % q)
    return fail(GQA_ERR_UNSUPPORTED, "%s strides must be multiples of %lld elements (16 bytes)", name,
                (long long)q);
  return GQA_OK;
}

hipError_t path_prefill_mfma(const gqa::AttnArgs& a, int dtype, bool softcap, hipStream_t stream) {
  g_path = GQA_PATH_MATRIX_PREFILL;
  return gqa::launch_prefill_mfma(a, dtype, softcap, stream);
}
hipError_t path_decode_mfma(const gqa::AttnArgs& a, int dtype, bool softcap, const gqa::DecodeGeometry& geo,
                            float* ws, hipStream_t stream) {
  g_path = GQA_PATH_MATRIX_DECODE;
  return gqa::launch_decode_mfma(a, dtype, softcap, geo, ws, stream);
}
hipError_t path_streaming(const gqa::AttnArgs& a, int dtype, hipStream_t stream) {
  g_path = GQA_PATH_STREAMING;
  return gqa::launch_attn_generic(a, dtype, stream);
}

gqa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GQA_OK;
  g_path = GQA_PATH_NONE;
  return fail(GQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

gqa::AttnArgs make_args(const gqa_plan_s* p, const gqa_tensor& q, const gqa_tensor& k,
                        const gqa_tensor& v, const gqa_tensor& o, int B, int Lq, int64_t Lk, int mode) {
  gqa::AttnArgs a{};
  a.q = q.data;
  a.k = k.data;
  a.v = v.data;
  a.o = o.data;
  a.q_sb = q.stride_b; a.q_sh = q.stride_h; a.q_ss = q.stride_s;
  a.k_sb = k.stride_b; a.k_sh = k.stride_h; a.k_ss = k.stride_s;
  a.v_sb = v.stride_b; a.v_sh = v.stride_h; a.v_ss = v.stride_s;
  a.o_sb = o.stride_b; a.o_sh = o.stride_h; a.o_ss = o.stride_s;
  a.B = B;
  a.Hq = p->attrs.num_heads;
  a.Hkv = p->attrs.kv_num_heads;
  a.G = p->G;
  a.D = p->attrs.head_size;
  a.Lq = Lq;
  a.Lk = (int32_t)Lk;
  a.mode = mode;
  a.causal = p->attrs.is_causal;
  a.window = p->attrs.local_window_size;
  a.use_sink = (p->attrs.use_head_sink || p->attrs.smooth_softmax) ? 1 : 0;
  a.ring = (mode == 1 && p->attrs.rolling_cache) ? (int32_t)Lk : 0;
  const float log2e = 1.4426950408889634f;
  a.scale_log2 = p->scale * log2e;
  a.scale_over_cap = p->attrs.softcap > 0 ? p->scale / p->attrs.softcap : 0.0f;
  a.cap_log2 = p->attrs.softcap > 0 ? p->attrs.softcap * log2e : 0.0f;
  a.inv_cap = p->attrs.softcap > 0 ? 1.0f / p->attrs.softcap : 0.0f;
  a.v_scale = 1.0f;
  return a;
}

// A rolling cache must still hold every key a step's rows may see.
gqa_status check_ring(const gqa_plan_s* p, int32_t curr, int64_t capacity) {
  if (!p->attrs.rolling_cache) return GQA_OK;
  const int64_t need = (int64_t)p->attrs.local_window_size + curr - 1;
  if (capacity < need)
    return fail(GQA_ERR_CAPACITY, "a rolling cache of %lld slots loses keys the step needs: capacity >= "
                "local_window_size + curr - 1 = %lld", (long long)capacity, (long long)need);
  return GQA_OK;
}

gqa_status check_sink(const gqa_plan_s* p, const float* head_sink) {
  if (p->attrs.use_head_sink && head_sink == nullptr)
    return fail(GQA_ERR_INVALID_ARG, "use_head_sink is set but head_sink is NULL");
  if (!p->attrs.use_head_sink && head_sink != nullptr)
    return fail(GQA_ERR_INVALID_ARG, "head_sink passed but the plan has use_head_sink = 0");
  return GQA_OK;
}

}  // namespace

GQA_API gqa_status gqa_plan(const gqa_attrs* attrs, int32_t max_batch, int32_t max_q_len,
                            int64_t max_kv_len, gqa_plan_t* out_plan) {
  g_path = GQA_PATH_NONE;
  if (out_plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "out_plan is NULL");
  *out_plan = nullptr;
  if (attrs == nullptr) return fail(GQA_ERR_INVALID_ARG, "attrs is NULL");
  const gqa_attrs& a = *attrs;
  if (a.num_heads <= 0) return fail(GQA_ERR_INVALID_ARG, "num_heads must be > 0 (got %d)", a.num_heads);
  if (a.kv_num_heads <= 0)
    return fail(GQA_ERR_INVALID_ARG, "kv_num_heads must be > 0 (got %d)", a.kv_num_heads);
  if (a.num_heads % a.kv_num_heads != 0)
    return fail(GQA_ERR_INVALID_ARG, "num_heads (%d) must be a multiple of kv_num_heads (%d)",
                a.num_heads, a.kv_num_heads);
  if (a.num_heads > 65535) return fail(GQA_ERR_UNSUPPORTED, "num_heads above 65535");
  if (a.dtype != GQA_F32 && a.dtype != GQA_F16 && a.dtype != GQA_BF16)
    return fail(GQA_ERR_INVALID_ARG, "dtype %d is not F32, F16 or BF16", (int)a.dtype);
  if (a.head_size < 8 || a.head_size > 256 || a.head_size % 8 != 0)
    return fail(GQA_ERR_UNSUPPORTED, "head_size %d: need a multiple of 8 in [8, 256]", a.head_size);
  if (!(a.scale >= 0.0f) || std::isinf(a.scale))
    return fail(GQA_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 = 1/sqrt(head_size))");
  if (a.local_window_size != -1 && a.local_window_size < 1)
    return fail(GQA_ERR_INVALID_ARG, "local_window_size must be -1 (off) or >= 1 (got %d)",
                a.local_window_size);
  if (!(a.softcap >= 0.0f) || std::isinf(a.softcap))
    return fail(GQA_ERR_INVALID_ARG, "softcap must be finite and >= 0 (0 = off)");
  if (a.smooth_softmax != 0 && a.smooth_softmax != 1)
    return fail(GQA_ERR_INVALID_ARG, "smooth_softmax must be 0 or 1");
  if (a.use_head_sink != 0 && a.use_head_sink != 1)
    return fail(GQA_ERR_INVALID_ARG, "use_head_sink must be 0 or 1");
  if (a.is_causal != 0 && a.is_causal != 1) return fail(GQA_ERR_INVALID_ARG, "is_causal must be 0 or 1");
  if (a.rolling_cache != 0 && a.rolling_cache != 1) return fail(GQA_ERR_INVALID_ARG, "rolling_cache must be 0 or 1");
  if (a.rolling_cache && a.local_window_size < 1)
    return fail(GQA_ERR_INVALID_ARG, "rolling_cache needs local_window_size >= 1 (the ring holds the window)");
  if (!a.is_causal && a.local_window_size != -1)
    return fail(GQA_ERR_INVALID_ARG, "local_window_size needs is_causal = 1 (the window is one-sided)");
  if (max_batch < 1 || max_q_len < 1 || max_kv_len < 1)
    return fail(GQA_ERR_INVALID_ARG, "max_batch, max_q_len and max_kv_len must be >= 1");
  if (max_batch > 65535) return fail(GQA_ERR_UNSUPPORTED, "max_batch above 65535");
  if (max_q_len > kMaxLen || max_kv_len > kMaxLen)
    return fail(GQA_ERR_UNSUPPORTED, "sequence lengths above 2^30");

  gqa_plan_s* p = new (std::nothrow) gqa_plan_s;
  if (p == nullptr) return fail(GQA_ERR_INVALID_ARG, "out of host memory");
  p->attrs = a;
  p->scale = a.scale > 0.0f ? a.scale : 1.0f / std::sqrt((float)a.head_size);
  p->G = a.num_heads / a.kv_num_heads;
  p->max_batch = max_batch;
  p->max_q_len = max_q_len;
  p->max_kv_len = max_kv_len;
  p->ws_bytes = 0;
  if (gqa::decode_mfma_supported(a.dtype, a.head_size)) {
    gqa::DecodeGeometry geo = gqa::decode_geometry(max_batch, a.kv_num_heads, p->G, max_q_len, a.head_size);
    p->ws_bytes = geo.ws_floats * sizeof(float);
  }
  *out_plan = p;
  return GQA_OK;
}

GQA_API void gqa_plan_destroy(gqa_plan_t plan) { delete plan; }

GQA_API size_t gqa_workspace_size(gqa_plan_t plan) { return plan ? plan->ws_bytes : 0; }

GQA_API gqa_status gqa_prefill(gqa_plan_t plan, int32_t B, int32_t Lq, int64_t Lk, gqa_tensor q,
                               gqa_tensor k, gqa_tensor v, gqa_tensor out,
                               const int64_t* nonpad_kv_seqlen, const float* head_sink,
                               void* workspace, size_t ws_bytes, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  (void)workspace;
  (void)ws_bytes;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || Lq < 0 || Lk < 0) return fail(GQA_ERR_INVALID_ARG, "B, Lq and Lk must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (Lq > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "Lq = %d exceeds the plan's max_q_len %d", Lq, plan->max_q_len);
  if (Lk > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "Lk = %lld exceeds the plan's max_kv_len %lld", (long long)Lk,
                (long long)plan->max_kv_len);
  gqa_status st = check_sink(plan, head_sink);
  if (st != GQA_OK) return st;
  if (B == 0 || Lq == 0) return GQA_OK;
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("out", out, esz)) != GQA_OK) return st;
  if (Lk > 0) {
    if ((st = check_tensor("k", k, esz)) != GQA_OK) return st;
    if ((st = check_tensor("v", v, esz)) != GQA_OK) return st;
  }
  gqa::AttnArgs a = make_args(plan, q, k, v, out, B, Lq, Lk, 0);
  a.nonpad = nonpad_kv_seqlen;
  a.head_sink = head_sink;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int dtype = (int)plan->attrs.dtype;
  hipError_t e;
  // the matrix-core kernel addresses a 64-row K/V tile with 32-bit offsets
  const bool small_strides = a.k_ss < (int64_t(1) << 24) && a.v_ss < (int64_t(1) << 24);
  if (Lk > 0 && small_strides && gqa::prefill_mfma_supported(dtype, plan->attrs.head_size))
    e = path_prefill_mfma(a, dtype, plan->attrs.softcap > 0, stream);
  else
    e = path_streaming(a, dtype, stream);
  return hip_status(e, "prefill launch");
}

GQA_API gqa_status gqa_append_kv(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                 gqa_tensor k_new, gqa_tensor v_new, gqa_tensor k_cache,
                                 gqa_tensor v_cache, const int32_t* seqlens_k, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  gqa_status st = check_ring(plan, curr, capacity);
  if (st != GQA_OK) return st;
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("k_new", k_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_new", v_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, esz)) != GQA_OK) return st;
  gqa::AppendArgs a{};
  a.k_new = k_new.data;
  a.v_new = v_new.data;
  a.k_cache = k_cache.data;
  a.v_cache = v_cache.data;
  a.kn_sb = k_new.stride_b * esz; a.kn_sh = k_new.stride_h * esz; a.kn_ss = k_new.stride_s * esz;
  a.vn_sb = v_new.stride_b * esz; a.vn_sh = v_new.stride_h * esz; a.vn_ss = v_new.stride_s * esz;
  a.kc_sb = k_cache.stride_b * esz; a.kc_sh = k_cache.stride_h * esz; a.kc_ss = k_cache.stride_s * esz;
  a.vc_sb = v_cache.stride_b * esz; a.vc_sh = v_cache.stride_h * esz; a.vc_ss = v_cache.stride_s * esz;
  a.seqlens = seqlens_k;
  a.B = B;
  a.Hkv = plan->attrs.kv_num_heads;
  a.curr = curr;
  a.row_bytes = plan->attrs.head_size * esz;
  a.capacity = (int32_t)capacity;
  a.rolling = plan->attrs.rolling_cache;
  return hip_status(gqa::launch_append_kv(a, reinterpret_cast<hipStream_t>(hip_stream)), "append_kv launch");
}

namespace {

// gqa_decode, gqa_decode_noalloc and gqa_append_decode: `scratch_ws` set
// means the workspace is the library's static scratch array (workspace /
// ws_bytes are ignored); `k_new` / `v_new` set means the step's append is
// part of the call.
gqa_status decode_impl(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                       gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out, const int32_t* seqlens_k,
                       const float* head_sink, void* workspace, size_t ws_bytes, void* hip_stream,
                       bool scratch_ws, const gqa_tensor* k_new = nullptr, const gqa_tensor* v_new = nullptr);

}  // namespace

GQA_API gqa_status gqa_decode(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                              gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                              const int32_t* seqlens_k, const float* head_sink, void* workspace,
                              size_t ws_bytes, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  return decode_impl(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, workspace,
                     ws_bytes, hip_stream, false);
}

GQA_API gqa_status gqa_decode_noalloc(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                                      gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                      const int32_t* seqlens_k, const float* head_sink, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  return decode_impl(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, nullptr, 0,
                     hip_stream, true);
}

GQA_API gqa_status gqa_append_decode(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                                     gqa_tensor k_new, gqa_tensor v_new, gqa_tensor k_cache, gqa_tensor v_cache,
                                     gqa_tensor out, const int32_t* seqlens_k, const float* head_sink,
                                     void* workspace, size_t ws_bytes, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  return decode_impl(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, workspace,
                     ws_bytes, hip_stream, false, &k_new, &v_new);
}

// ---------------------------------------------------------------------------
// The static decode scratch of gqa_decode_noalloc: one array per GPU, held
// until the process ends.  In host code `scratch` names a host-side stand-in
// only; kernels get the device address that hipGetSymbolAddress returns for
// the current device, taken once per device.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// The arrival counters at the front of a decode workspace must start at zero;
// every decode leaves them at zero.  A kernel rather than a memset, so that a
// call under stream capture records an ordinary kernel node.
__global__ void zero_words(unsigned* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address, set up on its first use: the symbol
// address is looked up and the counters are cleared on `stream`.
gqa_status scratch_for_current_device(hipStream_t stream, float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GQA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(GQA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    hipLaunchKernelGGL(zero_words, dim3(8), dim3(256), 0, stream, reinterpret_cast<unsigned*>(ptr),
                       gqa::kDecodeMaxTiles);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = reinterpret_cast<float*>(g_scratch_ptr[dev]);
  return GQA_OK;
}

gqa::AppendArgs append_args(const gqa_plan_s* plan, int32_t B, int32_t curr, int64_t capacity,
                            const gqa_tensor& k_new, const gqa_tensor& v_new, const gqa_tensor& k_cache,
                            const gqa_tensor& v_cache, const int32_t* seqlens_k) {
  const int esz = elem_size(plan->attrs.dtype);
  gqa::AppendArgs a{};
  a.k_new = k_new.data;
  a.v_new = v_new.data;
  a.k_cache = k_cache.data;
  a.v_cache = v_cache.data;
  a.kn_sb = k_new.stride_b * esz; a.kn_sh = k_new.stride_h * esz; a.kn_ss = k_new.stride_s * esz;
  a.vn_sb = v_new.stride_b * esz; a.vn_sh = v_new.stride_h * esz; a.vn_ss = v_new.stride_s * esz;
  a.kc_sb = k_cache.stride_b * esz; a.kc_sh = k_cache.stride_h * esz; a.kc_ss = k_cache.stride_s * esz;
  a.vc_sb = v_cache.stride_b * esz; a.vc_sh = v_cache.stride_h * esz; a.vc_ss = v_cache.stride_s * esz;
  a.seqlens = seqlens_k;
  a.B = B;
  a.Hkv = plan->attrs.kv_num_heads;
  a.curr = curr;
  a.row_bytes = plan->attrs.head_size * esz;
  a.capacity = (int32_t)capacity;
  a.rolling = plan->attrs.rolling_cache;
  return a;
}

gqa_status decode_impl(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                       gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out, const int32_t* seqlens_k,
                       const float* head_sink, void* workspace, size_t ws_bytes, void* hip_stream,
                       bool scratch_ws, const gqa_tensor* k_new, const gqa_tensor* v_new) {
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  gqa_status st = check_sink(plan, head_sink);
  if (st != GQA_OK) return st;
  if ((st = check_ring(plan, curr, capacity)) != GQA_OK) return st;
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, esz)) != GQA_OK) return st;
  if ((st = check_tensor("out", out, esz)) != GQA_OK) return st;
  const bool fused = k_new != nullptr;
  if (fused) {
    if ((st = check_tensor("k_new", *k_new, esz)) != GQA_OK) return st;
    if ((st = check_tensor("v_new", *v_new, esz)) != GQA_OK) return st;
  }
  gqa::AttnArgs a = make_args(plan, q, k_cache, v_cache, out, B, curr, capacity, 1);
  a.seqlens = seqlens_k;
  a.head_sink = head_sink;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int dtype = (int)plan->attrs.dtype;
  const bool softcap = plan->attrs.softcap > 0;
  // The append and the decode in one launch (the matrix-core decode); on the
  // other path, the append kernel and then the decode.
  const bool one_launch = fused && gqa::decode_mfma_supported(dtype, plan->attrs.head_size) &&
                          gqa::decode_geometry(B, a.Hkv, a.G, curr, a.D).fits;
  if (fused && one_launch) {
    a.fuse_append = 1;
    a.k_new = k_new->data;
    a.v_new = v_new->data;
    a.kn_sb = k_new->stride_b; a.kn_sh = k_new->stride_h; a.kn_ss = k_new->stride_s;
    a.vn_sb = v_new->stride_b; a.vn_sh = v_new->stride_h; a.vn_ss = v_new->stride_s;
  }
  auto append_first = [&]() -> gqa_status {
    if (!fused || one_launch) return GQA_OK;
    return hip_status(gqa::launch_append_kv(append_args(plan, B, curr, capacity, *k_new, *v_new, k_cache, v_cache,
                                                        seqlens_k), stream),
                      "append_kv launch");
  };
  if (gqa::decode_mfma_supported(dtype, plan->attrs.head_size)) {
    gqa::DecodeGeometry geo = gqa::decode_geometry(B, a.Hkv, a.G, curr, a.D);
    float* ws = reinterpret_cast<float*>(workspace);
    if (scratch_ws) {
      if (geo.fits) {
        const size_t need = gqa::decode_mfma_scratch_floats(a, dtype, softcap, geo) * sizeof(float);
        if (need > kScratchBytes)
          return fail(GQA_ERR_CAPACITY,
                      "gqa_decode_noalloc: this call needs %zu bytes of decode scratch, above the static "
                      "%zu-byte array (use gqa_decode with a workspace)", need, kScratchBytes);
        if ((st = scratch_for_current_device(stream, &ws)) != GQA_OK) return st;
      }
    } else {
      const size_t need = geo.ws_floats * sizeof(float);
      if (workspace == nullptr || ws_bytes < need)
        return fail(GQA_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes,
                    workspace ? "" : ", NULL");
      if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return fail(GQA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    if (geo.fits)
      return hip_status(path_decode_mfma(a, dtype, softcap, geo, ws, stream), "decode launch");
  }
  if ((st = append_first()) != GQA_OK) return st;
  return hip_status(path_streaming(a, dtype, stream), "decode launch");
}

}  // namespace

namespace {

gqa_status check_tables(const gqa_rotary_tables* t, int64_t need_pos) {
  if (t == nullptr) return fail(GQA_ERR_INVALID_ARG, "rotary tables are NULL");
  if (t->cos == nullptr || t->sin == nullptr) return fail(GQA_ERR_INVALID_ARG, "rotary cos/sin table is NULL");
  if (reinterpret_cast<uintptr_t>(t->cos) % 16 != 0 || reinterpret_cast<uintptr_t>(t->sin) % 16 != 0)
    return fail(GQA_ERR_UNSUPPORTED, "rotary tables must be 16-byte aligned");
  if (t->max_pos < 1) return fail(GQA_ERR_INVALID_ARG, "rotary max_pos must be >= 1");
  if (need_pos > t->max_pos)
    return fail(GQA_ERR_CAPACITY, "positions up to %lld need rotary tables of at least %lld rows (got %lld)",
                (long long)need_pos - 1, (long long)need_pos, (long long)t->max_pos);
  return GQA_OK;
}

void set_job(gqa::RotaryArgs& a, int j, const gqa_tensor& src, const gqa_tensor& dst, int H, int turn,
             int to_slot) {
  a.src[j] = src.data;
  a.dst[j] = dst.data;
  a.s_sb[j] = src.stride_b; a.s_sh[j] = src.stride_h; a.s_ss[j] = src.stride_s;
  a.d_sb[j] = dst.stride_b; a.d_sh[j] = dst.stride_h; a.d_ss[j] = dst.stride_s;
  a.H[j] = H;
  a.turn[j] = turn;
  a.to_slot[j] = to_slot;
}

}  // namespace

GQA_API gqa_status gqa_apply_rotary(gqa_plan_t plan, int32_t B, int32_t H, int32_t L, int64_t pos0,
                                    gqa_tensor x, gqa_tensor y, const gqa_rotary_tables* tables,
                                    void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || H < 0 || L < 0 || pos0 < 0) return fail(GQA_ERR_INVALID_ARG, "B, H, L and pos0 must be >= 0");
  if (B > 65535 || H > 65535) return fail(GQA_ERR_UNSUPPORTED, "B and H must be <= 65535");
  if (L > kMaxLen || pos0 > kMaxLen) return fail(GQA_ERR_UNSUPPORTED, "positions above 2^30");
  gqa_status st = check_tables(tables, pos0 + L);
  if (st != GQA_OK) return st;
  if (B == 0 || H == 0 || L == 0) return GQA_OK;
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("x", x, esz)) != GQA_OK) return st;
  if ((st = check_tensor("y", y, esz)) != GQA_OK) return st;
  gqa::RotaryArgs a{};
  set_job(a, 0, x, y, H, 1, 0);
  a.jobs = 1;
  a.B = B;
  a.L = L;
  a.D = plan->attrs.head_size;
  a.pos0 = pos0;
  a.seqlens = nullptr;
  a.cos = tables->cos;
  a.sin = tables->sin;
  a.max_pos = tables->max_pos;
  return hip_status(gqa::launch_rotary(a, (int)plan->attrs.dtype, reinterpret_cast<hipStream_t>(hip_stream)),
                    "rotary launch");
}

GQA_API gqa_status gqa_prefill_rotary(gqa_plan_t plan, int32_t B, int32_t Lq, int64_t Lk, gqa_tensor q,
                                      gqa_tensor k, gqa_tensor v, gqa_tensor out,
                                      const int64_t* nonpad_kv_seqlen, const float* head_sink,
                                      const gqa_rotary_tables* tables, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || Lq < 0 || Lk < 0) return fail(GQA_ERR_INVALID_ARG, "B, Lq and Lk must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (Lq > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "Lq = %d exceeds the plan's max_q_len %d", Lq, plan->max_q_len);
  if (Lk > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "Lk = %lld exceeds the plan's max_kv_len %lld", (long long)Lk,
                (long long)plan->max_kv_len);
  gqa_status st = check_sink(plan, head_sink);
  if (st != GQA_OK) return st;
  // query row i sits at position Lk - Lq + i, at most Lk - 1
  if ((st = check_tables(tables, Lk)) != GQA_OK) return st;
  const int dtype = (int)plan->attrs.dtype;
  if (!gqa::prefill_mfma_supported(dtype, plan->attrs.head_size))
    return fail(GQA_ERR_UNSUPPORTED, "gqa_prefill_rotary needs a bf16 or fp16 plan of head size 32, 64, 128 or "
                "256 (otherwise call gqa_apply_rotary, then gqa_prefill)");
  if (B == 0 || Lq == 0) return GQA_OK;
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("out", out, esz)) != GQA_OK) return st;
  if (Lk > 0) {
    if ((st = check_tensor("k", k, esz)) != GQA_OK) return st;
    if ((st = check_tensor("v", v, esz)) != GQA_OK) return st;
  }
  gqa::AttnArgs a = make_args(plan, q, k, v, out, B, Lq, Lk, 0);
  if (a.k_ss >= (int64_t(1) << 24) || a.v_ss >= (int64_t(1) << 24))
    return fail(GQA_ERR_UNSUPPORTED, "gqa_prefill_rotary: K/V row strides of 2^24 elements or more");
  a.nonpad = nonpad_kv_seqlen;
  a.head_sink = head_sink;
  a.rot_cos = tables->cos;
  a.rot_sin = tables->sin;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  if (Lk == 0) return hip_status(path_streaming(a, dtype, stream), "prefill launch");  // zeros
  return hip_status(path_prefill_mfma(a, dtype, plan->attrs.softcap > 0, stream), "prefill_rotary launch");
}

GQA_API gqa_status gqa_append_kv_rotary(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                        gqa_tensor q, gqa_tensor q_rot, gqa_tensor k_new, gqa_tensor v_new,
                                        gqa_tensor k_cache, gqa_tensor v_cache, const int32_t* seqlens_k,
                                        const gqa_rotary_tables* tables, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  // every position is a cache slot below capacity (a rolling cache's positions
  // pass it: rows at or past max_pos are left unwritten by the kernel)
  gqa_status st = check_tables(tables, plan->attrs.rolling_cache ? 1 : capacity);
  if (st != GQA_OK) return st;
  if ((st = check_ring(plan, curr, capacity)) != GQA_OK) return st;
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("q_rot", q_rot, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_new", k_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_new", v_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, esz)) != GQA_OK) return st;
  gqa::RotaryArgs a{};
  set_job(a, 0, k_new, k_cache, plan->attrs.kv_num_heads, 1, 1);
  set_job(a, 1, v_new, v_cache, plan->attrs.kv_num_heads, 0, 1);
  set_job(a, 2, q, q_rot, plan->attrs.num_heads, 1, 0);
  a.jobs = 3;
  a.B = B;
  a.L = curr;
  a.D = plan->attrs.head_size;
  a.pos0 = 0;
  a.seqlens = seqlens_k;
  a.capacity = (int32_t)capacity;
  a.rolling = plan->attrs.rolling_cache;
  a.cos = tables->cos;
  a.sin = tables->sin;
  a.max_pos = tables->max_pos;
  return hip_status(gqa::launch_rotary(a, (int)plan->attrs.dtype, reinterpret_cast<hipStream_t>(hip_stream)),
                    "append_kv_rotary launch");
}

namespace {

gqa_status set_mask(gqa::AttnArgs& a, const gqa_mask* m) {
  if (m == nullptr) return fail(GQA_ERR_INVALID_ARG, "mask is NULL");
  if (m->data == nullptr) return fail(GQA_ERR_INVALID_ARG, "mask.data is NULL");
  if (m->kind != GQA_MASK_BOOL && m->kind != GQA_MASK_ADDITIVE)
    return fail(GQA_ERR_INVALID_ARG, "mask.kind %d is not GQA_MASK_BOOL or GQA_MASK_ADDITIVE", (int)m->kind);
  if (m->stride_b < 0 || m->stride_h < 0 || m->stride_q < 0)
    return fail(GQA_ERR_INVALID_ARG, "mask has a negative stride");
  if (m->kind == GQA_MASK_ADDITIVE && reinterpret_cast<uintptr_t>(m->data) % 4 != 0)
    return fail(GQA_ERR_UNSUPPORTED, "an additive mask must be 4-byte aligned");
  a.mask = m->data;
  a.m_sb = m->stride_b;
  a.m_sh = m->stride_h;
  a.m_sq = m->stride_q;
  a.mask_kind = (int32_t)m->kind;
  return GQA_OK;
}

}  // namespace

GQA_API gqa_status gqa_prefill_masked(gqa_plan_t plan, int32_t B, int32_t Lq, int64_t Lk, gqa_tensor q,
                                      gqa_tensor k, gqa_tensor v, gqa_tensor out,
                                      const int64_t* nonpad_kv_seqlen, const float* head_sink,
                                      const gqa_mask* mask, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || Lq < 0 || Lk < 0) return fail(GQA_ERR_INVALID_ARG, "B, Lq and Lk must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (Lq > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "Lq = %d exceeds the plan's max_q_len %d", Lq, plan->max_q_len);
  if (Lk > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "Lk = %lld exceeds the plan's max_kv_len %lld", (long long)Lk,
                (long long)plan->max_kv_len);
  gqa_status st = check_sink(plan, head_sink);
  if (st != GQA_OK) return st;
  gqa::AttnArgs a = make_args(plan, q, k, v, out, B, Lq, Lk, 0);
  if ((st = set_mask(a, mask)) != GQA_OK) return st;
  if (B == 0 || Lq == 0) return GQA_OK;
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("out", out, esz)) != GQA_OK) return st;
  if (Lk > 0) {
    if ((st = check_tensor("k", k, esz)) != GQA_OK) return st;
    if ((st = check_tensor("v", v, esz)) != GQA_OK) return st;
  }
  a.nonpad = nonpad_kv_seqlen;
  a.head_sink = head_sink;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int dtype = (int)plan->attrs.dtype;
  // Masks whose runs of 8 keys are aligned (boolean: rows at multiples of 8
  // bytes; additive: of 16 bytes) run on the matrix-core kernel; other
  // layouts on the streaming kernel.
  const bool small_strides = a.k_ss < (int64_t(1) << 24) && a.v_ss < (int64_t(1) << 24);
  const bool boolean = mask->kind == GQA_MASK_BOOL;
  const int64_t ealign = boolean ? 8 : 4;  // elements per aligned unit (8 or 16 bytes)
  const bool aligned = reinterpret_cast<uintptr_t>(mask->data) % (boolean ? 8 : 16) == 0 &&
                       mask->stride_b % ealign == 0 && mask->stride_h % ealign == 0 &&
                       mask->stride_q % ealign == 0;
  a.bias_mul = 1.0f / plan->scale;
  if (Lk > 0 && small_strides && gqa::prefill_mfma_supported(dtype, plan->attrs.head_size) &&
      aligned)
    return hip_status(path_prefill_mfma(a, dtype, plan->attrs.softcap > 0.0f, stream),
                      "masked prefill launch");
  return hip_status(path_streaming(a, dtype, stream), "masked prefill launch");
}

GQA_API gqa_status gqa_decode_masked(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                                     gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                     const int32_t* seqlens_k, const float* head_sink, const gqa_mask* mask,
                                     void* workspace, size_t ws_bytes, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  if (plan->attrs.rolling_cache)
    return fail(GQA_ERR_UNSUPPORTED, "a decode mask indexes keys by position: not with a rolling cache");
  gqa_status st = check_sink(plan, head_sink);
  if (st != GQA_OK) return st;
  gqa::AttnArgs a = make_args(plan, q, k_cache, v_cache, out, B, curr, capacity, 1);
  if ((st = set_mask(a, mask)) != GQA_OK) return st;
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, esz)) != GQA_OK) return st;
  if ((st = check_tensor("out", out, esz)) != GQA_OK) return st;
  a.seqlens = seqlens_k;
  a.head_sink = head_sink;
  a.bias_mul = 1.0f / plan->scale;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int dtype = (int)plan->attrs.dtype;
  // The matrix-core decode reads a lane's 4 mask entries of a unit as one
  // aligned load: boolean rows at multiples of 4 bytes, additive ones of 16.
  const bool boolean = mask->kind == GQA_MASK_BOOL;
  const bool aligned = reinterpret_cast<uintptr_t>(mask->data) % (boolean ? 4 : 16) == 0 &&
                       mask->stride_b % 4 == 0 && mask->stride_h % 4 == 0 && mask->stride_q % 4 == 0;
  if (workspace != nullptr && aligned && gqa::decode_mfma_supported(dtype, plan->attrs.head_size)) {
    gqa::DecodeGeometry geo = gqa::decode_geometry(B, a.Hkv, a.G, curr, a.D);
    const size_t need = geo.ws_floats * sizeof(float);
    if (ws_bytes < need) return fail(GQA_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(GQA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (geo.fits)
      return hip_status(path_decode_mfma(a, dtype, plan->attrs.softcap > 0.0f, geo,
                                                reinterpret_cast<float*>(workspace), stream),
                        "masked decode launch");
  }
  return hip_status(path_streaming(a, dtype, stream), "masked decode launch");
}

namespace {

gqa_status check_scales(float k_scale, float v_scale) {
  if (!(k_scale > 0.0f) || !std::isfinite(k_scale) || !(v_scale > 0.0f) || !std::isfinite(v_scale))
    return fail(GQA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  return GQA_OK;
}

// The FP8 cache path exists for the matrix-core decode's types and head sizes.
gqa_status check_fp8_plan(const gqa_plan_s* p) {
  const int dtype = (int)p->attrs.dtype;
  if (!gqa::decode_mfma_supported(dtype, p->attrs.head_size))
    return fail(GQA_ERR_UNSUPPORTED, "FP8 caches need a bf16 or fp16 plan of head size 64, 128 or 256");
  return GQA_OK;
}

}  // namespace

GQA_API gqa_status gqa_append_kv_fp8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                     gqa_tensor k_new, gqa_tensor v_new, gqa_tensor k_cache,
                                     gqa_tensor v_cache, const int32_t* seqlens_k, float k_scale,
                                     float v_scale, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  gqa_status st = check_scales(k_scale, v_scale);
  if (st != GQA_OK) return st;
  if ((st = check_ring(plan, curr, capacity)) != GQA_OK) return st;
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("k_new", k_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_new", v_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, 1)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, 1)) != GQA_OK) return st;
  gqa::AppendArgs a{};
  a.k_new = k_new.data;
  a.v_new = v_new.data;
  a.k_cache = k_cache.data;
  a.v_cache = v_cache.data;
  a.kn_sb = k_new.stride_b * esz; a.kn_sh = k_new.stride_h * esz; a.kn_ss = k_new.stride_s * esz;
  a.vn_sb = v_new.stride_b * esz; a.vn_sh = v_new.stride_h * esz; a.vn_ss = v_new.stride_s * esz;
  a.kc_sb = k_cache.stride_b; a.kc_sh = k_cache.stride_h; a.kc_ss = k_cache.stride_s;
  a.vc_sb = v_cache.stride_b; a.vc_sh = v_cache.stride_h; a.vc_ss = v_cache.stride_s;
  a.seqlens = seqlens_k;
  a.B = B;
  a.Hkv = plan->attrs.kv_num_heads;
  a.curr = curr;
  a.row_bytes = plan->attrs.head_size * esz;
  a.capacity = (int32_t)capacity;
  a.rolling = plan->attrs.rolling_cache;
  a.k_rcp = 1.0f / k_scale;
  a.v_rcp = 1.0f / v_scale;
  return hip_status(gqa::launch_append_kv_fp8(a, (int)plan->attrs.dtype, reinterpret_cast<hipStream_t>(hip_stream)),
                    "append_kv_fp8 launch");
}

namespace {

// gqa_decode_fp8 and gqa_decode_fp8_masked (mask NULL for the former).
gqa_status decode_fp8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                      gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out, const int32_t* seqlens_k,
                      const float* head_sink, float k_scale, float v_scale, const gqa_mask* mask,
                      void* workspace, size_t ws_bytes, void* hip_stream) {
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  gqa_status st = check_fp8_plan(plan);
  if (st != GQA_OK) return st;
  if ((st = check_scales(k_scale, v_scale)) != GQA_OK) return st;
  if ((st = check_sink(plan, head_sink)) != GQA_OK) return st;
  if ((st = check_ring(plan, curr, capacity)) != GQA_OK) return st;
  if (mask != nullptr && plan->attrs.rolling_cache)
    return fail(GQA_ERR_UNSUPPORTED, "a decode mask indexes keys by position: not with a rolling cache");
  gqa::AttnArgs a = make_args(plan, q, k_cache, v_cache, out, B, curr, capacity, 1);
  if (mask != nullptr) {
    if ((st = set_mask(a, mask)) != GQA_OK) return st;
    // the matrix-core decode reads a lane's 4 mask entries of a unit as one
    // aligned load; FP8 caches have no other kernel
    const bool boolean = mask->kind == GQA_MASK_BOOL;
    if (reinterpret_cast<uintptr_t>(mask->data) % (boolean ? 4 : 16) != 0 || mask->stride_b % 4 != 0 ||
        mask->stride_h % 4 != 0 || mask->stride_q % 4 != 0)
      return fail(GQA_ERR_UNSUPPORTED,
                  "FP8 caches need a mask whose data and strides are multiples of %d bytes and 4 elements",
                  boolean ? 4 : 16);
  }
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, 1)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, 1)) != GQA_OK) return st;
  if ((st = check_tensor("out", out, esz)) != GQA_OK) return st;
  a.seqlens = seqlens_k;
  a.head_sink = head_sink;
  a.kv_fp8 = 1;
  a.scale_log2 *= k_scale;      // scores of the codes times k_scale
  a.scale_over_cap *= k_scale;
  a.bias_mul = 1.0f / (plan->scale * k_scale);  // an additive mask value in code-score units
  a.v_scale = v_scale;
  gqa::DecodeGeometry geo = gqa::decode_geometry(B, a.Hkv, a.G, curr, a.D);
  const size_t need = geo.ws_floats * sizeof(float);
  if (workspace == nullptr || ws_bytes < need)
    return fail(GQA_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes,
                workspace ? "" : ", NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(GQA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (!geo.fits)
    return fail(GQA_ERR_UNSUPPORTED, "FP8 caches: at most %d row tiles per call", 2048);
  return hip_status(path_decode_mfma(a, (int)plan->attrs.dtype, plan->attrs.softcap > 0, geo,
                                            reinterpret_cast<float*>(workspace), reinterpret_cast<hipStream_t>(hip_stream)),
                    "decode_fp8 launch");
}

}  // namespace

GQA_API gqa_status gqa_decode_fp8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                                  gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                  const int32_t* seqlens_k, const float* head_sink, float k_scale,
                                  float v_scale, void* workspace, size_t ws_bytes, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  return decode_fp8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scale, v_scale,
                    nullptr, workspace, ws_bytes, hip_stream);
}

GQA_API gqa_status gqa_decode_fp8_masked(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                         gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                         const int32_t* seqlens_k, const float* head_sink, float k_scale,
                                         float v_scale, const gqa_mask* mask, void* workspace, size_t ws_bytes,
                                         void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (mask == nullptr) return fail(GQA_ERR_INVALID_ARG, "mask is NULL");
  return decode_fp8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scale, v_scale,
                    mask, workspace, ws_bytes, hip_stream);
}

GQA_API gqa_status gqa_append_kv_int8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                      gqa_tensor k_new, gqa_tensor v_new, gqa_tensor k_cache,
                                      gqa_tensor v_cache, const int32_t* seqlens_k, const float* k_scales,
                                      const float* v_scales, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  if (k_scales == nullptr || v_scales == nullptr) return fail(GQA_ERR_INVALID_ARG, "k_scales and v_scales are required");
  gqa_status st = check_ring(plan, curr, capacity);
  if (st != GQA_OK) return st;
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("k_new", k_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("v_new", v_new, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, 1)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, 1)) != GQA_OK) return st;
  gqa::AppendArgs a = append_args(plan, B, curr, capacity, k_new, v_new, k_cache, v_cache, seqlens_k);
  // code caches: strides are bytes already
  a.kc_sb = k_cache.stride_b; a.kc_sh = k_cache.stride_h; a.kc_ss = k_cache.stride_s;
  a.vc_sb = v_cache.stride_b; a.vc_sh = v_cache.stride_h; a.vc_ss = v_cache.stride_s;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  return hip_status(gqa::launch_append_kv_int8(a, (int)plan->attrs.dtype, reinterpret_cast<hipStream_t>(hip_stream)),
                    "append_kv_int8 launch");
}

namespace {
gqa_status decode_int8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                       gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out, const int32_t* seqlens_k,
                       const float* head_sink, const float* k_scales, const float* v_scales, const gqa_mask* mask,
                       void* workspace, size_t ws_bytes, void* hip_stream) {
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  if (B < 0 || curr < 0 || capacity < 0) return fail(GQA_ERR_INVALID_ARG, "B, curr and capacity must be >= 0");
  if (B > plan->max_batch) return fail(GQA_ERR_CAPACITY, "B = %d exceeds the plan's max_batch %d", B, plan->max_batch);
  if (curr > plan->max_q_len)
    return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the plan's max_q_len %d", curr, plan->max_q_len);
  if (capacity > plan->max_kv_len)
    return fail(GQA_ERR_CAPACITY, "capacity = %lld exceeds the plan's max_kv_len %lld", (long long)capacity,
                (long long)plan->max_kv_len);
  if (curr > capacity) return fail(GQA_ERR_CAPACITY, "curr = %d exceeds the cache capacity %lld", curr, (long long)capacity);
  gqa_status st = check_fp8_plan(plan);
  if (st != GQA_OK) return fail(GQA_ERR_UNSUPPORTED, "INT8 caches need a bf16 or fp16 plan of head size 64, 128 or 256");
  if (k_scales == nullptr || v_scales == nullptr) return fail(GQA_ERR_INVALID_ARG, "k_scales and v_scales are required");
  if ((st = check_sink(plan, head_sink)) != GQA_OK) return st;
  if ((st = check_ring(plan, curr, capacity)) != GQA_OK) return st;
  if (mask != nullptr && plan->attrs.rolling_cache)
    return fail(GQA_ERR_UNSUPPORTED, "a decode mask indexes keys by position: not with a rolling cache");
  gqa::AttnArgs a = make_args(plan, q, k_cache, v_cache, out, B, curr, capacity, 1);
  if (mask != nullptr) {
    if ((st = set_mask(a, mask)) != GQA_OK) return st;
    // the matrix-core decode reads a lane's 4 mask entries of a unit as one
    // aligned load; INT8 caches have no other kernel
    const bool boolean = mask->kind == GQA_MASK_BOOL;
    if (reinterpret_cast<uintptr_t>(mask->data) % (boolean ? 4 : 16) != 0 || mask->stride_b % 4 != 0 ||
        mask->stride_h % 4 != 0 || mask->stride_q % 4 != 0)
      return fail(GQA_ERR_UNSUPPORTED,
                  "INT8 caches need a mask whose data and strides are multiples of %d bytes and 4 elements",
                  boolean ? 4 : 16);
  }
  if (B == 0 || curr == 0) return GQA_OK;
  if (seqlens_k == nullptr) return fail(GQA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const int esz = elem_size(plan->attrs.dtype);
  if ((st = check_tensor("q", q, esz)) != GQA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, 1)) != GQA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, 1)) != GQA_OK) return st;
  if ((st = check_tensor("out", out, esz)) != GQA_OK) return st;
  a.seqlens = seqlens_k;
  a.head_sink = head_sink;
  a.kv_fp8 = 2;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.bias_mul = 1.0f / plan->scale;  // divided by the head's k_scale in the kernel (code-score units)
  gqa::DecodeGeometry geo = gqa::decode_geometry(B, a.Hkv, a.G, curr, a.D);
  const size_t need = geo.ws_floats * sizeof(float);
  if (workspace == nullptr || ws_bytes < need)
    return fail(GQA_ERR_INVALID_ARG, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes,
                workspace ? "" : ", NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(GQA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (!geo.fits) return fail(GQA_ERR_UNSUPPORTED, "INT8 caches: at most %d row tiles per call", gqa::kDecodeMaxTiles);
  return hip_status(path_decode_mfma(a, (int)plan->attrs.dtype, plan->attrs.softcap > 0, geo,
                                     reinterpret_cast<float*>(workspace), reinterpret_cast<hipStream_t>(hip_stream)),
                    "decode_int8 launch");
}
}  // namespace

GQA_API gqa_status gqa_decode_int8(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity, gqa_tensor q,
                                   gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                   const int32_t* seqlens_k, const float* head_sink, const float* k_scales,
                                   const float* v_scales, void* workspace, size_t ws_bytes, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  return decode_int8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scales, v_scales,
                     nullptr, workspace, ws_bytes, hip_stream);
}

GQA_API gqa_status gqa_decode_int8_masked(gqa_plan_t plan, int32_t B, int32_t curr, int64_t capacity,
                                          gqa_tensor q, gqa_tensor k_cache, gqa_tensor v_cache, gqa_tensor out,
                                          const int32_t* seqlens_k, const float* head_sink, const float* k_scales,
                                          const float* v_scales, const gqa_mask* mask, void* workspace,
                                          size_t ws_bytes, void* hip_stream) {
  g_path = GQA_PATH_NONE;
  if (mask == nullptr) return fail(GQA_ERR_INVALID_ARG, "mask is NULL");
  return decode_int8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scales, v_scales,
                     mask, workspace, ws_bytes, hip_stream);
}

GQA_API const char* gqa_last_error(void) { return g_err.c_str(); }

GQA_API gqa_path gqa_last_path(void) { return (gqa_path)g_path; }
