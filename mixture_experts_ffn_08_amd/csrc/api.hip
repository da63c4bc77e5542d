// C ABI of libmoe.so (declared in include/moe.h): argument checks on the host,
// then the kernel launchers.  Nothing is enqueued unless every check passes.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;
// Set by moe_layer_forward while it runs every call's checks: the entry points
// then return after their checks, before enqueueing anything.
thread_local bool g_check_only = false;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
int elem_bytes(int dt) { return dt == MOE_BF16 ? 2 : 4; }

// Row width rule: multiples of 8 (fp32) or 128 (bf16).
int width_check(const char* fn, const char* name, int v, int dt) {
  if (v <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: %s = %d must be positive", fn, name, v);
  const int m = dt == MOE_BF16 ? 128 : 8;
  if (v % m != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: %s = %d must be a multiple of %d for %s", fn, name, v, m,
                dt == MOE_BF16 ? "bf16" : "fp32");
  return MOE_OK;
}

int experts_check(const char* fn, int E, int k) {
  if (E < 1 || E > MOE_MAX_EXPERTS)
    return fail(E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED, "%s: E = %d outside [1, %d]", fn, E,
                MOE_MAX_EXPERTS);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, E = %d]", fn, k, E);
  return MOE_OK;
}

int assignments_check(const char* fn, int T, int k) {
  if ((int64_t)T * k > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k = %lld exceeds 2^31-1", fn,
                                              (long long)T * k);
  return MOE_OK;
}

#define CHECK(x)                  \
  do {                            \
    const int _s = (x);           \
    if (_s != MOE_OK) return _s;  \
  } while (0)
#define NEED(p, fn)                                                                           \
  do {                                                                                        \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: %s must not be NULL", fn, #p); \
  } while (0)

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int64_t moe_capacity(int64_t T, int k, int E, double phi) {
  if (!(phi >= 0.0) || isinf(phi) || T < 0 || k < 1 || E < 1) return -1;
  // phi = m * 2^ex exactly, m an integer below 2^53.
  int ex = 0;
  const double fr = frexp(phi, &ex);
  int64_t m = (int64_t)ldexp(fr, 53);
  ex -= 53;
  while (m != 0 && (m & 1) == 0) {
    m >>= 1;
    ++ex;
  }
  // C = ceil(m * 2^ex * T * k / E), in 128-bit integers.
  __int128 num = (__int128)m * T * k;
  __int128 den = E;
  if (ex >= 0) {
    if (ex > 40) return INT64_MAX;
    num <<= ex;
  } else {
    if (-ex >= 120) return num == 0 ? 0 : 1;
    den <<= -ex;
  }
  const __int128 c = (num + den - 1) / den;
  return c > (__int128)INT64_MAX ? INT64_MAX : (int64_t)c;
}

size_t moe_permute_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || k < 1 || E < 1) return 0;
  const size_t nblk = (size_t)moe::permute_blocks(T, k);
  return 2 * round_up(nblk * (size_t)E * sizeof(int32_t), 256);
}

size_t moe_stats_workspace_bytes(int T, int E) {
  if (T <= 0 || E < 1) return 0;
  return round_up((size_t)moe::stats_blocks(T) * (size_t)E * sizeof(float), 256);
}

int moe_route(const void* x, const void* w_router, const float* logit_bias, const float* select_bias, int dtype,
              int T, int d, int E, int k, int mode, int renorm, float* logits, int32_t* topk_idx, float* topk_w,
              int32_t* near_tie, hipStream_t stream) {
  static const char* fn = "moe_route";
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (mode != MOE_SOFTMAX_THEN_TOPK && mode != MOE_TOPK_THEN_SOFTMAX && mode != MOE_SIGMOID_THEN_TOPK)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown score mode %d", fn, mode);
  CHECK(experts_check(fn, E, k));
  if (d <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: d = %d must be positive", fn, d);
  CHECK(width_check(fn, "d", d, dtype));
  CHECK(assignments_check(fn, T, k));
  if (T == 0) return ok();
  NEED(x, fn);
  NEED(w_router, fn);
  NEED(logits, fn);
  NEED(topk_idx, fn);
  NEED(topk_w, fn);
  NEED(near_tie, fn);
  if (g_check_only) return ok();
  moe::RouteArgs a{x, w_router, logit_bias, select_bias, dtype, T, d, E, k, mode, renorm ? 1 : 0,
                   logits, topk_idx, topk_w, near_tie};
  return hip_status(moe::launch_route(a, stream), fn);
}

int moe_bias_update(const int32_t* counts, int T, int k, int E, float rate, float* select_bias,
                    hipStream_t stream) {
  static const char* fn = "moe_bias_update";
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  CHECK(experts_check(fn, E, k));
  CHECK(assignments_check(fn, T, k));
  if (!(rate == rate)) return fail(MOE_ERR_INVALID_ARG, "%s: rate is NaN", fn);
  if (T == 0) return ok();
  NEED(counts, fn);
  NEED(select_bias, fn);
  return hip_status(moe::launch_bias_update(counts, T, k, E, rate, select_bias, stream), fn);
}

}  // extern "C"

namespace {

// Checks of moe_permute and moe_permute_noalloc on everything but the workspace:
// the sizes first (T = 0 is then a valid no-op), then the pointers.
int permute_size_check(const char* fn, int T, int k, int E, int dtype, int d) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  CHECK(experts_check(fn, E, k));
  if (d <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: d = %d must be positive", fn, d);
  if (d % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: d = %d must be a multiple of 8", fn, d);
  CHECK(assignments_check(fn, T, k));
  return MOE_OK;
}

int permute_pointer_check(const char* fn, const int32_t* topk_idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* row_of, int32_t* perm_token, void* x_perm) {
  NEED(topk_idx, fn);
  NEED(counts, fn);
  NEED(offsets, fn);
  NEED(row_of, fn);
  NEED(perm_token, fn);
  if (x_perm != nullptr) NEED(x, fn);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_permute(const int32_t* topk_idx, int T, int k, int E, int64_t capacity, const void* x, int dtype,
                int d, int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* perm_token, void* x_perm,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "moe_permute";
  CHECK(permute_size_check(fn, T, k, E, dtype, d));
  if (T == 0) return ok();
  CHECK(permute_pointer_check(fn, topk_idx, x, counts, offsets, row_of, perm_token, x_perm));
  const size_t need = moe_permute_workspace_bytes(T, k, E);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if (g_check_only) return ok();
  const size_t half = need / 2;
  moe::PermuteArgs a{topk_idx, T, k, E, capacity < 0 ? -1 : capacity, x, d * elem_bytes(dtype), counts,
                     offsets, row_of, perm_token, x_perm, static_cast<int32_t*>(workspace),
                     reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + half), 0};
  return hip_status(moe::launch_permute(a, stream), fn);
}

}  // extern "C"

// Scratch of moe_permute_noalloc: the per-block expert histograms and running
// bases that moe_permute keeps in its workspace argument.  One copy per device,
// held from the library's load until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first
// call on that device, with that device current).
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || p == nullptr)
      return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  r != hipSuccess ? hipGetErrorString(r) : "null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, int64_t capacity, const void* x, int dtype,
                        int d, int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* perm_token,
                        void* x_perm, hipStream_t stream) {
  static const char* fn = "moe_permute_noalloc";
  CHECK(permute_size_check(fn, T, k, E, dtype, d));
  if (T == 0) return ok();
  CHECK(permute_pointer_check(fn, topk_idx, x, counts, offsets, row_of, perm_token, x_perm));
  const size_t need = moe_permute_workspace_bytes(T, k, E);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: T = %d, k = %d, E = %d need %zu bytes of scratch, more than the %zu this entry point "
                "holds; call moe_permute with a workspace instead",
                fn, T, k, E, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  CHECK(scratch_address(fn, &ws));
  // Every scratch word the kernels read is written earlier in the same call (the
  // histograms by hist_kernel, the bases by scan_kernel): nothing needs clearing.
  const size_t half = need / 2;
  moe::PermuteArgs a{topk_idx, T, k, E, capacity < 0 ? -1 : capacity, x, d * elem_bytes(dtype), counts,
                     offsets, row_of, perm_token, x_perm, static_cast<int32_t*>(ws),
                     reinterpret_cast<int32_t*>(static_cast<char*>(ws) + half), 0};
  return hip_status(moe::launch_permute(a, stream), fn);
}

int moe_permute_padded(const int32_t* topk_idx, int T, int k, int E, int64_t capacity, const void* x, int dtype,
                       int d, int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* slot_token,
                       void* x_slots, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "moe_permute_padded";
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  CHECK(experts_check(fn, E, k));
  if (capacity < 1) return fail(MOE_ERR_INVALID_ARG, "%s: capacity = %lld must be at least 1", fn,
                                (long long)capacity);
  if ((int64_t)E * capacity > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E*capacity = %lld exceeds 2^31-1", fn, (long long)((int64_t)E * capacity));
  if (d <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: d = %d must be positive", fn, d);
  if (d % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: d = %d must be a multiple of 8", fn, d);
  CHECK(assignments_check(fn, T, k));
  if (T == 0) return ok();
  NEED(topk_idx, fn);
  NEED(counts, fn);
  NEED(offsets, fn);
  NEED(row_of, fn);
  NEED(slot_token, fn);
  if (x_slots != nullptr) NEED(x, fn);
  const size_t need = moe_permute_workspace_bytes(T, k, E);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  const size_t half = need / 2;
  moe::PermuteArgs a{topk_idx, T, k, E, capacity, x, d * elem_bytes(dtype), counts, offsets, row_of, slot_token,
                     x_slots, static_cast<int32_t*>(workspace),
                     reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + half), 1};
  return hip_status(moe::launch_permute(a, stream), fn);
}

static int grouped_check(const char* fn, int G, int max_rows, int d, int F, int dtype) {
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (G < 1 || G > MOE_MAX_EXPERTS)
    return fail(G < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED, "%s: G = %d outside [1, %d]", fn, G,
                MOE_MAX_EXPERTS);
  if (max_rows < 0) return fail(MOE_ERR_INVALID_ARG, "%s: max_rows = %d < 0", fn, max_rows);
  CHECK(width_check(fn, "d", d, dtype));
  CHECK(width_check(fn, "F", F, dtype));
  // the bf16 kernel addresses each operand (rows x width, one expert's weights)
  // with 32-bit byte offsets
  const int64_t eb = elem_bytes(dtype), lim = (int64_t)UINT32_MAX;
  if ((int64_t)max_rows * d * eb > lim || (int64_t)max_rows * F * eb > lim || (int64_t)d * F * eb > lim)
    return fail(MOE_ERR_UNSUPPORTED, "%s: an operand exceeds 4 GiB (max_rows=%d d=%d F=%d)", fn, max_rows, d, F);
  return MOE_OK;
}

int moe_grouped_gate_up(const void* x, const int32_t* row_index, int src_rows, const int32_t* offsets, int G,
                        int max_rows, int d, int F, const void* w_gate, const void* w_up, int dtype, void* a,
                        hipStream_t stream) {
  static const char* fn = "moe_grouped_gate_up";
  CHECK(grouped_check(fn, G, max_rows, d, F, dtype));
  if (row_index != nullptr && src_rows < 1)
    return fail(MOE_ERR_INVALID_ARG, "%s: src_rows = %d must be positive with a row index", fn, src_rows);
  if (row_index != nullptr && (int64_t)src_rows * d * elem_bytes(dtype) > (int64_t)UINT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: x exceeds 4 GiB (src_rows=%d d=%d)", fn, src_rows, d);
  if (max_rows == 0) return ok();
  NEED(x, fn);
  NEED(offsets, fn);
  NEED(w_gate, fn);
  NEED(w_up, fn);
  NEED(a, fn);
  if (g_check_only) return ok();
  moe::GroupedGemmArgs g{x, row_index, row_index ? src_rows : max_rows, offsets, G, max_rows, F, d,
                         w_gate, w_up, a, dtype};
  return hip_status(moe::launch_grouped_gemm(g, true, stream), fn);
}

int moe_grouped_down(const void* a, const int32_t* offsets, int G, int max_rows, int F, int d,
                     const void* w_down, int dtype, void* y_perm, hipStream_t stream) {
  static const char* fn = "moe_grouped_down";
  CHECK(grouped_check(fn, G, max_rows, d, F, dtype));
  if (max_rows == 0) return ok();
  NEED(a, fn);
  NEED(offsets, fn);
  NEED(w_down, fn);
  NEED(y_perm, fn);
  if (g_check_only) return ok();
  moe::GroupedGemmArgs g{a, nullptr, max_rows, offsets, G, max_rows, d, F, w_down, nullptr, y_perm, dtype};
  return hip_status(moe::launch_grouped_gemm(g, false, stream), fn);
}

int moe_grouped_swiglu(const void* x, const int32_t* row_index, int src_rows, const int32_t* offsets, int G,
                       int max_rows, int d, int F, const void* w_gate, const void* w_up, const void* w_down,
                       int dtype, void* a, void* y_perm, hipStream_t stream) {
  static const char* fn = "moe_grouped_swiglu";
  CHECK(grouped_check(fn, G, max_rows, d, F, dtype));
  if (max_rows == 0) return ok();
  NEED(w_down, fn);
  NEED(y_perm, fn);
  CHECK(moe_grouped_gate_up(x, row_index, src_rows, offsets, G, max_rows, d, F, w_gate, w_up, dtype, a,
                            stream));
  return moe_grouped_down(a, offsets, G, max_rows, F, d, w_down, dtype, y_perm, stream);
}

int moe_combine(const void* y_perm, int y_rows, const int32_t* row_of, const float* topk_w, const void* shared_y,
                int dtype, int T, int k, int d, void* y, hipStream_t stream) {
  static const char* fn = "moe_combine";
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  if (y_rows < 0) return fail(MOE_ERR_INVALID_ARG, "%s: y_rows = %d < 0", fn, y_rows);
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "%s: k = %d < 1", fn, k);
  if (d <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: d = %d must be positive", fn, d);
  if (d % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: d = %d must be a multiple of 8", fn, d);
  CHECK(assignments_check(fn, T, k));
  if (T == 0) return ok();
  if (y_rows > 0) NEED(y_perm, fn);
  NEED(row_of, fn);
  NEED(topk_w, fn);
  NEED(y, fn);
  if (g_check_only) return ok();
  moe::CombineArgs c{y_perm, row_of, topk_w, shared_y, dtype, T, k, d, y_rows, y};
  return hip_status(moe::launch_combine(c, stream), fn);
}

static size_t round256(size_t n) { return (n + 255) / 256 * 256; }

size_t moe_down_combine_workspace_bytes(int T, int d, int max_rows) {
  if (T < 0 || d < 0 || max_rows < 0) return 0;
  return round256((size_t)T * (size_t)d * 4u) + round256((size_t)max_rows * 4u);
}

int moe_grouped_down_combine(const void* a, const int32_t* offsets, int G, int max_rows, int F, int d,
                             const void* w_down, int dtype, const int32_t* perm_token, const int32_t* row_of,
                             const float* topk_w, int T, int k, const void* shared_y, void* y, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "moe_grouped_down_combine";
  CHECK(grouped_check(fn, G, max_rows, d, F, dtype));
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "%s: k = %d < 1", fn, k);
  CHECK(assignments_check(fn, T, k));
  if (T == 0) return ok();
  NEED(row_of, fn);
  NEED(topk_w, fn);
  NEED(y, fn);
  if (max_rows > 0) {
    NEED(a, fn);
    NEED(offsets, fn);
    NEED(w_down, fn);
    NEED(perm_token, fn);
  }
  const size_t need = moe_down_combine_workspace_bytes(T, d, max_rows);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  float* y_acc = static_cast<float*>(workspace);
  float* row_w = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)T * (size_t)d * 4u));
  hipError_t e = moe::launch_scatter_prologue(y_acc, row_w, row_of, topk_w, T, k, d, max_rows, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  if (max_rows > 0) {
    moe::GroupedGemmArgs g{a, nullptr, max_rows, offsets, G, max_rows, d, F, w_down, nullptr, nullptr, dtype};
    g.out_tok = perm_token;
    g.out_w = row_w;
    g.y_acc = y_acc;
    g.T = T;
    e = moe::launch_grouped_gemm(g, false, stream);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return hip_status(moe::launch_scatter_finish(y_acc, shared_y, dtype, T, d, y, stream), fn);
}

size_t moe_layer_args_size(void) { return sizeof(moe_layer_args); }

}  // extern "C"

namespace {

// The layer's calls in order on `stream` (route and permute, or their fused
// decode form, then the GEMMs, the shared expert, the combine and the
// statistics).  `check` runs every call's checks and enqueues nothing.
int layer_calls(const moe_layer_args& L, hipStream_t stream, bool check) {
  const int64_t R = (int64_t)L.T * L.k;
  const bool fused = moe::route_dispatch_small_fits(L.dtype, L.T, L.k, L.E);
  auto mark = [&](int i) -> int {
    if (check || L.marks[i] == nullptr) return MOE_OK;
    return hip_status(hipEventRecord(L.marks[i], stream), "moe_layer_forward");
  };
  // The router's blocks can write the dispatch's per-block histograms (into the
  // permute workspace), which then skips its histogram launch.
  const bool hist = moe::route_writes_block_hist(L.dtype, L.T, L.E, L.k);
  if (check || (!fused && !hist)) {
    CHECK(moe_route(L.x, L.w_router, L.logit_bias, L.select_bias, L.dtype, L.T, L.d, L.E, L.k, L.mode, L.renorm,
                    L.logits, L.topk_idx, L.topk_w, L.near_tie, stream));
    CHECK(moe_permute(L.topk_idx, L.T, L.k, L.E, L.capacity, L.x, L.dtype, L.d, L.counts, L.offsets, L.row_of,
                      L.perm_token, nullptr, L.permute_workspace, L.permute_workspace_bytes, stream));
  }
  if (!check && !fused && hist) {
    // the two calls above, their checks passed, with the histogram handed over
    int32_t* block_counts = static_cast<int32_t*>(L.permute_workspace);
    int32_t* block_base = reinterpret_cast<int32_t*>(static_cast<char*>(L.permute_workspace) +
                                                     moe_permute_workspace_bytes(L.T, L.k, L.E) / 2);
    float* stats_partial = static_cast<float*>(L.stats_workspace);
    moe::RouteArgs r{L.x, L.w_router, L.logit_bias, L.select_bias, L.dtype, L.T, L.d, L.E, L.k, L.mode,
                     L.renorm ? 1 : 0, L.logits, L.topk_idx, L.topk_w, L.near_tie, block_counts, stats_partial};
    CHECK(hip_status(moe::launch_route(r, stream), "moe_layer_forward"));
    // The router wrote the statistics' partial sums: their final reduction needs
    // only the counts.  It runs as one more block of the dispatch's rank launch,
    // or right after the dispatch; no side stream is used.
    moe::StatsArgs sa{L.counts, L.logits, L.T, L.k, L.E, L.alpha, L.f, L.P, L.l_aux, L.max_over_mean, stats_partial};
    const bool fuse = moe::permute_fuses_stats(L.T, L.k);
    moe::PermuteArgs pa{L.topk_idx, L.T, L.k, L.E, L.capacity < 0 ? -1 : L.capacity, L.x, L.d * elem_bytes(L.dtype),
                        L.counts, L.offsets, L.row_of, L.perm_token, nullptr, block_counts, block_base, 0, 1,
                        fuse ? &sa : nullptr};
    CHECK(hip_status(moe::launch_permute(pa, stream), "moe_layer_forward"));
    if (!fuse) CHECK(hip_status(moe::launch_stats_final(sa, stream), "moe_layer_forward"));
  }
  if (!check && fused) {
    moe::RouteDispatchArgs a{{L.x, L.w_router, L.logit_bias, L.select_bias, L.dtype, L.T, L.d, L.E, L.k, L.mode,
                              L.renorm ? 1 : 0, L.logits, L.topk_idx, L.topk_w, L.near_tie},
                             L.capacity < 0 ? -1 : L.capacity, L.counts, L.offsets, L.row_of, L.perm_token,
                             L.alpha, L.f, L.P, L.l_aux, L.max_over_mean};
    CHECK(hip_status(moe::launch_route_dispatch_small(a, stream), "moe_layer_forward"));
  }
  CHECK(mark(0));
  CHECK(moe_grouped_gate_up(L.x, L.perm_token, L.T, L.offsets, L.E, (int)R, L.d, L.F, L.w_gate, L.w_up, L.dtype,
                            L.a, stream));
  CHECK(mark(1));
  CHECK(moe_grouped_down(L.a, L.offsets, L.E, (int)R, L.F, L.d, L.w_down, L.dtype, L.y_perm, stream));
  CHECK(mark(2));
  if (L.F_shared > 0)
    CHECK(moe_grouped_swiglu(L.x, nullptr, 0, L.shared_offsets, 1, L.T, L.d, L.F_shared, L.shared_gate,
                             L.shared_up, L.shared_down, L.dtype, L.shared_a, L.shared_y, stream));
  CHECK(mark(3));
  const bool side = !fused && !hist && L.side_stream != nullptr && L.fork_event != nullptr &&
                    L.join_event != nullptr;
  auto stats = [&](hipStream_t st) {
    return moe_stats(L.counts, L.logits, L.T, L.k, L.E, L.alpha, L.f, L.P, L.l_aux, L.max_over_mean,
                     L.stats_workspace, L.stats_workspace_bytes, st);
  };
  if (side && !check) {
    CHECK(hip_status(hipEventRecord(L.fork_event, stream), "moe_layer_forward"));
    CHECK(hip_status(hipStreamWaitEvent(L.side_stream, L.fork_event, 0), "moe_layer_forward"));
    CHECK(stats(L.side_stream));
    CHECK(hip_status(hipEventRecord(L.join_event, L.side_stream), "moe_layer_forward"));
  }
  CHECK(moe_combine(L.y_perm, (int)R, L.row_of, L.topk_w, L.F_shared > 0 ? L.shared_y : nullptr, L.dtype, L.T, L.k,
                    L.d, L.y, stream));
  if (side && !check) return hip_status(hipStreamWaitEvent(stream, L.join_event, 0), "moe_layer_forward");
  if (check || (!fused && !hist)) CHECK(stats(stream));
  return ok();
}

}  // namespace

extern "C" {

int moe_layer_forward(const moe_layer_args* args, hipStream_t stream) {
  static const char* fn = "moe_layer_forward";
  if (args == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: args must not be NULL", fn);
  const moe_layer_args& L = *args;
  if (L.T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, L.T);
  if (L.F_shared < 0) return fail(MOE_ERR_INVALID_ARG, "%s: F_shared = %d < 0", fn, L.F_shared);
  if (L.T == 0) return ok();
  if (L.F_shared > 0) NEED(L.shared_offsets, fn);
  if ((int64_t)L.T * L.k > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: T*k = %lld exceeds 2^31-1", fn, (long long)L.T * L.k);
  g_check_only = true;
  const int checked = layer_calls(L, stream, true);
  g_check_only = false;
  if (checked != MOE_OK) return checked;
  return layer_calls(L, stream, false);
}

int moe_stats(const int32_t* counts, const float* logits, int T, int k, int E, float alpha, float* f, float* P,
              float* l_aux, float* max_over_mean, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  static const char* fn = "moe_stats";
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  CHECK(experts_check(fn, E, k));
  CHECK(assignments_check(fn, T, k));
  if (!isfinite(alpha)) return fail(MOE_ERR_INVALID_ARG, "%s: alpha is not finite", fn);
  if (T == 0) return ok();
  NEED(counts, fn);
  NEED(logits, fn);
  NEED(f, fn);
  NEED(P, fn);
  NEED(l_aux, fn);
  NEED(max_over_mean, fn);
  const size_t need = moe_stats_workspace_bytes(T, E);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if (g_check_only) return ok();
  moe::StatsArgs s{counts, logits, T, k, E, alpha, f, P, l_aux, max_over_mean, static_cast<float*>(workspace)};
  return hip_status(moe::launch_stats(s, stream), fn);
}

}  // extern "C"
