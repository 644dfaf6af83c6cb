// Host side of the C ABI declared in include/moe.h: argument checks (pure
// host code, before anything is enqueued), workspace carving and kernel
// dispatch.  No allocation happens on any call path after moe_create.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <new>
#include <vector>

#include "../../include/moe.h"
#include "internal.h"

namespace moe {

const char* const kKernelNames[K_COUNT] = {
    "router_logits", "router_topk",     "permute",         "fill",
    "encode_rows",   "ffn_i8_gate_up",  "ffn_i8_down",     "ffn_i4_gate_up",
    "ffn_i4_down",   "ffn_f32_gate_up", "ffn_f32_down",    "combine",
    "router_tail",   "ffn_i8_gate_up_gemm", "ffn_i8_down_gemm", "quant_i8_rows",
    "quant_i4_blocks"};

// Event pairs recorded around launches while a context has timing on.
struct KernelTimer {
  struct Mark {
    int id;
    hipEvent_t a, b;
  };
  std::vector<hipEvent_t> pool;  // created when timing is switched on
  std::vector<Mark> marks;
  size_t next = 0;
  long long dropped = 0;
  int open_id = -1;
  hipEvent_t open_a = nullptr;
};

thread_local KernelTimer* g_timer = nullptr;

void timer_begin(int id, hipStream_t s) {
  KernelTimer* t = g_timer;
  if (t->next + 2 > t->pool.size()) {
    t->open_id = -1;
    ++t->dropped;
    return;
  }
  t->open_a = t->pool[t->next++];
  t->open_id = id;
  (void)hipEventRecord(t->open_a, s);
}

void timer_end(hipStream_t s) {
  KernelTimer* t = g_timer;
  if (t->open_id < 0) return;
  hipEvent_t b = t->pool[t->next++];
  (void)hipEventRecord(b, s);
  t->marks.push_back({t->open_id, t->open_a, b});
  t->open_id = -1;
}
}  // namespace moe

struct moe_ctx {
  int device;
  int cu_count;
  int max_lds;
  char arch[64];
  char err[512];
  bool timing;
  moe::KernelTimer timer;
};

namespace {

thread_local char g_create_err[512] = "";

moe_status fail(moe_ctx* ctx, moe_status st, const char* fmt, ...) {
  char* buf = ctx ? ctx->err : g_create_err;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, 512, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// Run f with ctx->device current, restoring the caller's device afterwards.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

moe_status device_result(moe_ctx* ctx, hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(ctx, MOE_E_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

moe_status check_ctx(moe_ctx* ctx) {
  if (!ctx) return MOE_E_INVALID;
  ctx->err[0] = '\0';
  moe::g_timer = ctx->timing ? &ctx->timer : nullptr;
  return MOE_OK;
}

void release_timer(moe::KernelTimer& t) {
  for (hipEvent_t e : t.pool) (void)hipEventDestroy(e);
  t.pool.clear();
  t.marks.clear();
  t.next = 0;
  t.dropped = 0;
}

// moe_forward workspace: router partials | idx | w | offsets | row_token |
// token_row | rows [R][d] | shared rows [T][d] | FFN workspace.
struct FwdWs {
  float* partial;
  int32_t* idx;
  float* w;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* token_row;
  float* rows;
  float* sh_rows;
  void* ffn;
  size_t ffn_bytes;
  size_t bytes;
};

size_t ffn_need(int T, int R, int d, int inter, int fmt);

FwdWs fwd_layout(void* base, const moe_layer* L, int T) {
  FwdWs f{};
  const int E = L->experts.n_experts, d = L->experts.d, k = L->k;
  const int R = T * k;
  const bool has_sh = L->shared.n_experts > 0;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t n) {
    char* p = b ? b + off : nullptr;
    off = moe::align_up(off + n, 256);
    return p;
  };
  f.partial = reinterpret_cast<float*>(take(moe::route_ws_bytes(T, d, E)));
  f.idx = reinterpret_cast<int32_t*>(take((size_t)R * 4));
  f.w = reinterpret_cast<float*>(take((size_t)R * 4));
  f.offsets = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
  f.row_token = reinterpret_cast<int32_t*>(take((size_t)R * 4));
  f.token_row = reinterpret_cast<int32_t*>(take((size_t)R * 4));
  f.rows = reinterpret_cast<float*>(take((size_t)R * d * 4));
  f.sh_rows = has_sh ? reinterpret_cast<float*>(take((size_t)T * d * 4)) : nullptr;
  const bool fused = has_sh && L->shared.fmt == L->experts.fmt &&
                     L->shared.layout == L->experts.layout && L->experts.fmt != MOE_W_FP32;
  size_t ffn;
  if (fused) {
    int Rs[2] = {R, T}, Is[2] = {L->experts.inter, L->shared.inter};
    ffn = moe::ffn_ws_layout(nullptr, T, d, 2, Rs, Is, true).bytes;
  } else {
    ffn = ffn_need(T, R, d, L->experts.inter, L->experts.fmt);
    if (has_sh) {
      size_t s2 = ffn_need(T, T, d, L->shared.inter, L->shared.fmt);
      ffn = ffn > s2 ? ffn : s2;
    }
  }
  f.ffn_bytes = ffn;
  f.ffn = take(ffn);
  f.bytes = off;
  return f;
}

size_t ffn_need(int T, int R, int d, int inter, int fmt) {
  return moe::ffn_ws_layout(nullptr, T, d, 1, &R, &inter, fmt != MOE_W_FP32).bytes;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_INVALID: return "MOE_E_INVALID";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED";
    case MOE_E_DEVICE: return "MOE_E_DEVICE";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE";
  }
  return "unknown moe_status";
}

moe_status moe_create(int device, moe_ctx** out) {
  if (!out) return fail(nullptr, MOE_E_INVALID, "moe_create: out is NULL");
  *out = nullptr;
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n == 0)
    return fail(nullptr, MOE_E_DEVICE, "moe_create: no HIP device (%s)",
                e != hipSuccess ? hipGetErrorString(e) : "device count is 0");
  if (device < 0 || device >= n)
    return fail(nullptr, MOE_E_INVALID, "moe_create: device %d out of range [0, %d)", device, n);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess)
    return fail(nullptr, MOE_E_DEVICE, "moe_create: hipGetDeviceProperties: %s",
                hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, MOE_E_UNSUPPORTED,
                "moe_create: device %d is %s; this library is built for gfx950 (MI355X)", device,
                prop.gcnArchName);
  moe_ctx* ctx = new (std::nothrow) moe_ctx;
  if (!ctx) return fail(nullptr, MOE_E_DEVICE, "moe_create: out of host memory");
  ctx->device = device;
  ctx->cu_count = prop.multiProcessorCount;
  ctx->max_lds = (int)prop.sharedMemPerBlock;
  snprintf(ctx->arch, sizeof(ctx->arch), "%s", prop.gcnArchName);
  ctx->err[0] = '\0';
  ctx->timing = false;

  moe::set_device_info(ctx->cu_count);
  *out = ctx;
  return MOE_OK;
}

void moe_destroy(moe_ctx* ctx) {
  if (!ctx) return;
  if (moe::g_timer == &ctx->timer) moe::g_timer = nullptr;
  release_timer(ctx->timer);
  delete ctx;
}

moe_status moe_timing(moe_ctx* ctx, int capacity) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (capacity < 0) return fail(ctx, MOE_E_INVALID, "moe_timing: capacity=%d", capacity);
  DeviceGuard g(ctx->device);
  release_timer(ctx->timer);
  ctx->timing = false;
  moe::g_timer = nullptr;
  if (capacity == 0) return MOE_OK;
  ctx->timer.pool.reserve(2 * (size_t)capacity);
  ctx->timer.marks.reserve((size_t)capacity);
  for (int i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      release_timer(ctx->timer);
      return device_result(ctx, err, "moe_timing: hipEventCreate");
    }
    ctx->timer.pool.push_back(e);
  }
  ctx->timing = true;
  return MOE_OK;
}

moe_status moe_timing_read(moe_ctx* ctx, moe_kernel_time* out, int max_out, int* n_out) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (!n_out || (max_out > 0 && !out))
    return fail(ctx, MOE_E_INVALID, "moe_timing_read: out or n_out is NULL");
  DeviceGuard g(ctx->device);
  double total[moe::K_COUNT] = {0};
  long long count[moe::K_COUNT] = {0};
  for (const auto& m : ctx->timer.marks) {
    hipError_t err = hipEventSynchronize(m.b);
    if (err != hipSuccess) return device_result(ctx, err, "moe_timing_read: hipEventSynchronize");
    float ms = 0.0f;
    err = hipEventElapsedTime(&ms, m.a, m.b);
    if (err != hipSuccess) return device_result(ctx, err, "moe_timing_read: hipEventElapsedTime");
    total[m.id] += ms;
    count[m.id] += 1;
  }
  int n = 0;
  for (int i = 0; i < moe::K_COUNT; ++i) {
    if (count[i] == 0) continue;
    if (n < max_out) {
      out[n].name = moe::kKernelNames[i];
      out[n].launches = count[i];
      out[n].total_ms = total[i];
    }
    ++n;
  }
  *n_out = n;
  ctx->timer.marks.clear();
  ctx->timer.next = 0;
  if (ctx->timer.dropped)
    fail(ctx, MOE_OK, "moe_timing_read: %lld launches were not timed (capacity)",
         ctx->timer.dropped);
  ctx->timer.dropped = 0;
  return MOE_OK;
}

const char* moe_last_error(const moe_ctx* ctx) { return ctx ? ctx->err : g_create_err; }

moe_status moe_workspace_size(const moe_ctx* cctx, int T, int k, int E, int d, int inter, int fmt,
                              size_t* bytes) {
  moe_ctx* ctx = const_cast<moe_ctx*>(cctx);
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (!bytes) return fail(ctx, MOE_E_INVALID, "moe_workspace_size: bytes is NULL");
  if (T < 0 || k < 1 || E < 1 || d < 1 || inter < 1)
    return fail(ctx, MOE_E_INVALID,
                "moe_workspace_size: need T >= 0, k >= 1, E >= 1, d >= 1, inter >= 1 "
                "(got T=%d k=%d E=%d d=%d inter=%d)", T, k, E, d, inter);
  if (fmt < MOE_W_FP32 || fmt > MOE_W_INT4_B128)
    return fail(ctx, MOE_E_INVALID, "moe_workspace_size: unknown weight format %d", fmt);
  const long long R = (long long)T * k;
  if (R > 0x7fffffffLL) return fail(ctx, MOE_E_INVALID, "moe_workspace_size: T*k overflows");
  size_t a = moe::route_ws_bytes(T, d, E);
  size_t b = ffn_need(T, (int)R, d, inter, fmt);
  *bytes = a > b ? a : b;
  return MOE_OK;
}

moe_status moe_route(moe_ctx* ctx, int router, const float* x, const float* w_router,
                     const float* bias, int T, int d, int E, int k, float scale,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream) {
  return moe_route_masked(ctx, router, x, w_router, bias, nullptr, T, d, E, k, scale, topk_idx,
                          topk_w, ws, ws_bytes, stream);
}

moe_status moe_route_masked(moe_ctx* ctx, int router, const float* x, const float* w_router,
                            const float* bias, const uint8_t* mask, int T, int d, int E,
                            int k, float scale, int32_t* topk_idx, float* topk_w, void* ws,
                            size_t ws_bytes, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (router != MOE_ROUTER_SIGMOID_BIAS && router != MOE_ROUTER_SOFTMAX)
    return fail(ctx, MOE_E_INVALID, "moe_route: unknown router %d", router);
  if (T < 0) return fail(ctx, MOE_E_INVALID, "moe_route: T=%d is negative", T);
  if (E < 1 || E > moe::kMaxE)
    return fail(ctx, MOE_E_INVALID, "moe_route: E=%d outside [1, %d]", E, moe::kMaxE);
  if (k < 1 || k > E || k > moe::kMaxK)
    return fail(ctx, MOE_E_INVALID, "moe_route: k=%d outside [1, min(E=%d, %d)]", k, E,
                moe::kMaxK);
  if (d < 1) return fail(ctx, MOE_E_INVALID, "moe_route: d=%d", d);
  if (d % 64 != 0)
    return fail(ctx, MOE_E_UNSUPPORTED, "moe_route: d=%d is not a multiple of 64", d);
  if (!std::isfinite(scale)) return fail(ctx, MOE_E_INVALID, "moe_route: scale is not finite");
  if (router == MOE_ROUTER_SOFTMAX && bias)
    return fail(ctx, MOE_E_INVALID, "moe_route: the softmax router takes no bias");
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w)
    return fail(ctx, MOE_E_INVALID, "moe_route: %s is NULL",
                !x ? "x" : !w_router ? "w_router" : !topk_idx ? "topk_idx" : "topk_w");
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(bias) || !aligned16(topk_idx) ||
      !aligned16(topk_w))
    return fail(ctx, MOE_E_INVALID, "moe_route: a pointer is not 16-byte aligned");
  const size_t need = moe::route_ws_bytes(T, d, E);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(ctx, MOE_E_WORKSPACE, "moe_route: workspace %s (need %zu bytes, got %zu)",
                !ws ? "is NULL" : !aligned16(ws) ? "is not 16-byte aligned" : "too small",
                need, ws_bytes);
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "moe_route: hipSetDevice(%d) failed", ctx->device);
  hipError_t e = moe::launch_router(router, x, w_router, bias, mask, T, d, E, k, scale,
                                    topk_idx, topk_w, static_cast<float*>(ws),
                                    (hipStream_t)stream);
  return device_result(ctx, e, "moe_route");
}

moe_status moe_expert_counts(moe_ctx* ctx, const int32_t* topk_idx, int T, int k, int E,
                             unsigned long long* counts, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (T < 0 || k < 1 || (long long)T * k > 0x7fffffffLL)
    return fail(ctx, MOE_E_INVALID, "moe_expert_counts: T=%d k=%d", T, k);
  if (E < 1 || E > moe::kMaxE)
    return fail(ctx, MOE_E_INVALID, "moe_expert_counts: E=%d outside [1, %d]", E, moe::kMaxE);
  if (T == 0) return MOE_OK;
  if (!topk_idx || !counts)
    return fail(ctx, MOE_E_INVALID, "moe_expert_counts: %s is NULL",
                !topk_idx ? "topk_idx" : "counts");
  if (!aligned16(topk_idx) || (reinterpret_cast<uintptr_t>(counts) & 7) != 0)
    return fail(ctx, MOE_E_INVALID, "moe_expert_counts: a pointer is misaligned");
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_expert_counts: hipSetDevice(%d) failed", ctx->device);
  hipError_t e = moe::launch_expert_counts(topk_idx, (long long)T * k, E, counts,
                                           (hipStream_t)stream);
  return device_result(ctx, e, "moe_expert_counts");
}

moe_status moe_quantize(moe_ctx* ctx, int fmt, int in_type, const void* w, long long rows,
                        int K, void* codes, float* scales, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (fmt != MOE_W_INT8_ROW && fmt != MOE_W_INT4_B32 && fmt != MOE_W_INT4_B128)
    return fail(ctx, MOE_E_UNSUPPORTED, "moe_quantize: format %d has no quantizer", fmt);
  if (in_type != MOE_IN_F32 && in_type != MOE_IN_BF16)
    return fail(ctx, MOE_E_INVALID, "moe_quantize: unknown input type %d", in_type);
  if (rows < 0) return fail(ctx, MOE_E_INVALID, "moe_quantize: rows=%lld is negative", rows);
  const int kmul = fmt == MOE_W_INT8_ROW ? 8 : (fmt == MOE_W_INT4_B32 ? 32 : 128);
  if (K < kmul || K % kmul != 0 || K > (1 << 24))
    return fail(ctx, MOE_E_UNSUPPORTED,
                "moe_quantize: K=%d must be a positive multiple of %d, at most 2^24", K, kmul);
  if (rows > (1LL << 32) || rows > (1LL << 40) / K)
    return fail(ctx, MOE_E_UNSUPPORTED, "moe_quantize: rows above 2^32 or rows*K above 2^40");
  if (rows == 0) return MOE_OK;
  if (!w || !codes || !scales)
    return fail(ctx, MOE_E_INVALID, "moe_quantize: %s is NULL",
                !w ? "w" : !codes ? "codes" : "scales");
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales))
    return fail(ctx, MOE_E_INVALID, "moe_quantize: a pointer is not 16-byte aligned");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "moe_quantize: hipSetDevice(%d) failed", ctx->device);
  hipError_t e = moe::launch_quantize(fmt, in_type, w, rows, K, codes, scales,
                                      (hipStream_t)stream);
  return device_result(ctx, e, "moe_quantize");
}

moe_status moe_permute(moe_ctx* ctx, const int32_t* topk_idx, int T, int k, int E,
                       int32_t* offsets, int32_t* row_token, int32_t* token_row, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (T < 0) return fail(ctx, MOE_E_INVALID, "moe_permute: T=%d is negative", T);
  if (E < 1 || E > moe::kMaxE)
    return fail(ctx, MOE_E_INVALID, "moe_permute: E=%d outside [1, %d]", E, moe::kMaxE);
  if (k < 1 || k > moe::kMaxK)
    return fail(ctx, MOE_E_INVALID, "moe_permute: k=%d outside [1, %d]", k, moe::kMaxK);
  if ((long long)T * k > 0x7fffffffLL)
    return fail(ctx, MOE_E_INVALID, "moe_permute: T*k overflows");
  if (!offsets) return fail(ctx, MOE_E_INVALID, "moe_permute: offsets is NULL");
  if (T > 0 && (!topk_idx || !row_token || !token_row))
    return fail(ctx, MOE_E_INVALID, "moe_permute: %s is NULL",
                !topk_idx ? "topk_idx" : !row_token ? "row_token" : "token_row");
  if (!aligned16(topk_idx) || !aligned16(offsets) || !aligned16(row_token) ||
      !aligned16(token_row))
    return fail(ctx, MOE_E_INVALID, "moe_permute: a pointer is not 16-byte aligned");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "moe_permute: hipSetDevice(%d) failed", ctx->device);
  if (T == 0) {  // every expert is empty: offsets = 0 (a fill kernel, not a memset node)
    hipError_t e = moe::launch_fill_i32(offsets, E + 1, 0, (hipStream_t)stream);
    return device_result(ctx, e, "moe_permute");
  }
  hipError_t e = moe::launch_permute(topk_idx, T, k, E, offsets, row_token, token_row,
                                     (hipStream_t)stream);
  return device_result(ctx, e, "moe_permute");
}

namespace {
moe_status check_weights(moe_ctx* ctx, const char* fn, const char* which, const moe_weights* w) {
  if (w->fmt < MOE_W_FP32 || w->fmt > MOE_W_INT4_B128)
    return fail(ctx, MOE_E_INVALID, "%s: %s: unknown weight format %d", fn, which, w->fmt);
  if (w->n_experts < 1 || w->d < 1 || w->inter < 1)
    return fail(ctx, MOE_E_INVALID, "%s: %s: n_experts=%d d=%d inter=%d", fn, which,
                w->n_experts, w->d, w->inter);
  if (w->d > moe::kMaxWidth || w->inter > moe::kMaxWidth)
    return fail(ctx, MOE_E_UNSUPPORTED, "%s: %s: d=%d and inter=%d must be at most %d", fn,
                which, w->d, w->inter, moe::kMaxWidth);
  const int mult = w->fmt == MOE_W_INT4_B32 || w->fmt == MOE_W_INT4_B128 ? 128 : 64;
  if (w->d % mult != 0 || w->inter % mult != 0)
    return fail(ctx, MOE_E_UNSUPPORTED, "%s: %s: d=%d and inter=%d must be multiples of %d", fn,
                which, w->d, w->inter, mult);
  if (w->layout != MOE_LAYOUT_ROWS && w->layout != MOE_LAYOUT_TILED)
    return fail(ctx, MOE_E_INVALID, "%s: %s: unknown layout %d", fn, which, w->layout);
  if (w->layout == MOE_LAYOUT_TILED && w->fmt == MOE_W_FP32)
    return fail(ctx, MOE_E_UNSUPPORTED, "%s: %s: fp32 weights have no tiled layout", fn, which);
  if (!w->w_gate_up || !w->w_down)
    return fail(ctx, MOE_E_INVALID, "%s: %s: weights are NULL", fn, which);
  if (w->fmt != MOE_W_FP32 && (!w->s_gate_up || !w->s_down))
    return fail(ctx, MOE_E_INVALID, "%s: %s: scales are NULL for a quantised format", fn, which);
  if (!aligned16(w->w_gate_up) || !aligned16(w->w_down) || !aligned16(w->s_gate_up) ||
      !aligned16(w->s_down))
    return fail(ctx, MOE_E_INVALID, "%s: %s: a pointer is not 16-byte aligned", fn, which);
  return MOE_OK;
}

}  // namespace

moe_status moe_expert_ffn(moe_ctx* ctx, const moe_weights* w, int act, const float* x, int T,
                          const int32_t* row_token, const int32_t* offsets, int R_max,
                          float* rows_out, void* ws, size_t ws_bytes, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (!w) return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: weights is NULL");
  if (act != MOE_ACT_SILU && act != MOE_ACT_GELU_TANH)
    return fail(ctx, MOE_E_UNSUPPORTED,
                "moe_expert_ffn: unsupported activation=%d (MOE_ACT_SILU=0 or "
                "MOE_ACT_GELU_TANH=1)", act);
  {
    moe_status st = check_weights(ctx, "moe_expert_ffn", "weights", w);
    if (st != MOE_OK) return st;
  }
  if (T < 0 || R_max < 0)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: T=%d R_max=%d", T, R_max);
  if (!offsets && w->n_experts != 1)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: offsets may be NULL only for one expert");
  if (!offsets && !row_token && R_max > T)
    return fail(ctx, MOE_E_INVALID,
                "moe_expert_ffn: with identity rows R_max=%d may not exceed T=%d", R_max, T);
  if (T == 0 || R_max == 0) return MOE_OK;
  if (!x || !rows_out)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: %s is NULL", !x ? "x" : "rows_out");
  if (!aligned16(x) || !aligned16(row_token) || !aligned16(offsets) || !aligned16(rows_out))
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: a pointer is not 16-byte aligned");
  const size_t need = ffn_need(T, R_max, w->d, w->inter, w->fmt);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(ctx, MOE_E_WORKSPACE, "moe_expert_ffn: workspace %s (need %zu bytes, got %zu)",
                !ws ? "is NULL" : !aligned16(ws) ? "is not 16-byte aligned" : "too small", need,
                ws_bytes);
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_expert_ffn: hipSetDevice(%d) failed", ctx->device);
  hipError_t e;
  int inter = w->inter;
  if (w->fmt == MOE_W_FP32) {
    moe::FfnWs lay = moe::ffn_ws_layout(ws, T, w->d, 1, &R_max, &inter, false);
    e = moe::launch_ffn_f32(static_cast<const float*>(w->w_gate_up),
                            static_cast<const float*>(w->w_down), w->n_experts, w->d, w->inter,
                            x, T, row_token, offsets, R_max, rows_out, lay.h, act,
                            (hipStream_t)stream);
  } else {
    moe::FfnWs lay = moe::ffn_ws_layout(ws, T, w->d, 1, &R_max, &inter, true);
    moe::FfnSet set{w->fmt, w->layout, w->n_experts, w->inter, R_max, w->w_gate_up, w->s_gate_up,
                    w->w_down, w->s_down, row_token, offsets, lay.hq[0], lay.hs[0], rows_out,
                    nullptr, 1, act};
    e = moe::launch_ffn_quant(&set, 1, w->d, x, T, lay, false, (hipStream_t)stream);
  }
  return device_result(ctx, e, "moe_expert_ffn");
}

namespace {
moe_status check_layer(moe_ctx* ctx, const char* fn, const moe_layer* L) {
  if (!L) return fail(ctx, MOE_E_INVALID, "%s: layer is NULL", fn);
  moe_status st = check_weights(ctx, fn, "experts", &L->experts);
  if (st != MOE_OK) return st;
  const int E = L->experts.n_experts, d = L->experts.d;
  if (L->router != MOE_ROUTER_SIGMOID_BIAS && L->router != MOE_ROUTER_SOFTMAX)
    return fail(ctx, MOE_E_INVALID, "%s: unknown router %d", fn, L->router);
  if (E > moe::kMaxE)
    return fail(ctx, MOE_E_INVALID, "%s: E=%d above %d", fn, E, moe::kMaxE);
  if (L->k < 1 || L->k > E || L->k > moe::kMaxK)
    return fail(ctx, MOE_E_INVALID, "%s: k=%d outside [1, min(E=%d, %d)]", fn, L->k, E,
                moe::kMaxK);
  if (!std::isfinite(L->scale)) return fail(ctx, MOE_E_INVALID, "%s: scale is not finite", fn);
  if (L->router == MOE_ROUTER_SOFTMAX && L->bias)
    return fail(ctx, MOE_E_INVALID, "%s: the softmax router takes no bias", fn);
  if (!L->w_router) return fail(ctx, MOE_E_INVALID, "%s: w_router is NULL", fn);
  if (!aligned16(L->w_router) || !aligned16(L->bias))
    return fail(ctx, MOE_E_INVALID, "%s: a pointer is not 16-byte aligned", fn);
  if (L->shared.n_experts != 0) {
    if (L->shared.n_experts != 1)
      return fail(ctx, MOE_E_INVALID, "%s: shared.n_experts=%d (0 or 1)", fn,
                  L->shared.n_experts);
    st = check_weights(ctx, fn, "shared", &L->shared);
    if (st != MOE_OK) return st;
    if (L->shared.d != d)
      return fail(ctx, MOE_E_INVALID, "%s: shared.d=%d differs from d=%d", fn, L->shared.d, d);
  }
  return MOE_OK;
}
}  // namespace

moe_status moe_layer_workspace_size(const moe_ctx* cctx, const moe_layer* L, int T,
                                    size_t* bytes) {
  moe_ctx* ctx = const_cast<moe_ctx*>(cctx);
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (!bytes) return fail(ctx, MOE_E_INVALID, "moe_layer_workspace_size: bytes is NULL");
  moe_status st = check_layer(ctx, "moe_layer_workspace_size", L);
  if (st != MOE_OK) return st;
  if (T < 0 || (long long)T * L->k > 0x7fffffffLL)
    return fail(ctx, MOE_E_INVALID, "moe_layer_workspace_size: T=%d", T);
  *bytes = fwd_layout(nullptr, L, T).bytes;
  return MOE_OK;
}

moe_status moe_forward(moe_ctx* ctx, const moe_layer* L, int act, const float* x, int T,
                       const float* residual, float* y, int32_t* topk_idx, float* topk_w,
                       void* ws, size_t ws_bytes, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = check_layer(ctx, "moe_forward", L);
  if (st != MOE_OK) return st;
  if (act != MOE_ACT_SILU && act != MOE_ACT_GELU_TANH)
    return fail(ctx, MOE_E_UNSUPPORTED,
                "moe_forward: unsupported activation=%d (MOE_ACT_SILU=0 or MOE_ACT_GELU_TANH=1)",
                act);
  if (T < 0 || (long long)T * L->k > 0x7fffffffLL)
    return fail(ctx, MOE_E_INVALID, "moe_forward: T=%d", T);
  if (T == 0) return MOE_OK;
  if (!x || !y) return fail(ctx, MOE_E_INVALID, "moe_forward: %s is NULL", !x ? "x" : "y");
  if (!aligned16(x) || !aligned16(y) || !aligned16(residual) || !aligned16(topk_idx) ||
      !aligned16(topk_w))
    return fail(ctx, MOE_E_INVALID, "moe_forward: a pointer is not 16-byte aligned");
  FwdWs f = fwd_layout(ws, L, T);
  if (!ws || ws_bytes < f.bytes || !aligned16(ws))
    return fail(ctx, MOE_E_WORKSPACE, "moe_forward: workspace %s (need %zu bytes, got %zu)",
                !ws ? "is NULL" : !aligned16(ws) ? "is not 16-byte aligned" : "too small",
                f.bytes, ws_bytes);
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "moe_forward: hipSetDevice(%d) failed", ctx->device);
  hipStream_t s = (hipStream_t)stream;
  const int E = L->experts.n_experts, d = L->experts.d, k = L->k, R = T * k;
  int32_t* idx = topk_idx ? topk_idx : f.idx;
  float* w = topk_w ? topk_w : f.w;
  const bool has_sh = L->shared.n_experts > 0;
  const bool fused = has_sh && L->shared.fmt == L->experts.fmt &&
                     L->shared.layout == L->experts.layout && L->experts.fmt != MOE_W_FP32;
  const moe_weights& X = L->experts;
  const moe_weights& S = L->shared;
  // When every expert set reads x as digits, the selection kernel encodes x
  // too (its row loads overlap the selection); small batches also skip the
  // permutation (the FFN groups the pairs itself).
  const bool enc = X.fmt != MOE_W_FP32 && (fused || !has_sh);
  const bool small = enc && T <= moe::kSmallT;
  hipError_t e;
  if (enc) {
    int Rs[2] = {R, T}, Is[2] = {X.inter, S.inter};
    moe::FfnWs lay = moe::ffn_ws_layout(f.ffn, T, d, fused ? 2 : 1, Rs, Is, true);
    // x digits in the order the routed experts' kernels read (int4: permuted)
    const bool perm = X.fmt == MOE_W_INT4_B32 || X.fmt == MOE_W_INT4_B128;
    e = moe::launch_router_encode(L->router, x, L->w_router, L->bias, L->expert_mask, T, d, E,
                                  k, L->scale, idx, w, f.partial, lay.xq, lay.xs, perm, lay.cnt,
                                  s);
    if (e == hipSuccess && !small)
      e = moe::launch_permute(idx, T, k, E, f.offsets, f.row_token, f.token_row, s);
  } else {
    e = moe::launch_router(L->router, x, L->w_router, L->bias, L->expert_mask, T, d, E, k,
                           L->scale, idx, w, f.partial, s);
    if (e == hipSuccess)
      e = moe::launch_permute(idx, T, k, E, f.offsets, f.row_token, f.token_row, s);
  }
  if (e != hipSuccess) return device_result(ctx, e, "moe_forward");
  if (fused) {
    int Rs[2] = {R, T}, Is[2] = {X.inter, S.inter};
    moe::FfnWs lay = moe::ffn_ws_layout(f.ffn, T, d, 2, Rs, Is, true);
    moe::FfnSet sets[2] = {
        {X.fmt, X.layout, E, X.inter, R, X.w_gate_up, X.s_gate_up, X.w_down, X.s_down, f.row_token,
         f.offsets, lay.hq[0], lay.hs[0], f.rows, small ? idx : nullptr, k, act},
        {S.fmt, S.layout, 1, S.inter, T, S.w_gate_up, S.s_gate_up, S.w_down, S.s_down, nullptr,
         nullptr, lay.hq[1], lay.hs[1], f.sh_rows, nullptr, 1, act}};
    e = moe::launch_ffn_quant(sets, 2, d, x, T, lay, enc, s);
  } else {
    auto run = [&](const moe_weights& W, int Ew, int Rw, const int32_t* rt, const int32_t* of,
                   float* out) -> hipError_t {
      int Iw = W.inter;
      if (W.fmt == MOE_W_FP32) {
        moe::FfnWs lay = moe::ffn_ws_layout(f.ffn, T, d, 1, &Rw, &Iw, false);
        return moe::launch_ffn_f32(static_cast<const float*>(W.w_gate_up),
                                   static_cast<const float*>(W.w_down), Ew, d, W.inter, x, T, rt,
                                   of, Rw, out, lay.h, act, s);
      }
      moe::FfnWs lay = moe::ffn_ws_layout(f.ffn, T, d, 1, &Rw, &Iw, true);
      const bool pairs = small && &W == &X;
      moe::FfnSet set{W.fmt, W.layout, Ew, W.inter, Rw, W.w_gate_up, W.s_gate_up, W.w_down,
                      W.s_down, rt, of, lay.hq[0], lay.hs[0], out, pairs ? idx : nullptr, k,
                      act};
      // x was encoded by the router when only routed experts run here
      return moe::launch_ffn_quant(&set, 1, d, x, T, lay, enc && &W == &X, s);
    };
    e = run(X, E, R, f.row_token, f.offsets, f.rows);
    if (e == hipSuccess && has_sh) e = run(S, 1, T, nullptr, nullptr, f.sh_rows);
  }
  if (e == hipSuccess)  // small batches leave the rows in (token, slot) order
    e = moe::launch_combine(f.rows, small ? nullptr : f.token_row, w,
                            has_sh ? f.sh_rows : nullptr, residual, T, k, d, y, s);
  return device_result(ctx, e, "moe_forward");
}

moe_status moe_tile_weights(moe_ctx* ctx, const moe_weights* src, void* dst_gate_up,
                            void* dst_down, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (!src) return fail(ctx, MOE_E_INVALID, "moe_tile_weights: src is NULL");
  moe_status st = check_weights(ctx, "moe_tile_weights", "src", src);
  if (st != MOE_OK) return st;
  if (src->fmt == MOE_W_FP32)
    return fail(ctx, MOE_E_UNSUPPORTED, "moe_tile_weights: fp32 weights have no tiled layout");
  if (src->layout != MOE_LAYOUT_ROWS)
    return fail(ctx, MOE_E_INVALID, "moe_tile_weights: src layout must be MOE_LAYOUT_ROWS");
  if (!dst_gate_up || !dst_down || !aligned16(dst_gate_up) || !aligned16(dst_down))
    return fail(ctx, MOE_E_INVALID, "moe_tile_weights: a destination is NULL or misaligned");
  const long long E = src->n_experts, d = src->d, I = src->inter;
  const long long half = src->fmt == MOE_W_INT8_ROW ? 1 : 2;
  const long long gu_bytes = E * 2 * I * d / half, dn_bytes = E * d * I / half;
  auto overlap = [](const void* a, long long na, const void* b, long long nb) {
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
  };
  if (overlap(dst_gate_up, gu_bytes, src->w_gate_up, gu_bytes) ||
      overlap(dst_down, dn_bytes, src->w_down, dn_bytes) ||
      overlap(dst_gate_up, gu_bytes, dst_down, dn_bytes))
    return fail(ctx, MOE_E_INVALID, "moe_tile_weights: buffers overlap");
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_tile_weights: hipSetDevice(%d) failed", ctx->device);
  hipError_t e = moe::launch_tile_weights(src->fmt, src->w_gate_up, dst_gate_up, E * 2 * I,
                                          (int)d, (hipStream_t)stream);
  if (e == hipSuccess)
    e = moe::launch_tile_weights(src->fmt, src->w_down, dst_down, E * d, (int)I,
                                 (hipStream_t)stream);
  return device_result(ctx, e, "moe_tile_weights");
}

moe_status moe_combine(moe_ctx* ctx, const float* rows, const int32_t* token_row,
                       const float* topk_w, const float* shared, const float* residual, int T,
                       int k, int d, float* y, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (T < 0 || k < 1 || k > moe::kMaxK || d < 1)
    return fail(ctx, MOE_E_INVALID, "moe_combine: T=%d k=%d d=%d", T, k, d);
  if (d % 4 != 0)
    return fail(ctx, MOE_E_UNSUPPORTED, "moe_combine: d=%d is not a multiple of 4", d);
  if (T == 0) return MOE_OK;
  if (!rows || !topk_w || !y)
    return fail(ctx, MOE_E_INVALID, "moe_combine: %s is NULL",
                !rows ? "rows" : !topk_w ? "topk_w" : "y");
  if (!aligned16(rows) || !aligned16(token_row) || !aligned16(topk_w) || !aligned16(shared) ||
      !aligned16(residual) || !aligned16(y))
    return fail(ctx, MOE_E_INVALID, "moe_combine: a pointer is not 16-byte aligned");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "moe_combine: hipSetDevice(%d) failed", ctx->device);
  hipError_t e = moe::launch_combine(rows, token_row, topk_w, shared, residual, T, k, d, y,
                                     (hipStream_t)stream);
  return device_result(ctx, e, "moe_combine");
}

}  // extern "C"
