// Host side of the C ABI declared in include/moe.h: argument checks (pure
// host code, before anything is enqueued), workspace carving and kernel
// dispatch.  No allocation happens on any call path after moe_create.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <new>

#include "../../include/moe.h"
#include "internal.h"

namespace moe {
void set_max_lds(int bytes);
}

struct moe_ctx {
  int device;
  int cu_count;
  int max_lds;
  char arch[64];
  char err[512];
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
  return MOE_OK;
}

size_t ffn_need(int T, int R, int d, int inter, int fmt) {
  return moe::ffn_ws_layout(nullptr, T, R, d, inter, fmt != MOE_W_FP32).bytes;
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
  moe::set_max_lds(ctx->max_lds);
  *out = ctx;
  return MOE_OK;
}

void moe_destroy(moe_ctx* ctx) { delete ctx; }

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
  if (fmt < MOE_W_FP32 || fmt > MOE_W_INT4_B32)
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
  hipError_t e = moe::launch_router(router, x, w_router, bias, T, d, E, k, scale, topk_idx,
                                    topk_w, static_cast<float*>(ws), (hipStream_t)stream);
  return device_result(ctx, e, "moe_route");
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

moe_status moe_expert_ffn(moe_ctx* ctx, const moe_weights* w, int act, const float* x, int T,
                          const int32_t* row_token, const int32_t* offsets, int R_max,
                          float* rows_out, void* ws, size_t ws_bytes, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  if (!w) return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: weights is NULL");
  if (act != MOE_ACT_SILU)
    return fail(ctx, MOE_E_UNSUPPORTED,
                "moe_expert_ffn: unsupported activation=%d (only MOE_ACT_SILU=0)", act);
  if (w->fmt < MOE_W_FP32 || w->fmt > MOE_W_INT4_B32)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: unknown weight format %d", w->fmt);
  if (w->n_experts < 1 || w->d < 1 || w->inter < 1)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: n_experts=%d d=%d inter=%d", w->n_experts,
                w->d, w->inter);
  if (w->d % 64 != 0 || w->inter % 64 != 0)
    return fail(ctx, MOE_E_UNSUPPORTED,
                "moe_expert_ffn: d=%d and inter=%d must be multiples of 64", w->d, w->inter);
  if (T < 0 || R_max < 0)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: T=%d R_max=%d", T, R_max);
  if (!offsets && w->n_experts != 1)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: offsets may be NULL only for one expert");
  if (!offsets && !row_token && R_max > T)
    return fail(ctx, MOE_E_INVALID,
                "moe_expert_ffn: with identity rows R_max=%d may not exceed T=%d", R_max, T);
  if (T == 0 || R_max == 0) return MOE_OK;
  if (!x || !rows_out || !w->w_gate_up || !w->w_down)
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: %s is NULL",
                !x ? "x" : !rows_out ? "rows_out" : !w->w_gate_up ? "w_gate_up" : "w_down");
  if (w->fmt != MOE_W_FP32 && (!w->s_gate_up || !w->s_down))
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: scales are NULL for a quantised format");
  if (!aligned16(x) || !aligned16(row_token) || !aligned16(offsets) || !aligned16(rows_out) ||
      !aligned16(w->w_gate_up) || !aligned16(w->w_down) || !aligned16(w->s_gate_up) ||
      !aligned16(w->s_down))
    return fail(ctx, MOE_E_INVALID, "moe_expert_ffn: a pointer is not 16-byte aligned");
  const size_t need = ffn_need(T, R_max, w->d, w->inter, w->fmt);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(ctx, MOE_E_WORKSPACE, "moe_expert_ffn: workspace %s (need %zu bytes, got %zu)",
                !ws ? "is NULL" : !aligned16(ws) ? "is not 16-byte aligned" : "too small", need,
                ws_bytes);
  if (w->fmt != MOE_W_FP32) {
    const size_t lds = (size_t)moe::kTileRows * (2 * (size_t)(w->d > w->inter ? w->d : w->inter) + 16);
    if (lds > (size_t)ctx->max_lds)
      return fail(ctx, MOE_E_UNSUPPORTED,
                  "moe_expert_ffn: width %d needs %zu bytes of LDS per workgroup (device has %d)",
                  w->d > w->inter ? w->d : w->inter, lds, ctx->max_lds);
  }
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_expert_ffn: hipSetDevice(%d) failed", ctx->device);
  hipError_t e;
  if (w->fmt == MOE_W_FP32) {
    moe::FfnWs lay = moe::ffn_ws_layout(ws, T, R_max, w->d, w->inter, false);
    e = moe::launch_ffn_f32(static_cast<const float*>(w->w_gate_up),
                            static_cast<const float*>(w->w_down), w->n_experts, w->d, w->inter,
                            x, T, row_token, offsets, R_max, rows_out, lay.h,
                            (hipStream_t)stream);
  } else {
    moe::FfnWs lay = moe::ffn_ws_layout(ws, T, R_max, w->d, w->inter, true);
    e = moe::launch_ffn_quant(w->fmt, w->w_gate_up, w->s_gate_up, w->w_down, w->s_down,
                              w->n_experts, w->d, w->inter, x, T, row_token, offsets, R_max,
                              rows_out, lay, (hipStream_t)stream);
  }
  return device_result(ctx, e, "moe_expert_ffn");
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
  if (!rows || !token_row || !topk_w || !y)
    return fail(ctx, MOE_E_INVALID, "moe_combine: %s is NULL",
                !rows ? "rows" : !token_row ? "token_row" : !topk_w ? "topk_w" : "y");
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
