// Host side of the C ABI declared in include/moe.h: argument checks (pure
// host code, before anything is enqueued), workspace carving and kernel
// dispatch.  No allocation happens on any call path after moe_create.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/moe.h"
#include "checks.h"
#include "internal.h"

namespace moe {

const char* const kKernelNames[K_COUNT] = {
    "router_logits", "router_topk",     "permute",         "fill",
    "encode_rows",   "ffn_i8_gate_up",  "ffn_i8_down",     "ffn_i4_gate_up",
    "ffn_i4_down",   "ffn_f32_gate_up", "ffn_f32_down",    "combine",
    "router_tail",   "ffn_i8_gate_up_gemm", "ffn_i8_down_gemm", "quant_i8_rows",
    "quant_i4_blocks", "ffn_i4_gate_up_gemm", "ffn_i4_down_gemm"};

// Event pairs that launches record their kernels' start and stop on while a
// context has timing on.
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
};

thread_local KernelTimer* g_timer = nullptr;

void timer_open(int id) { g_timer->open_id = id; }

void timer_close() { g_timer->open_id = -1; }

bool timer_take(hipEvent_t* start, hipEvent_t* stop) {
  KernelTimer* t = g_timer;
  if (t->open_id < 0) return false;
  const int id = t->open_id;
  t->open_id = -1;
  if (t->next + 2 > t->pool.size()) {
    ++t->dropped;
    return false;
  }
  *start = t->pool[t->next++];
  *stop = t->pool[t->next++];
  t->marks.push_back({id, *start, *stop});
  return true;
}
}  // namespace moe

struct moe_ctx {
  int device;
  int cu_count;
  int max_lds;
  char arch[64];
  char err[moe::kErrBytes];
  bool timing;
  moe::KernelTimer timer;
  void* scratch;  // this device's copy of `scratch` (below), for moe_forward_noalloc
};

// The workspace of moe_forward_noalloc: one copy per GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, never device memory: every host use goes through the address
// hipGetSymbolAddress returns for the current device (scratch_address).
static constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on `device`, taken once per device with
// that device current.  NULL (and the HIP error in *err) on failure.
void* scratch_address(int device, hipError_t* err) {
  *err = hipSuccess;
  if (device < 0 || device >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[device]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_dev[device] = ptr;
  }
  return g_scratch_dev[device];
}

thread_local char g_create_err[512] = "";

moe_status fail(moe_ctx* ctx, moe_status st, const char* fmt, ...) {
  char* buf = ctx ? ctx->err : g_create_err;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, 512, fmt, ap);
  va_end(ap);
  return st;
}

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
  {
    DeviceGuard g(device);
    hipError_t se = g.ok ? hipSuccess : hipErrorInvalidDevice;
    ctx->scratch = g.ok ? scratch_address(device, &se) : nullptr;
    if (!ctx->scratch) {
      delete ctx;
      return fail(nullptr, MOE_E_DEVICE, "moe_create: address of the scratch array on device %d: "
                  "%s", device, hipGetErrorString(se));
    }
  }

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
  moe_status st = moe::check_workspace_size(ctx->err, T, k, E, d, inter, fmt, bytes);
  if (st != MOE_OK) return st;
  size_t a = moe::route_ws_bytes(T, d, E);
  size_t b = moe::ffn_need(T, T * k, d, inter, fmt);
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
  moe_status st = moe::check_route(ctx->err, router, x, w_router, bias, T, d, E, k, scale,
                                   topk_idx, topk_w, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
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
  moe_status st = moe::check_expert_counts(ctx->err, topk_idx, T, k, E, counts);
  if (st != MOE_OK || T == 0) return st;
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
  moe_status st = moe::check_quantize(ctx->err, fmt, in_type, w, rows, K, codes, scales);
  if (st != MOE_OK || rows == 0) return st;
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "moe_quantize: hipSetDevice(%d) failed", ctx->device);
  hipError_t e = moe::launch_quantize(fmt, in_type, w, rows, K, codes, scales,
                                      (hipStream_t)stream);
  return device_result(ctx, e, "moe_quantize");
}

moe_status moe_permute(moe_ctx* ctx, const int32_t* topk_idx, int T, int k, int E,
                       int32_t* offsets, int32_t* row_token, int32_t* token_row, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_permute(ctx->err, topk_idx, T, k, E, offsets, row_token, token_row);
  if (st != MOE_OK) return st;
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
  moe_status st = moe::check_expert_ffn(ctx->err, w, act, x, T, row_token, offsets, R_max,
                                        rows_out, ws, ws_bytes);
  if (st != MOE_OK || T == 0 || R_max == 0) return st;
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

moe_status moe_layer_workspace_size(const moe_ctx* cctx, const moe_layer* L, int T,
                                    size_t* bytes) {
  moe_ctx* ctx = const_cast<moe_ctx*>(cctx);
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_layer_workspace_size(ctx->err, L, T, bytes);
  if (st != MOE_OK) return st;
  *bytes = moe::fwd_layout(nullptr, L, T).bytes;
  return MOE_OK;
}

}  // extern "C"

namespace {
// The layer after its checks passed, with ws (at least fwd_layout's bytes)
// as the workspace: every launch of moe_forward and moe_forward_noalloc.
// chain (moe_forward_chained): the router launch forms x from the previous
// layer's pending output; pend: leave this layer's output pending there
// instead of combining (both only on the small-batch path, checked before).
moe_status forward_launch(moe_ctx* ctx, const moe_layer* L, int act, const float* x, int T,
                          const float* residual, float* y, int32_t* topk_idx, float* topk_w,
                          void* ws, void* stream, const char* fn,
                          const moe::ChainIn* chain = nullptr, moe_pending* pend = nullptr) {
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "%s: hipSetDevice(%d) failed", fn, ctx->device);
  const moe::FwdWs f = moe::fwd_layout(ws, L, T);
  hipStream_t s = (hipStream_t)stream;
  const int E = L->experts.n_experts, d = L->experts.d, k = L->k, R = T * k;
  int32_t* idx = topk_idx ? topk_idx : f.idx;
  float* w = topk_w ? topk_w : f.w;
  const bool has_sh = L->shared.n_experts > 0;
  const bool fused = moe::layer_fused(L);
  const moe_weights& X = L->experts;
  const moe_weights& S = L->shared;
  // When every expert set reads x as digits, the selection kernel encodes x
  // too (its row loads overlap the selection); small batches also skip the
  // permutation (the FFN groups the pairs itself).
  const bool enc = X.fmt != MOE_W_FP32 && (fused || !has_sh);
  const bool small = moe::forward_small(L, T);
  // x digits in the order the routed experts' kernels read (int4: permuted)
  const bool perm = X.fmt == MOE_W_INT4_B32 || X.fmt == MOE_W_INT4_B128;
  // one token: the gate/up launch selects and encodes for itself (SelIn)
  const bool selfsel = enc && small && T == 1 && E <= 256 && moe::sel_fits(d);
  moe::SelIn si{};
  if (selfsel)
    si = moe::SelIn{f.partial, (d + moe::kRouterChunk - 1) / moe::kRouterChunk, L->bias,
                    L->expert_mask, E, k, L->router, L->scale, chain ? chain->x_out : x,
                    idx, w, perm};
  hipError_t e;
  if (enc) {
    int Rs[2] = {R, T}, Is[2] = {X.inter, S.inter};
    moe::FfnWs lay = moe::ffn_ws_layout(f.ffn, T, d, fused ? 2 : 1, Rs, Is, true);
    e = moe::launch_router_encode(L->router, x, L->w_router, L->bias, L->expert_mask, T, d, E,
                                  k, L->scale, idx, w, f.partial, lay.xq, lay.xs, perm, lay.cnt,
                                  s, chain, selfsel);
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
    e = moe::launch_ffn_quant(sets, 2, d, x, T, lay, enc, s, selfsel ? &si : nullptr);
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
      return moe::launch_ffn_quant(&set, 1, d, x, T, lay, enc && &W == &X, s,
                                   selfsel && &W == &X ? &si : nullptr);
    };
    e = run(X, E, R, f.row_token, f.offsets, f.rows);
    if (e == hipSuccess && has_sh) e = run(S, 1, T, nullptr, nullptr, f.sh_rows);
  }
  if (e == hipSuccess && pend) {  // the next chained layer (or a moe_combine) sums them
    *pend = moe_pending{f.rows, has_sh ? f.sh_rows : nullptr, w, chain ? chain->x_out : x, T, k,
                        d};
    return MOE_OK;
  }
  if (e == hipSuccess)  // small batches leave the rows in (token, slot) order
    e = moe::launch_combine(f.rows, small ? nullptr : f.token_row, w,
                            has_sh ? f.sh_rows : nullptr, residual, T, k, d, y, s);
  return device_result(ctx, e, fn);
}
}  // namespace

extern "C" {

moe_status moe_forward(moe_ctx* ctx, const moe_layer* L, int act, const float* x, int T,
                       const float* residual, float* y, int32_t* topk_idx, float* topk_w,
                       void* ws, size_t ws_bytes, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_forward(ctx->err, "moe_forward", L, act, x, T, residual, y,
                                     topk_idx, topk_w, ws, ws_bytes, moe::device_cu_count());
  if (st != MOE_OK || T == 0) return st;
  return forward_launch(ctx, L, act, x, T, residual, y, topk_idx, topk_w, ws, stream,
                        "moe_forward");
}

moe_status moe_forward_chained(moe_ctx* ctx, const moe_layer* L, int act, const float* x,
                               const moe_pending* in, float* x_out, int T, moe_pending* out,
                               int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                               void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_forward_chained(ctx->err, L, act, x, in, x_out, T, out, topk_idx,
                                             topk_w, ws, ws_bytes, moe::device_cu_count());
  if (st != MOE_OK) return st;
  if (T == 0) {
    *out = moe_pending{nullptr, nullptr, nullptr, nullptr, 0, L->k, L->experts.d};
    return MOE_OK;
  }
  moe::ChainIn chain{};
  if (in) chain = moe::ChainIn{in->rows, in->shared, in->w, in->residual, in->k, x_out};
  return forward_launch(ctx, L, act, in ? x_out : x, T, nullptr, nullptr, topk_idx, topk_w, ws,
                        stream, "moe_forward_chained", in ? &chain : nullptr, out);
}

moe_status moe_forward_noalloc(moe_ctx* ctx, const moe_layer* L, int act, const float* x, int T,
                               const float* residual, float* y, int32_t* topk_idx,
                               float* topk_w, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_forward(ctx->err, "moe_forward_noalloc", L, act, x, T, residual, y,
                                     topk_idx, topk_w, ctx->scratch, kScratchBytes,
                                     moe::device_cu_count());
  if (st == MOE_E_WORKSPACE)  // the layer at T needs more than the library's scratch
    return fail(ctx, MOE_E_UNSUPPORTED,
                "moe_forward_noalloc: T=%d needs %zu bytes of workspace, above the %zu-byte "
                "scratch array; call moe_forward with a workspace", T,
                moe::fwd_layout(nullptr, L, T).bytes, kScratchBytes);
  if (st != MOE_OK || T == 0) return st;
  return forward_launch(ctx, L, act, x, T, residual, y, topk_idx, topk_w, ctx->scratch, stream,
                        "moe_forward_noalloc");
}

moe_status moe_tile_weights(moe_ctx* ctx, const moe_weights* src, void* dst_gate_up,
                            void* dst_down, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_tile_weights(ctx->err, src, dst_gate_up, dst_down);
  if (st != MOE_OK) return st;
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_tile_weights: hipSetDevice(%d) failed", ctx->device);
  const long long E = src->n_experts, d = src->d, I = src->inter;
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
  moe_status st = moe::check_combine(ctx->err, rows, token_row, topk_w, shared, residual, T, k, d,
                                     y);
  if (st != MOE_OK || T == 0) return st;
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(ctx, MOE_E_DEVICE, "moe_combine: hipSetDevice(%d) failed", ctx->device);
  hipError_t e = moe::launch_combine(rows, token_row, topk_w, shared, residual, T, k, d, y,
                                     (hipStream_t)stream);
  return device_result(ctx, e, "moe_combine");
}

moe_status moe_coverage_set(moe_ctx* ctx, const unsigned long long* counts, int E, double cover,
                            int k, int32_t* keep, int32_t* n_keep, void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_coverage_set(ctx->err, counts, E, cover, k, keep, n_keep);
  if (st != MOE_OK) return st;
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_coverage_set: hipSetDevice(%d) failed", ctx->device);
  return device_result(ctx, moe::launch_coverage_set(counts, E, cover, k, keep, n_keep,
                                                     (hipStream_t)stream),
                       "moe_coverage_set");
}

moe_status moe_probe_read(moe_ctx* ctx, const void* buf, size_t bytes, int blocks, void* sink,
                          void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_probe_read(ctx->err, buf, bytes, blocks, sink);
  if (st != MOE_OK) return st;
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_probe_read: hipSetDevice(%d) failed", ctx->device);
  const int nb = blocks > 0 ? blocks : 8 * ctx->cu_count;
  return device_result(ctx, moe::launch_probe_read(buf, bytes, nb, sink, (hipStream_t)stream),
                       "moe_probe_read");
}

moe_status moe_probe_mfma(moe_ctx* ctx, int shape, int iters, int blocks, void* sink,
                          void* stream) {
  if (check_ctx(ctx) != MOE_OK) return MOE_E_INVALID;
  moe_status st = moe::check_probe_mfma(ctx->err, shape, iters, blocks, sink);
  if (st != MOE_OK) return st;
  DeviceGuard g(ctx->device);
  if (!g.ok)
    return fail(ctx, MOE_E_DEVICE, "moe_probe_mfma: hipSetDevice(%d) failed", ctx->device);
  const int nb = blocks > 0 ? blocks : 8 * ctx->cu_count;
  return device_result(ctx, moe::launch_probe_mfma(shape, iters, nb, sink, (hipStream_t)stream),
                       "moe_probe_mfma");
}

}  // extern "C"
