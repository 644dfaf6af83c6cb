// Argument checks of the C ABI; see checks.h.  Plain host C++ (built into the
// library and, for the CPU tests, on its own with the host compiler).
#include "checks.h"

#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "layout.h"

namespace moe {

moe_status errorf(char* err, moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(err, kErrBytes, fmt, ap);
  va_end(ap);
  return st;
}

namespace {
bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

const char* ws_problem(const void* ws, size_t got, size_t need) {
  return !ws ? "is NULL" : !aligned16(ws) ? "is not 16-byte aligned"
                                          : got < need ? "too small" : nullptr;
}
}  // namespace

bool forward_small(const moe_layer* L, int T) {
  const bool has_sh = L->shared.n_experts > 0;
  const bool enc = L->experts.fmt != MOE_W_FP32 && (layer_fused(L) || !has_sh);
  return enc && T <= kSmallT;
}

moe_status check_workspace_size(char* err, int T, int k, int E, int d, int inter, int fmt,
                                const size_t* bytes) {
  if (!bytes) return errorf(err, MOE_E_INVALID, "moe_workspace_size: bytes is NULL");
  if (T < 0 || k < 1 || E < 1 || d < 1 || inter < 1)
    return errorf(err, MOE_E_INVALID,
                  "moe_workspace_size: need T >= 0, k >= 1, E >= 1, d >= 1, inter >= 1 "
                  "(got T=%d k=%d E=%d d=%d inter=%d)", T, k, E, d, inter);
  if (fmt < MOE_W_FP32 || fmt > MOE_W_INT4_B128)
    return errorf(err, MOE_E_INVALID, "moe_workspace_size: unknown weight format %d", fmt);
  if ((long long)T * k > 0x7fffffffLL)
    return errorf(err, MOE_E_INVALID, "moe_workspace_size: T*k overflows");
  return MOE_OK;
}

moe_status check_route(char* err, int router, const float* x, const float* w_router,
                       const float* bias, int T, int d, int E, int k, float scale,
                       const int32_t* topk_idx, const float* topk_w, const void* ws,
                       size_t ws_bytes) {
  if (router != MOE_ROUTER_SIGMOID_BIAS && router != MOE_ROUTER_SOFTMAX)
    return errorf(err, MOE_E_INVALID, "moe_route: unknown router %d", router);
  if (T < 0) return errorf(err, MOE_E_INVALID, "moe_route: T=%d is negative", T);
  if (E < 1 || E > kMaxE)
    return errorf(err, MOE_E_INVALID, "moe_route: E=%d outside [1, %d]", E, kMaxE);
  if (k < 1 || k > E || k > kMaxK)
    return errorf(err, MOE_E_INVALID, "moe_route: k=%d outside [1, min(E=%d, %d)]", k, E, kMaxK);
  if (d < 1) return errorf(err, MOE_E_INVALID, "moe_route: d=%d", d);
  if (d % 64 != 0)
    return errorf(err, MOE_E_UNSUPPORTED, "moe_route: d=%d is not a multiple of 64", d);
  if (d > kMaxWidth)
    return errorf(err, MOE_E_UNSUPPORTED, "moe_route: d=%d above %d", d, kMaxWidth);
  if (!std::isfinite(scale)) return errorf(err, MOE_E_INVALID, "moe_route: scale is not finite");
  if (router == MOE_ROUTER_SOFTMAX && bias)
    return errorf(err, MOE_E_INVALID, "moe_route: the softmax router takes no bias");
  if ((long long)T * k > 0x7fffffffLL)
    return errorf(err, MOE_E_INVALID, "moe_route: T*k overflows");
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w)
    return errorf(err, MOE_E_INVALID, "moe_route: %s is NULL",
                  !x ? "x" : !w_router ? "w_router" : !topk_idx ? "topk_idx" : "topk_w");
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(bias) || !aligned16(topk_idx) ||
      !aligned16(topk_w))
    return errorf(err, MOE_E_INVALID, "moe_route: a pointer is not 16-byte aligned");
  const size_t need = route_ws_bytes(T, d, E);
  if (const char* why = ws_problem(ws, ws_bytes, need))
    return errorf(err, MOE_E_WORKSPACE, "moe_route: workspace %s (need %zu bytes, got %zu)", why,
                  need, ws_bytes);
  return MOE_OK;
}

moe_status check_expert_counts(char* err, const int32_t* topk_idx, int T, int k, int E,
                               const unsigned long long* counts) {
  if (T < 0 || k < 1 || (long long)T * k > 0x7fffffffLL)
    return errorf(err, MOE_E_INVALID, "moe_expert_counts: T=%d k=%d", T, k);
  if (E < 1 || E > kMaxE)
    return errorf(err, MOE_E_INVALID, "moe_expert_counts: E=%d outside [1, %d]", E, kMaxE);
  if (T == 0) return MOE_OK;
  if (!topk_idx || !counts)
    return errorf(err, MOE_E_INVALID, "moe_expert_counts: %s is NULL",
                  !topk_idx ? "topk_idx" : "counts");
  if (!aligned16(topk_idx) || (reinterpret_cast<uintptr_t>(counts) & 7) != 0)
    return errorf(err, MOE_E_INVALID, "moe_expert_counts: a pointer is misaligned");
  return MOE_OK;
}

moe_status check_quantize(char* err, int fmt, int in_type, const void* w, long long rows, int K,
                          const void* codes, const float* scales) {
  if (fmt != MOE_W_INT8_ROW && fmt != MOE_W_INT4_B32 && fmt != MOE_W_INT4_B128)
    return errorf(err, MOE_E_UNSUPPORTED, "moe_quantize: format %d has no quantizer", fmt);
  if (in_type != MOE_IN_F32 && in_type != MOE_IN_BF16)
    return errorf(err, MOE_E_INVALID, "moe_quantize: unknown input type %d", in_type);
  if (rows < 0) return errorf(err, MOE_E_INVALID, "moe_quantize: rows=%lld is negative", rows);
  const int kmul = fmt == MOE_W_INT8_ROW ? 8 : (fmt == MOE_W_INT4_B32 ? 32 : 128);
  if (K < kmul || K % kmul != 0 || K > (1 << 24))
    return errorf(err, MOE_E_UNSUPPORTED,
                  "moe_quantize: K=%d must be a positive multiple of %d, at most 2^24", K, kmul);
  if (rows > (1LL << 32) || rows > (1LL << 40) / K)
    return errorf(err, MOE_E_UNSUPPORTED, "moe_quantize: rows above 2^32 or rows*K above 2^40");
  if (rows == 0) return MOE_OK;
  if (!w || !codes || !scales)
    return errorf(err, MOE_E_INVALID, "moe_quantize: %s is NULL",
                  !w ? "w" : !codes ? "codes" : "scales");
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales))
    return errorf(err, MOE_E_INVALID, "moe_quantize: a pointer is not 16-byte aligned");
  return MOE_OK;
}

moe_status check_permute(char* err, const int32_t* topk_idx, int T, int k, int E,
                         const int32_t* offsets, const int32_t* row_token,
                         const int32_t* token_row) {
  if (T < 0) return errorf(err, MOE_E_INVALID, "moe_permute: T=%d is negative", T);
  if (E < 1 || E > kMaxE)
    return errorf(err, MOE_E_INVALID, "moe_permute: E=%d outside [1, %d]", E, kMaxE);
  if (k < 1 || k > kMaxK)
    return errorf(err, MOE_E_INVALID, "moe_permute: k=%d outside [1, %d]", k, kMaxK);
  if ((long long)T * k > 0x7fffffffLL)
    return errorf(err, MOE_E_INVALID, "moe_permute: T*k overflows");
  if (!offsets) return errorf(err, MOE_E_INVALID, "moe_permute: offsets is NULL");
  if (T > 0 && (!topk_idx || !row_token || !token_row))
    return errorf(err, MOE_E_INVALID, "moe_permute: %s is NULL",
                  !topk_idx ? "topk_idx" : !row_token ? "row_token" : "token_row");
  if (!aligned16(topk_idx) || !aligned16(offsets) || !aligned16(row_token) ||
      !aligned16(token_row))
    return errorf(err, MOE_E_INVALID, "moe_permute: a pointer is not 16-byte aligned");
  return MOE_OK;
}

moe_status check_weights(char* err, const char* fn, const char* which, const moe_weights* w) {
  if (!w) return errorf(err, MOE_E_INVALID, "%s: %s is NULL", fn, which);
  if (w->fmt < MOE_W_FP32 || w->fmt > MOE_W_INT4_B128)
    return errorf(err, MOE_E_INVALID, "%s: %s: unknown weight format %d", fn, which, w->fmt);
  if (w->n_experts < 1 || w->d < 1 || w->inter < 1)
    return errorf(err, MOE_E_INVALID, "%s: %s: n_experts=%d d=%d inter=%d", fn, which,
                  w->n_experts, w->d, w->inter);
  if (w->d > kMaxWidth || w->inter > kMaxWidth)
    return errorf(err, MOE_E_UNSUPPORTED, "%s: %s: d=%d and inter=%d must be at most %d", fn,
                  which, w->d, w->inter, kMaxWidth);
  const int mult = w->fmt == MOE_W_INT4_B32 || w->fmt == MOE_W_INT4_B128 ? 128 : 64;
  if (w->d % mult != 0 || w->inter % mult != 0)
    return errorf(err, MOE_E_UNSUPPORTED, "%s: %s: d=%d and inter=%d must be multiples of %d",
                  fn, which, w->d, w->inter, mult);
  if (w->layout != MOE_LAYOUT_ROWS && w->layout != MOE_LAYOUT_TILED)
    return errorf(err, MOE_E_INVALID, "%s: %s: unknown layout %d", fn, which, w->layout);
  if (w->layout == MOE_LAYOUT_TILED && w->fmt == MOE_W_FP32)
    return errorf(err, MOE_E_UNSUPPORTED, "%s: %s: fp32 weights have no tiled layout", fn,
                  which);
  if (!w->w_gate_up || !w->w_down)
    return errorf(err, MOE_E_INVALID, "%s: %s: weights are NULL", fn, which);
  if (w->fmt != MOE_W_FP32 && (!w->s_gate_up || !w->s_down))
    return errorf(err, MOE_E_INVALID, "%s: %s: scales are NULL for a quantised format", fn,
                  which);
  if (!aligned16(w->w_gate_up) || !aligned16(w->w_down) || !aligned16(w->s_gate_up) ||
      !aligned16(w->s_down))
    return errorf(err, MOE_E_INVALID, "%s: %s: a pointer is not 16-byte aligned", fn, which);
  return MOE_OK;
}

moe_status check_expert_ffn(char* err, const moe_weights* w, int act, const float* x, int T,
                            const int32_t* row_token, const int32_t* offsets, int R_max,
                            const float* rows_out, const void* ws, size_t ws_bytes) {
  if (!w) return errorf(err, MOE_E_INVALID, "moe_expert_ffn: weights is NULL");
  if (act != MOE_ACT_SILU && act != MOE_ACT_GELU_TANH)
    return errorf(err, MOE_E_UNSUPPORTED,
                  "moe_expert_ffn: unsupported activation=%d (MOE_ACT_SILU=0 or "
                  "MOE_ACT_GELU_TANH=1)", act);
  moe_status st = check_weights(err, "moe_expert_ffn", "weights", w);
  if (st != MOE_OK) return st;
  if (T < 0 || R_max < 0)
    return errorf(err, MOE_E_INVALID, "moe_expert_ffn: T=%d R_max=%d", T, R_max);
  if (!offsets && w->n_experts != 1)
    return errorf(err, MOE_E_INVALID, "moe_expert_ffn: offsets may be NULL only for one expert");
  if (!offsets && !row_token && R_max > T)
    return errorf(err, MOE_E_INVALID,
                  "moe_expert_ffn: with identity rows R_max=%d may not exceed T=%d", R_max, T);
  if (T == 0 || R_max == 0) return MOE_OK;
  if (!x || !rows_out)
    return errorf(err, MOE_E_INVALID, "moe_expert_ffn: %s is NULL", !x ? "x" : "rows_out");
  if (!aligned16(x) || !aligned16(row_token) || !aligned16(offsets) || !aligned16(rows_out))
    return errorf(err, MOE_E_INVALID, "moe_expert_ffn: a pointer is not 16-byte aligned");
  const size_t need = ffn_need(T, R_max, w->d, w->inter, w->fmt);
  if (const char* why = ws_problem(ws, ws_bytes, need))
    return errorf(err, MOE_E_WORKSPACE, "moe_expert_ffn: workspace %s (need %zu bytes, got %zu)",
                  why, need, ws_bytes);
  return MOE_OK;
}

moe_status check_layer(char* err, const char* fn, const moe_layer* L) {
  if (!L) return errorf(err, MOE_E_INVALID, "%s: layer is NULL", fn);
  moe_status st = check_weights(err, fn, "experts", &L->experts);
  if (st != MOE_OK) return st;
  const int E = L->experts.n_experts, d = L->experts.d;
  if (L->router != MOE_ROUTER_SIGMOID_BIAS && L->router != MOE_ROUTER_SOFTMAX)
    return errorf(err, MOE_E_INVALID, "%s: unknown router %d", fn, L->router);
  if (E > kMaxE) return errorf(err, MOE_E_INVALID, "%s: E=%d above %d", fn, E, kMaxE);
  if (L->k < 1 || L->k > E || L->k > kMaxK)
    return errorf(err, MOE_E_INVALID, "%s: k=%d outside [1, min(E=%d, %d)]", fn, L->k, E,
                  kMaxK);
  if (!std::isfinite(L->scale)) return errorf(err, MOE_E_INVALID, "%s: scale is not finite", fn);
  if (L->router == MOE_ROUTER_SOFTMAX && L->bias)
    return errorf(err, MOE_E_INVALID, "%s: the softmax router takes no bias", fn);
  if (!L->w_router) return errorf(err, MOE_E_INVALID, "%s: w_router is NULL", fn);
  if (!aligned16(L->w_router) || !aligned16(L->bias))
    return errorf(err, MOE_E_INVALID, "%s: a pointer is not 16-byte aligned", fn);
  if (L->shared.n_experts != 0) {
    if (L->shared.n_experts != 1)
      return errorf(err, MOE_E_INVALID, "%s: shared.n_experts=%d (0 or 1)", fn,
                    L->shared.n_experts);
    st = check_weights(err, fn, "shared", &L->shared);
    if (st != MOE_OK) return st;
    if (L->shared.d != d)
      return errorf(err, MOE_E_INVALID, "%s: shared.d=%d differs from d=%d", fn, L->shared.d, d);
  }
  return MOE_OK;
}

moe_status check_layer_workspace_size(char* err, const moe_layer* L, int T, const size_t* bytes) {
  if (!bytes) return errorf(err, MOE_E_INVALID, "moe_layer_workspace_size: bytes is NULL");
  moe_status st = check_layer(err, "moe_layer_workspace_size", L);
  if (st != MOE_OK) return st;
  if (T < 0 || (long long)T * L->k > 0x7fffffffLL)
    return errorf(err, MOE_E_INVALID, "moe_layer_workspace_size: T=%d", T);
  return MOE_OK;
}

moe_status check_forward(char* err, const char* fn, const moe_layer* L, int act, const float* x,
                         int T, const float* residual, const float* y, const int32_t* topk_idx,
                         const float* topk_w, const void* ws, size_t ws_bytes, int cu_count) {
  moe_status st = check_layer(err, fn, L);
  if (st != MOE_OK) return st;
  if (act != MOE_ACT_SILU && act != MOE_ACT_GELU_TANH)
    return errorf(err, MOE_E_UNSUPPORTED,
                  "%s: unsupported activation=%d (MOE_ACT_SILU=0 or MOE_ACT_GELU_TANH=1)",
                  fn, act);
  if (T < 0 || (long long)T * L->k > 0x7fffffffLL)
    return errorf(err, MOE_E_INVALID, "%s: T=%d", fn, T);
  if (T == 0) return MOE_OK;
  if (!x || !y) return errorf(err, MOE_E_INVALID, "%s: %s is NULL", fn, !x ? "x" : "y");
  if (!aligned16(x) || !aligned16(y) || !aligned16(residual) || !aligned16(topk_idx) ||
      !aligned16(topk_w))
    return errorf(err, MOE_E_INVALID, "%s: a pointer is not 16-byte aligned", fn);
  const FwdWs f = fwd_layout(nullptr, L, T);
  if (const char* why = ws_problem(ws, ws_bytes, f.bytes))
    return errorf(err, MOE_E_WORKSPACE, "%s: workspace %s (need %zu bytes, got %zu)", fn, why,
                  f.bytes, ws_bytes);
  if (forward_small(L, T)) {
    // small batches may split K across workgroups, which meet in the
    // workspace's join area: the launch plan (plan.h, the one the launcher
    // computes) must fit it
    const moe_weights& X = L->experts;
    const FfnPlan p = plan_ffn(X.fmt, T, T * L->k, X.n_experts, true, X.d, X.inter,
                               layer_fused(L) ? L->shared.inter : 0, cu_count, true);
    if (!p.ok)
      return errorf(err, MOE_E_UNSUPPORTED,
                    "%s: the small-batch launch plan for T=%d, E=%d, d=%d, inter=%d "
                    "exceeds the split-K join area (%d slots)", fn, T, X.n_experts, X.d, X.inter,
                    kSplitSlots);
  }
  return MOE_OK;
}

moe_status check_forward_chained(char* err, const moe_layer* L, int act, const float* x,
                                 const moe_pending* in, const float* x_out, int T,
                                 const moe_pending* out, const int32_t* topk_idx,
                                 const float* topk_w, const void* ws, size_t ws_bytes,
                                 int cu_count) {
  const char* fn = "moe_forward_chained";
  if (!out) return errorf(err, MOE_E_INVALID, "%s: out is NULL", fn);
  if ((x == nullptr) == (in == nullptr))
    return errorf(err, MOE_E_INVALID, "%s: give exactly one of x and in", fn);
  moe_status st = check_layer(err, fn, L);
  if (st != MOE_OK) return st;
  if (T < 0) return errorf(err, MOE_E_INVALID, "%s: T=%d", fn, T);
  if (T > kSmallT || (T > 0 && !forward_small(L, T)))
    return errorf(err, MOE_E_UNSUPPORTED,
                  "%s: only layers on the small-batch path chain (T <= %d, quantised experts, "
                  "a shared expert in the routed experts' format and layout)", fn, kSmallT);
  if (in) {
    const int d = L->experts.d;
    if (in->T != T || in->d != d || in->k < 1 || in->k > kMaxK)
      return errorf(err, MOE_E_INVALID, "%s: in has T=%d d=%d k=%d (layer: T=%d d=%d)", fn,
                    in->T, in->d, in->k, T, d);
    if (T > 0) {
      if (!in->rows || !in->w || !x_out)
        return errorf(err, MOE_E_INVALID, "%s: %s is NULL", fn,
                      !in->rows ? "in->rows" : !in->w ? "in->w" : "x_out");
      if (!aligned16(in->rows) || !aligned16(in->w) || !aligned16(in->shared) ||
          !aligned16(in->residual) || !aligned16(x_out))
        return errorf(err, MOE_E_INVALID, "%s: a pointer is not 16-byte aligned", fn);
      auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
        if (!a || !b) return false;
        const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
        return pa < pb + nb && pb < pa + na;
      };
      const size_t row = (size_t)d * sizeof(float), nx = (size_t)T * row;
      if (overlap(x_out, nx, in->rows, (size_t)T * in->k * row) ||
          overlap(x_out, nx, in->shared, nx) || overlap(x_out, nx, in->residual, nx) ||
          overlap(x_out, nx, in->w, (size_t)T * in->k * sizeof(float)))
        return errorf(err, MOE_E_INVALID, "%s: x_out overlaps the pending input", fn);
    }
  }
  // the rest as moe_forward's (the layer's input is x_out when chained; the
  // output rows stay in ws, so x stands in for y)
  const float* xin = in ? x_out : x;
  return check_forward(err, fn, L, act, xin, T, nullptr, xin, topk_idx, topk_w, ws, ws_bytes,
                       cu_count);
}

moe_status check_tile_weights(char* err, const moe_weights* src, const void* dst_gate_up,
                              const void* dst_down) {
  if (!src) return errorf(err, MOE_E_INVALID, "moe_tile_weights: src is NULL");
  moe_status st = check_weights(err, "moe_tile_weights", "src", src);
  if (st != MOE_OK) return st;
  if (src->fmt == MOE_W_FP32)
    return errorf(err, MOE_E_UNSUPPORTED, "moe_tile_weights: fp32 weights have no tiled layout");
  if (src->layout != MOE_LAYOUT_ROWS)
    return errorf(err, MOE_E_INVALID, "moe_tile_weights: src layout must be MOE_LAYOUT_ROWS");
  if (!dst_gate_up || !dst_down || !aligned16(dst_gate_up) || !aligned16(dst_down))
    return errorf(err, MOE_E_INVALID, "moe_tile_weights: a destination is NULL or misaligned");
  const long long E = src->n_experts, d = src->d, I = src->inter;
  const long long half = src->fmt == MOE_W_INT8_ROW ? 1 : 2;
  const long long gu_bytes = E * 2 * I * d / half, dn_bytes = E * d * I / half;
  auto overlap = [](const void* a, long long na, const void* b, long long nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
  };
  if (overlap(dst_gate_up, gu_bytes, src->w_gate_up, gu_bytes) ||
      overlap(dst_down, dn_bytes, src->w_down, dn_bytes) ||
      overlap(dst_gate_up, gu_bytes, dst_down, dn_bytes))
    return errorf(err, MOE_E_INVALID, "moe_tile_weights: buffers overlap");
  return MOE_OK;
}

moe_status check_combine(char* err, const float* rows, const int32_t* token_row,
                         const float* topk_w, const float* shared, const float* residual, int T,
                         int k, int d, const float* y) {
  if (T < 0 || k < 1 || k > kMaxK || d < 1)
    return errorf(err, MOE_E_INVALID, "moe_combine: T=%d k=%d d=%d", T, k, d);
  if (d % 4 != 0)
    return errorf(err, MOE_E_UNSUPPORTED, "moe_combine: d=%d is not a multiple of 4", d);
  if ((long long)T * k > 0x7fffffffLL)
    return errorf(err, MOE_E_INVALID, "moe_combine: T*k overflows");
  if (T == 0) return MOE_OK;
  if (!rows || !topk_w || !y)
    return errorf(err, MOE_E_INVALID, "moe_combine: %s is NULL",
                  !rows ? "rows" : !topk_w ? "topk_w" : "y");
  if (!aligned16(rows) || !aligned16(token_row) || !aligned16(topk_w) || !aligned16(shared) ||
      !aligned16(residual) || !aligned16(y))
    return errorf(err, MOE_E_INVALID, "moe_combine: a pointer is not 16-byte aligned");
  return MOE_OK;
}

moe_status check_coverage_set(char* err, const unsigned long long* counts, int E, double cover,
                              int k, const int32_t* keep, const int32_t* n_keep) {
  if (E < 1 || E > kMaxE)
    return errorf(err, MOE_E_INVALID, "moe_coverage_set: E=%d outside [1, %d]", E, kMaxE);
  if (k < 1) return errorf(err, MOE_E_INVALID, "moe_coverage_set: k=%d must be positive", k);
  if (!(cover >= 0.0 && cover <= 1.0))
    return errorf(err, MOE_E_INVALID, "moe_coverage_set: cover=%g outside [0, 1]", cover);
  if (!counts || !keep || !n_keep)
    return errorf(err, MOE_E_INVALID, "moe_coverage_set: %s is NULL",
                  !counts ? "counts" : !keep ? "keep" : "n_keep");
  if (!aligned16(counts) || !aligned16(keep) || !aligned16(n_keep))
    return errorf(err, MOE_E_INVALID, "moe_coverage_set: a pointer is not 16-byte aligned");
  return MOE_OK;
}

moe_status check_probe_read(char* err, const void* buf, size_t bytes, int blocks,
                            const void* sink) {
  if (bytes < 16 || bytes % 16 != 0)
    return errorf(err, MOE_E_INVALID, "moe_probe_read: bytes=%zu is not a positive multiple "
                  "of 16", bytes);
  if (blocks < 0 || blocks > kProbeMaxBlocks)
    return errorf(err, MOE_E_INVALID, "moe_probe_read: blocks=%d outside [0, %d]", blocks,
                  kProbeMaxBlocks);
  if (!buf || !sink)
    return errorf(err, MOE_E_INVALID, "moe_probe_read: %s is NULL", !buf ? "buf" : "sink");
  if (!aligned16(buf) || !aligned16(sink))
    return errorf(err, MOE_E_INVALID, "moe_probe_read: a pointer is not 16-byte aligned");
  return MOE_OK;
}

moe_status check_probe_mfma(char* err, int shape, int iters, int blocks, const void* sink) {
  if (shape != MOE_PROBE_MFMA_16X16X64 && shape != MOE_PROBE_MFMA_32X32X32)
    return errorf(err, MOE_E_INVALID, "moe_probe_mfma: unknown shape %d", shape);
  if (iters < 1) return errorf(err, MOE_E_INVALID, "moe_probe_mfma: iters=%d", iters);
  if (blocks < 0 || blocks > kProbeMaxBlocks)
    return errorf(err, MOE_E_INVALID, "moe_probe_mfma: blocks=%d outside [0, %d]", blocks,
                  kProbeMaxBlocks);
  if (!sink) return errorf(err, MOE_E_INVALID, "moe_probe_mfma: sink is NULL");
  if (!aligned16(sink))
    return errorf(err, MOE_E_INVALID, "moe_probe_mfma: sink is not 16-byte aligned");
  return MOE_OK;
}

}  // namespace moe
