// Limits and workspace layouts of the MoE library.  Plain host C++ (no HIP
// types): shared by the kernels' launchers, the C ABI's argument checks and
// the CPU tests of those checks.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "plan.h"

namespace moe {

// ---------------------------------------------------------------- limits
constexpr int kRouterChunk = 256;      // router logits are summed in fixed 256-input chunks
constexpr int kMaxK = 16;              // top-k limit
constexpr int kMaxE = 1024;            // experts per layer limit
constexpr int kMaxWidth = 16384;       // d and inter limit
// Up to kSmallT tokens moe_forward lets the router encode x and the FFN
// kernels group the (token, slot) pairs themselves (no permutation pass).
constexpr int kSmallT = 16;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- workspace layout
// Router: fp32 partial logits [ceil(d/256)][T][E].
inline size_t route_ws_bytes(int T, int d, int E) {
  size_t chunks = (size_t)((d + kRouterChunk - 1) / kRouterChunk);
  return align_up(chunks * (size_t)T * (size_t)E * sizeof(float), 256);
}

// Expert FFN, quantised formats (per expert set q = 0, 1):
//   xq    [T][2][d] int8     activations as two int8 digits (see ffn.hip)
//   xs    [T] fp32           per-row power-of-two scale of xq
//   hq[q] [R_q][2][I_q] int8 h = silu(gate) * up as two digits
//   hs[q] [R_q][I_q/64] fp32 scale per row and 64-column block
//   cnt, part: the split-K join area (plan.h)
// fp32 format: h [R][I] fp32 only.
struct FfnWs {
  int8_t* xq;
  float* xs;
  int8_t* hq[2];
  float* hs[2];
  float* h;
  int* cnt;     // split-K arrival counters (kSplitSlots), zero between launches
  float* part;  // split-K partial sums (kSplitSlots slots of kSplitSlotBytes)
  size_t bytes;
};

// rows/inter of up to two expert sets sharing one x; base NULL sizes only
inline FfnWs ffn_ws_layout(void* base, int T, int d, int nsets, const int* R, const int* inter,
                           bool quantised) {
  FfnWs w{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t n) {
    char* p = b ? b + off : nullptr;
    off = align_up(off + n, 256);
    return p;
  };
  if (quantised) {
    w.xq = reinterpret_cast<int8_t*>(take((size_t)T * 2 * d));
    w.xs = reinterpret_cast<float*>(take((size_t)T * sizeof(float)));
    for (int q = 0; q < nsets; ++q) {
      w.hq[q] = reinterpret_cast<int8_t*>(take((size_t)R[q] * 2 * inter[q]));
      w.hs[q] = reinterpret_cast<float*>(take((size_t)R[q] * (inter[q] / 64) * sizeof(float)));
    }
    w.cnt = reinterpret_cast<int*>(take((size_t)kSplitSlots * sizeof(int)));
    w.part = reinterpret_cast<float*>(take((size_t)kSplitSlots * kSplitSlotBytes));
  } else {
    w.h = reinterpret_cast<float*>(take((size_t)R[0] * inter[0] * sizeof(float)));
  }
  w.bytes = off;
  return w;
}

// Workspace of one expert set's moe_expert_ffn call.
inline size_t ffn_need(int T, int R, int d, int inter, int fmt) {
  return ffn_ws_layout(nullptr, T, d, 1, &R, &inter, fmt != MOE_W_FP32).bytes;
}

// Whether moe_forward runs the shared expert inside the routed experts' launches.
inline bool layer_fused(const moe_layer* L) {
  return L->shared.n_experts > 0 && L->shared.fmt == L->experts.fmt &&
         L->shared.layout == L->experts.layout && L->experts.fmt != MOE_W_FP32;
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

inline FwdWs fwd_layout(void* base, const moe_layer* L, int T) {
  FwdWs f{};
  const int E = L->experts.n_experts, d = L->experts.d, k = L->k;
  const int R = T * k;
  const bool has_sh = L->shared.n_experts > 0;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t n) {
    char* p = b ? b + off : nullptr;
    off = align_up(off + n, 256);
    return p;
  };
  f.partial = reinterpret_cast<float*>(take(route_ws_bytes(T, d, E)));
  f.idx = reinterpret_cast<int32_t*>(take((size_t)R * 4));
  f.w = reinterpret_cast<float*>(take((size_t)R * 4));
  f.offsets = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
  f.row_token = reinterpret_cast<int32_t*>(take((size_t)R * 4));
  f.token_row = reinterpret_cast<int32_t*>(take((size_t)R * 4));
  f.rows = reinterpret_cast<float*>(take((size_t)R * d * 4));
  f.sh_rows = has_sh ? reinterpret_cast<float*>(take((size_t)T * d * 4)) : nullptr;
  size_t ffn;
  if (layer_fused(L)) {
    int Rs[2] = {R, T}, Is[2] = {L->experts.inter, L->shared.inter};
    ffn = ffn_ws_layout(nullptr, T, d, 2, Rs, Is, true).bytes;
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

}  // namespace moe
