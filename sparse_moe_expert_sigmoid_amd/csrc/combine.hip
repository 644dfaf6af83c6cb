// Weighted combine: y[t] = sum_j w[t][j] * rows[token_row[t*k + j]]
// (token_row NULL: rows already in (token, slot) order, row t*k + j)
// (slot order) + shared[t] + residual[t].  The routed experts' outputs are
// weighted by the router weights and the shared expert is added with weight 1
// (Kimi-Linear LiteRT-LM DETAILS.md, Conversion notes, mixture-of-experts
// bullet); the residual add sits after the moe op (Qwen3-30B-A3B LiteRT card,
// Conversion Notes).
//
// HBM-bound gather: one thread per 4 consecutive outputs of a token, 16-byte
// loads of the k gathered rows; the k row indices and weights of a token are
// read once per thread and hit the cache.
#include "internal.h"

namespace moe {
namespace {

// KMAX >= k is a compile-time bound, so that every row load of a thread is
// issued before the first one is used: slots past k read a real row (the
// token's first) with weight 0.  Whether rows are found through
// token_row (TR) is a template parameter for the same reason: loads under a
// run-time condition would cost a round trip each.
template <int KMAX, bool TR>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ rows,
                                                      const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ shared,
                                                      const float* residual, int T, int k, int d,
                                                      float* y) {
  const int d4 = d / 4;
  const long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= (long long)T * d4) return;
  const int t = (int)(q / d4), c = (int)(q % d4);
  const size_t o = (size_t)t * d + 4 * c;
  // all loads are issued before any arithmetic: row ids and weights, then rows
  int r[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int jj = j < k ? j : 0;
    r[j] = TR ? token_row[(size_t)t * k + jj] : t * k + jj;
    const float wv = w[(size_t)t * k + jj];
    wj[j] = j < k ? wv : 0.0f;
  }
  const float4 sh = shared ? *reinterpret_cast<const float4*>(shared + o)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 rs = residual ? *reinterpret_cast<const float4*>(residual + o)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) v[j] = *reinterpret_cast<const float4*>(rows + (size_t)r[j] * d + 4 * c);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // slots in order; those past k add 0 * (a finite row value), which leaves
  // the sum unchanged, and keeps every load in front of the first use
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    acc.x = fmaf(wj[j], v[j].x, acc.x);
    acc.y = fmaf(wj[j], v[j].y, acc.y);
    acc.z = fmaf(wj[j], v[j].z, acc.z);
    acc.w = fmaf(wj[j], v[j].w, acc.w);
  }
  if (shared) {
    acc.x += sh.x; acc.y += sh.y; acc.z += sh.z; acc.w += sh.w;
  }
  if (residual) {
    acc.x += rs.x; acc.y += rs.y; acc.z += rs.z; acc.w += rs.w;
  }
  *reinterpret_cast<float4*>(y + o) = acc;
}

}  // namespace

hipError_t launch_combine(const float* rows, const int32_t* token_row, const float* w,
                          const float* shared, const float* residual, int T, int k, int d,
                          float* y, hipStream_t s) {
  const long long n = (long long)T * (d / 4);
  const int blocks = (int)((n + 255) / 256);
  TimedLaunch tl(K_COMBINE, s);
#define MOE_COMBINE(KM, TRV)                                                                   \
  moe_launch((combine_kernel<KM, TRV>), dim3(blocks), dim3(256), 0, s, rows, token_row, w, \
                     shared, residual, T, k, d, y)
  if (k <= 8) {
    if (token_row) MOE_COMBINE(8, true);
    else MOE_COMBINE(8, false);
  } else {
    if (token_row) MOE_COMBINE(kMaxK, true);
    else MOE_COMBINE(kMaxK, false);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
