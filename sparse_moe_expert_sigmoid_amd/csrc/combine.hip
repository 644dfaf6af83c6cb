// Weighted combine: y[t] = sum_j w[t][j] * rows[token_row[t*k + j]]
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
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int r = token_row[(size_t)t * k + j];
    if (r < 0) continue;
    const float wj = w[(size_t)t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(rows + (size_t)r * d + 4 * c);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  const size_t o = (size_t)t * d + 4 * c;
  if (shared) {
    const float4 v = *reinterpret_cast<const float4*>(shared + o);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (residual) {
    const float4 v = *reinterpret_cast<const float4*>(residual + o);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *reinterpret_cast<float4*>(y + o) = acc;
}

}  // namespace

hipError_t launch_combine(const float* rows, const int32_t* token_row, const float* w,
                          const float* shared, const float* residual, int T, int k, int d,
                          float* y, hipStream_t s) {
  const long long n = (long long)T * (d / 4);
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, rows, token_row, w, shared,
                     residual, T, k, d, y);
  return hipGetLastError();
}

}  // namespace moe
