// Router: logits, selection and weights for every token.
//
// Sigmoid router (Kimi-Linear LiteRT-LM DETAILS.md, Conversion notes, the
// mixture-of-experts bullet): s = sigmoid(l), top k on s + bias, weights
// s / sum(s) times a scale (2.446).  Softmax router (Qwen3-30B-A3B LiteRT card,
// Conversion Notes): p = softmax(l), top k on p, weights p / sum(p).
//
// Two kernels.  The first writes partial logits, each a sum over a fixed
// 256-wide slice of the input in ascending order; the second adds the slices
// in order, so a token's logits never depend on T or on the launch shape.
// The second kernel runs one wavefront per token: k rounds of a 64-bit
// wavefront arg-max over order-preserving keys (fp32 key bits, then the
// inverted expert id, so ties go to the lower id).
#include "internal.h"

namespace moe {
namespace {

constexpr int kSub = 64;  // inputs staged in LDS per step

// partial[c][t][e] = sum over i in [256c, 256c + 256) of Wr[e][i] * x[t][i].
// Block: 256 threads as a 16 x 16 grid, each thread PE x PT outputs.
template <int TE, int TT>
__global__ __launch_bounds__(256) void router_logits_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            int T, int d, int E,
                                                            float* __restrict__ partial) {
  constexpr int PE = TE / 16, PT = TT / 16;
  __shared__ float ws[TE][kSub + 1];
  __shared__ float xs[TT][kSub + 1];
  const int e0 = blockIdx.x * TE, t0 = blockIdx.y * TT, c = blockIdx.z;
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
  float acc[PE][PT];
#pragma unroll
  for (int a = 0; a < PE; ++a)
#pragma unroll
    for (int b = 0; b < PT; ++b) acc[a][b] = 0.0f;

  const int kbeg = c * kRouterChunk;
  const int kend = min(d, kbeg + kRouterChunk);
  for (int k0 = kbeg; k0 < kend; k0 += kSub) {
    for (int q = threadIdx.x; q < TE * (kSub / 4); q += 256) {
      const int r = q / (kSub / 4), c4 = q % (kSub / 4);
      const int e = e0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < E) v = *reinterpret_cast<const float4*>(wr + (size_t)e * d + k0 + 4 * c4);
      ws[r][4 * c4 + 0] = v.x;
      ws[r][4 * c4 + 1] = v.y;
      ws[r][4 * c4 + 2] = v.z;
      ws[r][4 * c4 + 3] = v.w;
    }
    for (int q = threadIdx.x; q < TT * (kSub / 4); q += 256) {
      const int r = q / (kSub / 4), c4 = q % (kSub / 4);
      const int t = t0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < T) v = *reinterpret_cast<const float4*>(x + (size_t)t * d + k0 + 4 * c4);
      xs[r][4 * c4 + 0] = v.x;
      xs[r][4 * c4 + 1] = v.y;
      xs[r][4 * c4 + 2] = v.z;
      xs[r][4 * c4 + 3] = v.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kSub; ++kk) {
      float wv[PE], xv[PT];
#pragma unroll
      for (int a = 0; a < PE; ++a) wv[a] = ws[ti + 16 * a][kk];
#pragma unroll
      for (int b = 0; b < PT; ++b) xv[b] = xs[tj + 16 * b][kk];
#pragma unroll
      for (int a = 0; a < PE; ++a)
#pragma unroll
        for (int b = 0; b < PT; ++b) acc[a][b] = fmaf(wv[a], xv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < PE; ++a)
#pragma unroll
    for (int b = 0; b < PT; ++b) {
      const int e = e0 + ti + 16 * a, t = t0 + tj + 16 * b;
      if (e < E && t < T) partial[((size_t)c * T + t) * E + e] = acc[a][b];
    }
}

__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)(v & 0xffffffffu), o, kWave);
    const unsigned hi = __shfl_xor((unsigned)(v >> 32), o, kWave);
    const unsigned long long u = ((unsigned long long)hi << 32) | lo;
    v = u > v ? u : v;
  }
  return v;
}

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// fp32 bits mapped so that unsigned order equals float order.
__device__ inline unsigned ordered_bits(float f) {
  const unsigned b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One wavefront per token; NPL experts per lane (e = lane + 64 m).
template <int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ partial,
                                                          int nchunk,
                                                          const float* __restrict__ bias,
                                                          int T, int E, int k, int router,
                                                          float scale, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;

  float score[NPL];
  unsigned long long key[NPL];
#pragma unroll
  for (int m = 0; m < NPL; ++m) {
    const int e = lane + kWave * m;
    float l = 0.0f;
    if (e < E) {
      for (int c = 0; c < nchunk; ++c) l += partial[((size_t)c * T + t) * E + e];
    }
    score[m] = l;
  }
  if (router == 0) {  // sigmoid + selection bias
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
      const int e = lane + kWave * m;
      const float s = 1.0f / (1.0f + expf(-score[m]));
      score[m] = s;
      const float kap = s + (bias ? bias[e < E ? e : 0] : 0.0f);
      key[m] = e < E ? ((unsigned long long)ordered_bits(kap) << 32) | (0xffffffffu - (unsigned)e)
                     : 0ull;
    }
  } else {  // softmax over all E
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < NPL; ++m)
      if (lane + kWave * m < E) mx = fmaxf(mx, score[m]);
    mx = wave_max_f(mx);
    float z = 0.0f;
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
      const int e = lane + kWave * m;
      const float p = e < E ? expf(score[m] - mx) : 0.0f;
      score[m] = p;
      z += p;
    }
    z = wave_sum_f(z);
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
      const int e = lane + kWave * m;
      const float p = score[m] / z;
      score[m] = p;
      key[m] = e < E ? ((unsigned long long)ordered_bits(p) << 32) | (0xffffffffu - (unsigned)e)
                     : 0ull;
    }
  }

  float sel_s[kMaxK];
  int sel_e[kMaxK];
  float denom = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    sel_s[j] = 0.0f;
    sel_e[j] = 0;
    if (j < k) {
      unsigned long long best = 0ull;
#pragma unroll
      for (int m = 0; m < NPL; ++m) best = key[m] > best ? key[m] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xffffffffu - (unsigned)(best & 0xffffffffu));
      const int owner = e & (kWave - 1), mm = e / kWave;
      float s_own = 0.0f;
#pragma unroll
      for (int m = 0; m < NPL; ++m)
        if (lane == owner && m == mm) {
          s_own = score[m];
          key[m] = 0ull;
        }
      const float s = __shfl(s_own, owner, kWave);
      sel_s[j] = s;
      sel_e[j] = e;
      denom += s;
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k && lane == j) {
      idx[(size_t)t * k + j] = sel_e[j];
      w[(size_t)t * k + j] = scale * (sel_s[j] / denom);
    }
}

template <int NPL>
hipError_t launch_topk(const float* partial, int nchunk, const float* bias, int T, int E, int k,
                       int router, float scale, int32_t* idx, float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(router_topk_kernel<NPL>, grid, dim3(256), 0, s, partial, nchunk, bias, T,
                     E, k, router, scale, idx, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(int router, const float* x, const float* wr, const float* bias, int T,
                         int d, int E, int k, float scale, int32_t* idx, float* w,
                         float* partial, hipStream_t s) {
  const int nchunk = (d + kRouterChunk - 1) / kRouterChunk;
  if (T <= 32) {
    dim3 grid((E + 15) / 16, (T + 15) / 16, nchunk);
    hipLaunchKernelGGL((router_logits_kernel<16, 16>), grid, dim3(256), 0, s, x, wr, T, d, E,
                       partial);
  } else {
    dim3 grid((E + 63) / 64, (T + 63) / 64, nchunk);
    hipLaunchKernelGGL((router_logits_kernel<64, 64>), grid, dim3(256), 0, s, x, wr, T, d, E,
                       partial);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int npl = (E + kWave - 1) / kWave;
  if (npl <= 1) return launch_topk<1>(partial, nchunk, bias, T, E, k, router, scale, idx, w, s);
  if (npl <= 2) return launch_topk<2>(partial, nchunk, bias, T, E, k, router, scale, idx, w, s);
  if (npl <= 4) return launch_topk<4>(partial, nchunk, bias, T, E, k, router, scale, idx, w, s);
  if (npl <= 8) return launch_topk<8>(partial, nchunk, bias, T, E, k, router, scale, idx, w, s);
  return launch_topk<16>(partial, nchunk, bias, T, E, k, router, scale, idx, w, s);
}

}  // namespace moe
