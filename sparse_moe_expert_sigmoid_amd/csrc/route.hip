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
// The second kernel runs one workgroup per token and ranks the selection keys
// by counting (no sequential arg-max rounds).
#include "internal.h"

namespace moe {
namespace {

// partial[c][t][e] = sum over i in [256c, 256c + 256) of Wr[e][i] * x[t][i],
// one fmaf chain per output in ascending i (the same chain in every variant).
// Block: 256 threads as a 16 x 16 grid, each thread PE x PT outputs; kSub
// inputs are staged in LDS per step (the whole 256-chunk for the small tile,
// so a decode launch makes one trip to memory).
template <int TE, int TT, int kSub>
__global__ __launch_bounds__(256) void router_logits_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            int T, int d, int E,
                                                            float* __restrict__ partial) {
  constexpr int PE = TE / 16, PT = TT / 16;
  constexpr int kLd = kSub + 4;  // row stride: 16-byte aligned, rows 4 banks apart
  __shared__ __attribute__((aligned(16))) float ws[TE][kLd];
  __shared__ __attribute__((aligned(16))) float xs[TT][kLd];
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
    const int kn = min(kSub, kend - k0);  // the last slice of a row can be short
    for (int q = threadIdx.x; q < TE * (kSub / 4); q += 256) {
      const int r = q / (kSub / 4), c4 = q % (kSub / 4);
      const int e = e0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < E && 4 * c4 < kn)
        v = *reinterpret_cast<const float4*>(wr + (size_t)e * d + k0 + 4 * c4);
      *reinterpret_cast<float4*>(&ws[r][4 * c4]) = v;
    }
    for (int q = threadIdx.x; q < TT * (kSub / 4); q += 256) {
      const int r = q / (kSub / 4), c4 = q % (kSub / 4);
      const int t = t0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < T && 4 * c4 < kn)
        v = *reinterpret_cast<const float4*>(x + (size_t)t * d + k0 + 4 * c4);
      *reinterpret_cast<float4*>(&xs[r][4 * c4]) = v;
    }
    __syncthreads();
    // four inputs per LDS read; the fmaf chain still runs in ascending i
#pragma unroll 2
    for (int kk = 0; kk < kn; kk += 4) {
      float4 wv[PE], xv[PT];
#pragma unroll
      for (int a = 0; a < PE; ++a) wv[a] = *reinterpret_cast<const float4*>(&ws[ti + 16 * a][kk]);
#pragma unroll
      for (int b = 0; b < PT; ++b) xv[b] = *reinterpret_cast<const float4*>(&xs[tj + 16 * b][kk]);
#pragma unroll
      for (int a = 0; a < PE; ++a)
#pragma unroll
        for (int b = 0; b < PT; ++b) {
          acc[a][b] = fmaf(wv[a].x, xv[b].x, acc[a][b]);
          acc[a][b] = fmaf(wv[a].y, xv[b].y, acc[a][b]);
          acc[a][b] = fmaf(wv[a].z, xv[b].z, acc[a][b]);
          acc[a][b] = fmaf(wv[a].w, xv[b].w, acc[a][b]);
        }
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

// Selection for one token by a group of 256 threads (gtid = thread in the
// group; every group of the workgroup calls this in step, also for tokens past
// T with active = false, because it contains workgroup barriers).  Each thread
// owns EPT experts (e = gtid + 256 m): it adds the logit slices in order, forms
// the score and the selection key (fp32 bits made order-preserving, then the
// inverted expert id, so ties go to the lower id), and counts how many keys in
// LDS beat its own; a rank below k is the expert's output slot.  Weights are
// scale * s_j / sum_j s_j with the sum taken in slot order.
template <int EPT>
__device__ inline void select_token(const float* __restrict__ partial, int nchunk,
                                    const float* __restrict__ bias,
                                    const uint8_t* __restrict__ mask, int T, int E, int k,
                                    int router, float scale, int t, bool active, int gtid,
                                    unsigned long long* keys, float* red, float* sel_s,
                                    int32_t* __restrict__ idx, float* __restrict__ w,
                                    int* idx_lds) {
  const int lane = gtid & (kWave - 1), wave = gtid / kWave;
  float sc[EPT];
  unsigned long long key[EPT];
  float bv[EPT];
  bool ok[EPT];  // allowed by the expert mask (and inside E)
  // Every load of the selection is issued here and unconditionally, so that
  // one wait covers them all (a load under a condition makes the compiler
  // wait for every load in flight, the caller's early x loads included):
  // expert indices clamped into [0, E), slices clamped into [0, nchunk), and
  // an absent bias or mask read from a valid stand-in whose value is dropped.
  constexpr int kMaxChunks = 16;
  const float* bsrc = bias ? bias : partial;
  const uint8_t* msrc = mask ? mask : reinterpret_cast<const uint8_t*>(partial);
  float braw[EPT], pv[EPT][kMaxChunks];
  uint8_t mraw[EPT];
  const bool fast = nchunk <= kMaxChunks;
#pragma unroll
  for (int m = 0; m < EPT; ++m) {
    const int e = gtid + 256 * m;
    const int ec = e < E ? e : E - 1;
    braw[m] = bsrc[ec];
    mraw[m] = msrc[ec];
    if (fast) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        pv[m][c] = partial[((size_t)(c < nchunk ? c : nchunk - 1) * T + t) * E + ec];
    }
  }
#pragma unroll
  for (int m = 0; m < EPT; ++m) {
    const int e = gtid + 256 * m;
    bv[m] = (bias && e < E) ? braw[m] : 0.0f;
    ok[m] = e < E && (mask == nullptr || mraw[m] != 0);
  }
  // the slices added in ascending order
#pragma unroll
  for (int m = 0; m < EPT; ++m) {
    const int e = gtid + 256 * m;
    float l = 0.0f;
    if (fast) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (c < nchunk) l += pv[m][c];
    } else if (active && e < E) {
      for (int c = 0; c < nchunk; ++c) l += partial[((size_t)c * T + t) * E + e];
    }
    sc[m] = l;
  }
  if (router == 0) {
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
      const int e = gtid + 256 * m;
      const float s = 1.0f / (1.0f + expf(-sc[m]));
      sc[m] = ok[m] ? s : 0.0f;
      const float kap = s + bv[m];
      // A masked expert's key has a zero high word, below every real key (the
      // ordered bits of a non-NaN float are nonzero), and stays distinct by id.
      key[m] = ((unsigned long long)(ok[m] ? ordered_bits(kap) : 0u) << 32) |
               (0xffffffffu - (unsigned)e);
    }
  } else {
    // the softmax runs over the allowed experts only (masked logits removed)
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < EPT; ++m)
      if (ok[m]) mx = fmaxf(mx, sc[m]);
    mx = wave_max_f(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float z = 0.0f;
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
      const float p = ok[m] ? expf(sc[m] - mx) : 0.0f;
      sc[m] = p;
      z += p;
    }
    z = wave_sum_f(z);
    if (lane == 0) red[wave] = z;
    __syncthreads();
    z = (red[0] + red[1]) + (red[2] + red[3]);
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
      const int e = gtid + 256 * m;
      const float p = sc[m] / z;
      sc[m] = p;
      key[m] = ((unsigned long long)(ok[m] ? ordered_bits(p) : 0u) << 32) |
               (0xffffffffu - (unsigned)e);
    }
  }
#pragma unroll
  for (int m = 0; m < EPT; ++m) keys[gtid + 256 * m] = gtid + 256 * m < E ? key[m] : 0ull;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < EPT; ++m) {
    const int e = gtid + 256 * m;
    if (!active || e >= E) continue;
    int rank = 0;
#pragma unroll 16
    for (int q = 0; q < E; ++q) rank += keys[q] > key[m] ? 1 : 0;
    if (rank < k) {
      idx[(size_t)t * k + rank] = e;
      if (idx_lds) idx_lds[t * k + rank] = e;
      sel_s[rank] = sc[m];
    }
  }
  __syncthreads();
  if (active && gtid < k) {
    float denom = 0.0f;
    for (int j = 0; j < k; ++j) denom += sel_s[j];
    w[(size_t)t * k + gtid] = scale * (sel_s[gtid] / denom);
  }
}

// One workgroup per token.
template <int EPT>
__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ partial,
                                                            int nchunk,
                                                            const float* __restrict__ bias,
                                                            const uint8_t* __restrict__ mask,
                                                            int T, int E, int k, int router,
                                                            float scale,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ w) {
  __shared__ unsigned long long keys[256 * EPT];
  __shared__ float red[4];
  __shared__ float sel_s[kMaxK];
  select_token<EPT>(partial, nchunk, bias, mask, T, E, k, router, scale, blockIdx.x, true,
                    threadIdx.x,
                    keys, red, sel_s, idx, w, nullptr);
}

template <int EPT>
hipError_t launch_select(const float* partial, int nchunk, const float* bias,
                         const uint8_t* mask, int T, int E, int k,
                         int router, float scale, int32_t* idx, float* w, hipStream_t s) {
  TimedLaunch tl(K_ROUTER_TOPK, s);
  hipLaunchKernelGGL(router_select_kernel<EPT>, dim3(T), dim3(256), 0, s, partial, nchunk, bias,
                     mask,
                     T, E, k, router, scale, idx, w);
  return hipGetLastError();
}

// ------------------------------------------------------------------ small T: fused tail
// After the logits kernel, one workgroup per token selects that token's
// experts (select_token) and encodes its row of x as two-digit int8 for the
// FFN kernels, which then group the (token, slot) pairs themselves.
template <int EPT>
__global__ __launch_bounds__(256) void router_tail_kernel(
    const float* __restrict__ partial, int nchunk, const float* __restrict__ x, int d,
    const float* __restrict__ bias, const uint8_t* __restrict__ mask, int T, int E, int k,
    int router, float scale,
    int32_t* __restrict__ idx, float* __restrict__ w, int8_t* __restrict__ xq,
    float* __restrict__ xs, bool perm, int* __restrict__ split_cnt) {
  __shared__ unsigned long long keys[256 * EPT];
  if (split_cnt)  // the FFN launches that follow start from zero counters
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < kSplitSlots; q += gridDim.x * blockDim.x)
      split_cnt[q] = 0;
  __shared__ float red[4];
  __shared__ float xred[4];
  __shared__ float sel_s[kMaxK];
  const int t = blockIdx.x;
  const float* row = x + (size_t)t * d;
  // the token's row of x (up to 4096 values, in groups of 8 per thread) goes
  // into registers first, so its loads are in flight during the selection
  constexpr int kXPer = 2;
  const int n8 = d / 8;
  const bool in_regs = n8 <= kXPer * 256;
  float4 xv[kXPer][2];
#pragma unroll
  for (int m = 0; m < kXPer; ++m) {
    const int c = threadIdx.x + 256 * m;
    const bool ok = in_regs && c < n8;
    xv[m][0] = ok ? *reinterpret_cast<const float4*>(row + 8 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    xv[m][1] = ok ? *reinterpret_cast<const float4*>(row + 8 * c + 4)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  select_token<EPT>(partial, nchunk, bias, mask, T, E, k, router, scale, t, true, threadIdx.x,
                    keys,
                    red, sel_s, idx, w, nullptr);
  if (!in_regs) {
    if (threadIdx.x < kWave) encode_row(row, d, xq + (size_t)t * 2 * d, xs + t, perm);
    return;
  }
  // two-digit encoding of the row with one scale (as encode_row), by all threads
  float mx = 0.0f;
#pragma unroll
  for (int m = 0; m < kXPer; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[m][h].x), fabsf(xv[m][h].y)),
                           fmaxf(fabsf(xv[m][h].z), fabsf(xv[m][h].w))));
  mx = wave_max_f(mx);
  if ((threadIdx.x & (kWave - 1)) == 0) xred[threadIdx.x / kWave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(xred[0], xred[1]), fmaxf(xred[2], xred[3]));
  const int p = digit_exponent(mx);
  uint2* q0 = reinterpret_cast<uint2*>(xq + (size_t)t * 2 * d);
  uint2* q1 = reinterpret_cast<uint2*>(xq + (size_t)t * 2 * d + d);
#pragma unroll
  for (int m = 0; m < kXPer; ++m) {
    const int c = threadIdx.x + 256 * m;
    if (c >= n8) continue;
    uint2 w0, w1;
    encode8(xv[m][0], xv[m][1], p, perm, w0, w1);
    const int dst = perm ? int4_digit_chunk(c) : c;
    q0[dst] = w0;
    q1[dst] = w1;
  }
  if (threadIdx.x == 0) xs[t] = mx > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
}

template <int EPT>
hipError_t launch_tail(const float* partial, int nchunk, const float* x, int d, const float* bias,
                       const uint8_t* mask,
                       int T, int E, int k, int router, float scale, int32_t* idx, float* w,
                       int8_t* xq, float* xs, bool perm, int* split_cnt, hipStream_t s) {
  TimedLaunch tl(K_ROUTER_TAIL, s);
  hipLaunchKernelGGL(router_tail_kernel<EPT>, dim3(T), dim3(256), 0, s, partial, nchunk, x, d,
                     bias, mask, T, E, k, router, scale, idx, w, xq, xs, perm, split_cnt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(int router, const float* x, const float* wr, const float* bias,
                         const uint8_t* mask, int T,
                         int d, int E, int k, float scale, int32_t* idx, float* w,
                         float* partial, hipStream_t s) {
  const int nchunk = (d + kRouterChunk - 1) / kRouterChunk;
  {
  TimedLaunch tl(K_ROUTER_LOGITS, s);
  if (T <= 32) {
    dim3 grid((E + 15) / 16, (T + 15) / 16, nchunk);
    hipLaunchKernelGGL((router_logits_kernel<16, 16, 256>), grid, dim3(256), 0, s, x, wr, T, d,
                       E, partial);
  } else {
    dim3 grid((E + 63) / 64, (T + 63) / 64, nchunk);
    hipLaunchKernelGGL((router_logits_kernel<64, 64, 64>), grid, dim3(256), 0, s, x, wr, T, d,
                       E, partial);
  }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (E <= 256)
    return launch_select<1>(partial, nchunk, bias, mask, T, E, k, router, scale, idx, w, s);
  if (E <= 512)
    return launch_select<2>(partial, nchunk, bias, mask, T, E, k, router, scale, idx, w, s);
  return launch_select<4>(partial, nchunk, bias, mask, T, E, k, router, scale, idx, w, s);
}

hipError_t launch_router_small(int router, const float* x, const float* wr, const float* bias,
                               const uint8_t* mask,
                               int T, int d, int E, int k, float scale, int32_t* idx, float* w,
                               float* partial, int8_t* xq, float* xs, bool perm,
                               int* split_cnt, hipStream_t s) {
  const int nchunk = (d + kRouterChunk - 1) / kRouterChunk;
  {
    TimedLaunch tl(K_ROUTER_LOGITS, s);
    dim3 grid((E + 15) / 16, (T + 15) / 16, nchunk);
    hipLaunchKernelGGL((router_logits_kernel<16, 16, 256>), grid, dim3(256), 0, s, x, wr, T, d,
                       E, partial);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (E <= 256)
    return launch_tail<1>(partial, nchunk, x, d, bias, mask, T, E, k, router, scale, idx, w, xq,
                          xs, perm, split_cnt, s);
  if (E <= 512)
    return launch_tail<2>(partial, nchunk, x, d, bias, mask, T, E, k, router, scale, idx, w, xq,
                          xs, perm, split_cnt, s);
  return launch_tail<4>(partial, nchunk, x, d, bias, mask, T, E, k, router, scale, idx, w, xq,
                          xs, perm, split_cnt, s);
}

}  // namespace moe
