// Expert selection for one token, shared by the router's selection kernels
// (route.hip) and the one-token FFN launch that selects for itself (ffn.hip).
// Sigmoid router (Kimi-Linear LiteRT-LM DETAILS.md, Conversion notes, the
// mixture-of-experts bullet): s = sigmoid(l), top k on s + bias, weights
// s / sum(s) times a scale.  Softmax router (Qwen3-30B-A3B LiteRT card,
// Conversion Notes): p = softmax(l), top k on p, weights p / sum(p).
#pragma once
#include <hip/hip_runtime.h>

#include "internal.h"

namespace moe {

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
  // Top k in two rounds of rank counting (keys are distinct: the expert id
  // sits in the low word).  Only a key among the top k of its wavefront's
  // 64 EPT keys can be among the token's top k, and every key above a token
  // top-k key is such a candidate too, so ranking the 4 k candidates among
  // themselves gives the same ranks as ranking against all E keys, with
  // 64 EPT + 4 k comparisons per key instead of E.  Slots of wavefronts with
  // fewer than k keys stay 0, below every key.
  __shared__ unsigned long long cand[4 * kMaxK];
  __shared__ float cand_s[4 * kMaxK];
#pragma unroll
  for (int m = 0; m < EPT; ++m) keys[gtid + 256 * m] = gtid + 256 * m < E ? key[m] : 0ull;
  if (gtid < 4 * k) cand[gtid] = 0ull;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < EPT; ++m) {
    const int e = gtid + 256 * m;
    if (!active || e >= E) continue;
    int rank = 0;
#pragma unroll
    for (int mm = 0; mm < EPT; ++mm) {
      const unsigned long long* kw = keys + 256 * mm + kWave * wave;
#pragma unroll 16
      for (int q = 0; q < kWave; ++q) rank += kw[q] > key[m] ? 1 : 0;
    }
    if (rank < k) {
      cand[wave * k + rank] = key[m];
      cand_s[wave * k + rank] = sc[m];
    }
  }
  __syncthreads();
  if (active && gtid < 4 * k) {
    const unsigned long long c = cand[gtid];
    int rank = 0;
    for (int q = 0; q < 4 * k; ++q) rank += cand[q] > c ? 1 : 0;
    if (rank < k) {  // (an empty slot ranks below the k real candidates)
      const int e = (int)(0xffffffffu - (unsigned)(c & 0xffffffffull));
      idx[(size_t)t * k + rank] = e;
      if (idx_lds) idx_lds[t * k + rank] = e;
      sel_s[rank] = cand_s[gtid];
    }
  }
  __syncthreads();
  if (active && gtid < k) {
    float denom = 0.0f;
    for (int j = 0; j < k; ++j) denom += sel_s[j];
    w[(size_t)t * k + gtid] = scale * (sel_s[gtid] / denom);
  }
}

}  // namespace moe
