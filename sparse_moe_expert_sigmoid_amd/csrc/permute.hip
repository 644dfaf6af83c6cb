// Grouping of the T*k (token, slot) pairs by expert: a counting sort that is
// stable in (t, j) order.  Only the routed experts are computed for each
// token (Qwen3-30B-A3B LiteRT card, Conversion Notes), so each expert gets a
// contiguous run of rows holding exactly the tokens that chose it.
//
// One workgroup of W wavefronts.  The flat pair list is cut into W equal
// segments, one per wavefront:
//   1. per-wavefront histograms in LDS (integer atomics, order-free);
//   2. offsets = exclusive scan over experts, and each wavefront's base row
//      per expert = offsets[e] + counts of the lower segments;
//   3. each wavefront walks its segment 64 pairs at a time: a 64-bit mask per
//      expert (LDS atomic OR) gives each pair's rank among equal experts of
//      the lower lanes, so the scatter is stable without any sort.
// Every result is a pure function of the input (no order-dependent atomics).
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ idx, int n,
                                                       int k, int E, int seg,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ row_token,
                                                       int32_t* __restrict__ token_row) {
  extern __shared__ unsigned long long smem_u64[];
  const int W = blockDim.x / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  unsigned long long* masks = smem_u64;                        // [W][E]
  int* base = reinterpret_cast<int*>(masks + (size_t)W * E);   // [W][E]
  int* cnt = base + (size_t)W * E;                             // [E]

  for (int i = threadIdx.x; i < W * E; i += blockDim.x) base[i] = 0;
  __syncthreads();

  const int s0 = wave * seg;
  const int s1 = min(n, s0 + seg);
  for (int i = s0 + lane; i < s1; i += kWave) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&base[wave * E + e], 1);
  }
  __syncthreads();

  // per expert: exclusive prefix over wavefronts, total in cnt[e]
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int v = 0; v < W; ++v) {
      const int c = base[v * E + e];
      base[v * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();

  // exclusive scan of cnt over experts by wavefront 0, 64 experts per step
  if (wave == 0) {
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += kWave) {
      const int e = c0 + lane;
      const int v = e < E ? cnt[e] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
      }
      if (e < E) {
        offsets[e] = carry + incl - v;
        cnt[e] = carry + incl - v;  // reuse: first row of expert e
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) offsets[E] = carry;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < W * E; i += blockDim.x) base[i] += cnt[i % E];
  __syncthreads();

  // stable scatter; every wavefront runs the same number of steps (barriers)
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  unsigned long long* my_masks = masks + (size_t)wave * E;
  int* my_base = base + (size_t)wave * E;
  for (int c0 = 0; c0 < seg; c0 += kWave) {
    const int i = s0 + c0 + lane;
    const bool valid = (c0 + lane < seg) && i < s1;
    const int e = valid ? idx[i] : -1;
    const bool ok = valid && e >= 0 && e < E;
    if (ok) my_masks[e] = 0ull;
    __syncthreads();
    if (ok) atomicOr(&my_masks[e], 1ull << lane);
    __syncthreads();
    unsigned long long m = 0ull;
    int rank = 0;
    if (ok) {
      m = my_masks[e];
      rank = __popcll(m & below);
      const int pos = my_base[e] + rank;
      row_token[pos] = i / k;
      token_row[i] = pos;
    } else if (valid) {
      token_row[i] = -1;
    }
    __syncthreads();
    if (ok && rank == 0) my_base[e] += __popcll(m);
    __syncthreads();
  }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimedLaunch tl(K_FILL, s);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// Routing statistics: per-expert counts of the selections, accumulated into a
// 64-bit histogram (integer atomics, so the totals do not depend on order).
__global__ __launch_bounds__(256) void expert_counts_kernel(const int32_t* __restrict__ idx,
                                                            long long n, int E,
                                                            unsigned long long* counts) {
  extern __shared__ unsigned int hist_u32[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist_u32[e] = 0u;
  __syncthreads();
  for (long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (long long)gridDim.x * blockDim.x) {
    const int e = idx[q];
    if (e >= 0 && e < E) atomicAdd(&hist_u32[e], 1u);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (hist_u32[e]) atomicAdd(&counts[e], (unsigned long long)hist_u32[e]);
}

hipError_t launch_expert_counts(const int32_t* idx, long long n, int E,
                                unsigned long long* counts, hipStream_t s) {
  long long blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(expert_counts_kernel, dim3((unsigned)blocks), dim3(256),
                     (size_t)E * sizeof(unsigned int), s, idx, n, E, counts);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* row_token, int32_t* token_row, hipStream_t s) {
  const long long n = (long long)T * k;
  // LDS per wavefront: E masks (8 B) + E bases (4 B); plus E counts.
  const size_t per_wave = (size_t)E * 12;
  int W = (int)((150 * 1024 - (size_t)E * 4) / per_wave);
  W = W > 16 ? 16 : W;
  if (W < 1) W = 1;
  const int nw_needed = (int)((n + kWave - 1) / kWave);
  if (W > nw_needed) W = nw_needed > 0 ? nw_needed : 1;
  int seg = (int)((n + W - 1) / W);
  seg = (seg + kWave - 1) / kWave * kWave;
  const size_t lds = (size_t)W * E * 12 + (size_t)E * 4;
  TimedLaunch tl(K_PERMUTE, s);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(W * kWave), lds, s, idx, (int)n, k, E, seg,
                     offsets, row_token, token_row);
  return hipGetLastError();
}

}  // namespace moe
