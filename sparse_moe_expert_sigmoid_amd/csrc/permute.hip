// Grouping of the T*k (token, slot) pairs by expert: a counting sort that is
// stable in (t, j) order.  Only the routed experts are computed for each
// token (Qwen3-30B-A3B LiteRT card, Conversion Notes), so each expert gets a
// contiguous run of rows holding exactly the tokens that chose it.
//
// The flat pair list is cut into chunks, one per workgroup of W wavefronts,
// and each chunk into W segments of `seg` pairs, one per wavefront.  A
// workgroup needs no other workgroup's results:
//   1. it reads every pair (the whole list is a few hundred KB, L2-resident)
//      and counts in LDS, per expert, the pairs before its chunk, the pairs
//      after it, and each wavefront's pairs inside it (integer atomics,
//      order-free);
//   2. offsets = exclusive scan over experts of the totals (the first
//      workgroup writes them), and each wavefront's base row per expert =
//      offsets[e] + pairs of e before the chunk + those of the lower segments;
//   3. each wavefront walks its segment 64 pairs at a time: a 64-bit mask per
//      expert (LDS atomic OR) gives each pair's rank among equal experts of
//      the lower lanes, so the scatter is stable without any sort.
// Every result is a pure function of the input (no order-dependent atomics),
// the same for every chunking.
#include "internal.h"

namespace moe {
namespace {

constexpr int kCountBatch = 16;  // pair loads in flight per thread while counting

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
  int* below = cnt + E;                                        // [E]
  const long long c0 = (long long)blockIdx.x * W * seg;        // this chunk: [c0, c1)
  const long long c1 = min((long long)n, c0 + (long long)W * seg);

  for (int i = threadIdx.x; i < W * E; i += blockDim.x) base[i] = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = below[e] = 0;
  __syncthreads();

  // 1. counts: below[e] before the chunk, cnt[e] after it, base[w][e] inside
  // (loads issued a batch at a time from clamped indices, then counted)
  for (long long i0 = 0; i0 < n; i0 += kCountBatch * (long long)blockDim.x) {
    int ev[kCountBatch];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const long long i = i0 + u * (long long)blockDim.x + threadIdx.x;
      ev[u] = idx[i < n ? i : n - 1];
    }
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const long long i = i0 + u * (long long)blockDim.x + threadIdx.x;
      const int e = ev[u];
      if (i >= n || e < 0 || e >= E) continue;
      if (i < c0) atomicAdd(&below[e], 1);
      else if (i >= c1) atomicAdd(&cnt[e], 1);
      else atomicAdd(&base[(int)((i - c0) / seg) * E + e], 1);
    }
  }
  __syncthreads();

  // per expert: each wavefront's first row relative to the expert's first
  // row, and the expert's total in cnt[e]
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = below[e];
    for (int v = 0; v < W; ++v) {
      const int c = base[v * E + e];
      base[v * E + e] = run;
      run += c;
    }
    cnt[e] += run;
  }
  __syncthreads();

  // 2. exclusive scan of the totals over experts by wavefront 0, 64 experts
  // per step
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int v = e < E ? cnt[e] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
      }
      if (e < E) {
        if (blockIdx.x == 0) offsets[e] = carry + incl - v;
        cnt[e] = carry + incl - v;  // reuse: first row of expert e
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0 && blockIdx.x == 0) offsets[E] = carry;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < W * E; i += blockDim.x) base[i] += cnt[i % E];
  __syncthreads();

  // 3. stable scatter; every wavefront runs the same number of steps (barriers)
  const unsigned long long below_lanes = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  unsigned long long* my_masks = masks + (size_t)wave * E;
  int* my_base = base + (size_t)wave * E;
  const long long s0 = c0 + (long long)wave * seg;
  const long long s1 = min(c1, s0 + seg);
  for (int j0 = 0; j0 < seg; j0 += kWave) {
    const long long i = s0 + j0 + lane;
    const bool valid = i < s1;
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
      rank = __popcll(m & below_lanes);
      const int pos = my_base[e] + rank;
      row_token[pos] = (int)(i / k);
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
  moe_launch(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
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
  moe_launch(expert_counts_kernel, dim3((unsigned)blocks), dim3(256),
                     (size_t)E * sizeof(unsigned int), s, idx, n, E, counts);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* row_token, int32_t* token_row, hipStream_t s) {
  const long long n = (long long)T * k;
  if (n <= 0) return hipSuccess;
  // LDS per wavefront: E masks (8 B) + E bases (4 B); plus E counts twice.
  const size_t per_wave = (size_t)E * 12;
  int W = (int)((150 * 1024 - (size_t)E * 8) / per_wave);
  W = W > 16 ? 16 : W;
  if (W < 1) W = 1;
  const long long nw_needed = (n + kWave - 1) / kWave;
  if (W > nw_needed) W = (int)nw_needed;
  // one 64-pair step per wavefront while that needs at most kMaxChunks
  // workgroups (each reads the whole list), longer segments beyond
  constexpr long long kMaxChunks = 512;
  long long steps = (n + (long long)W * kWave * kMaxChunks - 1) / ((long long)W * kWave * kMaxChunks);
  if (steps < 1) steps = 1;
  const int seg = (int)(steps * kWave);
  const long long chunks = (n + (long long)W * seg - 1) / ((long long)W * seg);
  const size_t lds = (size_t)W * E * 12 + (size_t)E * 8;
  TimedLaunch tl(K_PERMUTE, s);
  moe_launch(permute_kernel, dim3((unsigned)chunks), dim3(W * kWave), lds, s, idx,
                     (int)n, k, E, seg, offsets, row_token, token_row);
  return hipGetLastError();
}

}  // namespace moe
