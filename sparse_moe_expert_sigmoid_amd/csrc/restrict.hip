// Expert restriction: the kept expert set from recorded selection counts
// (Kimi-Linear-48B-A3B-Code-CMF listing, "How it was made", step 3: per layer,
// the smallest set of experts that carries a given share of the selections).
//
// Taking experts by descending count, equal counts by ascending id, the first
// n whose running sum reaches cover * total form a smallest such set; it is
// padded in the same order to min(k, E) experts so that a token can still
// select k.  One workgroup does it all (E <= 1024):
//   1. rank of each expert in that order, by counting the experts before it;
//   2. counts placed in rank order, inclusive running sums (uint64, exact);
//   3. n = the first rank whose running sum, as a double, reaches
//      cover * (double) total (0 when that product is 0), then max(n, min(k, E));
//   4. kept = rank < n, written as ascending ids by counting the kept experts
//      of lower id.
// The pages fix no precision for the share; it is compared in double
// precision, so that the same product and the same conversions give the same
// set on any implementation.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kMaxE) void coverage_set_kernel(
    const unsigned long long* __restrict__ counts, int E, double cover, int k,
    int32_t* __restrict__ keep, int32_t* __restrict__ n_keep) {
  __shared__ unsigned long long c_sm[kMaxE];
  __shared__ unsigned long long run[2][kMaxE];
  __shared__ int rank_sm[kMaxE];
  __shared__ int n_sm;
  const int t = threadIdx.x;
  const bool live = t < E;
  const unsigned long long c = live ? counts[t] : 0ull;
  if (live) c_sm[t] = c;
  if (t == 0) n_sm = E;
  __syncthreads();

  int rank = 0;
  if (live) {
    for (int j = 0; j < E; ++j) {
      const unsigned long long cj = c_sm[j];
      rank += (cj > c) || (cj == c && j < t);
    }
    rank_sm[t] = rank;
    run[0][rank] = c;
  }
  __syncthreads();
  int cur = 0;
  for (int off = 1; off < E; off <<= 1) {  // uniform trip count: every thread reaches the barrier
    if (live) run[cur ^ 1][t] = run[cur][t] + (t >= off ? run[cur][t - off] : 0ull);
    cur ^= 1;
    __syncthreads();
  }
  const double need = cover * (double)run[cur][E - 1];
  if (!(need > 0.0)) {
    if (t == 0) n_sm = 0;
  } else if (live) {
    const bool reached = (double)run[cur][t] >= need;
    const bool before = t == 0 || (double)run[cur][t - 1] < need;
    if (reached && before) n_sm = t + 1;  // one thread: the sums are non-decreasing
  }
  __syncthreads();
  const int n = max(n_sm, min(k, E));
  if (live) {
    if (rank < n) {
      int pos = 0;
      for (int j = 0; j < t; ++j) pos += rank_sm[j] < n;
      keep[pos] = t;
    }
    if (t >= n) keep[t] = -1;
  }
  if (t == 0) n_keep[0] = n;
}

}  // namespace

hipError_t launch_coverage_set(const unsigned long long* counts, int E, double cover, int k,
                               int32_t* keep, int32_t* n_keep, hipStream_t s) {
  const int threads = (E + 63) / 64 * 64;
  moe_launch(coverage_set_kernel, dim3(1), dim3(threads), 0, s, counts, E, cover, k,
                     keep, n_keep);
  return hipGetLastError();
}

}  // namespace moe
