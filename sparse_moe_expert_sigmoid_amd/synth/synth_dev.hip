// Device twin of the seeded input generator (synth.c beside this file).
//
// Same counter-based SplitMix64 draws, evaluated on the GPU so that stacks of
// many layers (tens of GB of expert codes and scales) are filled in HBM
// directly instead of being produced on the host and copied.  Element i of
// tensor `tid` under `seed` is bit-identical to what synth.c produces: the
// hash is integer arithmetic, uniform24 is exact in fp32, and the scale is one
// fp32 add and one fp32 multiply (built with -ffp-contract=off, so nothing is
// fused).  Like synth.c it draws numbers only and holds none of the layer's
// arithmetic.
//
// Entry points return 0 on success or the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

inline uint64_t key_of(uint64_t seed, uint64_t tid) {
  return mix64(seed * kGolden + tid * 0xD1B54A32D192ED03ULL + 1ULL);
}

__device__ inline uint64_t hash_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1ULL) * kGolden); }

__device__ inline int8_t randint_at(uint64_t key, uint64_t i, int lo, uint64_t span) {
  const uint64_t h = hash_at(key, i);
  return (int8_t)(lo + (int)(((h >> 32) * span) >> 32));
}

// 16 elements per thread (one 16-byte store when the chunk is whole).
__global__ __launch_bounds__(256) void randint8_kernel(uint64_t key, uint64_t start, int64_t n, int lo,
                                                       uint64_t span, int8_t* __restrict__ out) {
  const int64_t nchunks = (n + 15) / 16;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * 256) {
    const int64_t j0 = c * 16;
    if (j0 + 16 <= n) {
      union { int8_t b[16]; int4 v; } u;
#pragma unroll
      for (int q = 0; q < 16; ++q) u.b[q] = randint_at(key, start + (uint64_t)(j0 + q), lo, span);
      *reinterpret_cast<int4*>(out + j0) = u.v;
    } else {
      for (int64_t j = j0; j < n; ++j) out[j] = randint_at(key, start + (uint64_t)j, lo, span);
    }
  }
}

struct Specials {
  float v[8];
};

__global__ __launch_bounds__(256) void scale_kernel(uint64_t key, uint64_t skey, int use_special, uint64_t start,
                                                    int64_t n, float c, Specials sp, int n_special,
                                                    float exact_value, float* __restrict__ out) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    const uint64_t i = start + (uint64_t)j;
    const float u = (float)(hash_at(key, i) >> 40) * (1.0f / 16777216.0f);
    float v = (0.5f + u) * c;
    if (use_special) {
      const uint64_t hs = hash_at(skey, i);
      const uint64_t sel = hs >> 54;
      if (sel == 0 && n_special > 0) v = sp.v[(hs >> 20) % (uint64_t)n_special];
      else if (sel == 1) v = exact_value;
    }
    out[j] = v;
  }
}

inline unsigned grid_for(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" {

// out[j] = element start + j of the int8 tensor (seed, tid) drawn uniformly
// on [lo, hi], for j < n.  `out` is 16-byte aligned device memory; enqueued
// on `stream`.
int synth_dev_randint8(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, int lo, int hi,
                       int8_t* out, hipStream_t stream) {
  if (n <= 0) return 0;
  if (hi < lo || out == nullptr || (reinterpret_cast<uintptr_t>(out) & 15) != 0)
    return (int)hipErrorInvalidValue;
  const uint64_t span = (uint64_t)(hi - lo + 1);
  hipLaunchKernelGGL(randint8_kernel, dim3(grid_for((n + 15) / 16)), dim3(256), 0, stream,
                     key_of(seed, tid), start, n, lo, span, out);
  return (int)hipGetLastError();
}

// out[j] = scale element start + j of (seed, tid): (0.5f + u) * c, with the
// hash-chosen special values of synth_scale when special_tid != 0.
// `special` is a host array of n_special <= 8 values.
int synth_dev_scale(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, float c,
                    uint64_t special_tid, const float* special, int n_special, float exact_value,
                    float* out, hipStream_t stream) {
  if (n <= 0) return 0;
  if (out == nullptr || n_special < 0 || n_special > 8 || (n_special > 0 && special == nullptr))
    return (int)hipErrorInvalidValue;
  Specials sp{};
  for (int q = 0; q < n_special; ++q) sp.v[q] = special[q];
  hipLaunchKernelGGL(scale_kernel, dim3(grid_for(n)), dim3(256), 0, stream, key_of(seed, tid),
                     key_of(seed, special_tid), special_tid != 0 ? 1 : 0, start, n, c, sp, n_special,
                     exact_value, out);
  return (int)hipGetLastError();
}

}  // extern "C"
