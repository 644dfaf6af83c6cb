// Attainable-peak probes: a plain streaming read of device memory and a loop
// of int8 MFMAs.  They compute nothing of the layer; a benchmark times them
// to report the ceilings this chip reaches in practice beside the published
// ones (HBM 8 TB/s, dense int8 MFMA 5.0 POP/s).
//
// Both kernels fold what they load or compute into a value that is stored
// only if it equals a constant, so the compiler keeps every load and MFMA; the
// store target is a caller buffer of at least 16 bytes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr int kReadUnroll = 8;             // 16-byte loads in flight per lane
constexpr int kImprobable = 0x5EED1234;    // stored only if the fold equals it

// Every wavefront reads contiguous chunks of kReadUnroll KB (one 1 KB load of
// 16 bytes per lane per step, all kReadUnroll in flight), the wavefronts of
// the grid taking chunks in turn; the words after the last whole chunk are
// read by a grid-stride loop.  The loads are non-temporal (streaming), as the
// layer's weight loads are: measured faster than plain loads for a stream
// read once (6.9 against 6.1 TB/s over 2 GiB).
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const v4i* __restrict__ src,
                                                                   size_t n16, int* sink) {
  constexpr size_t kChunk = 64 * kReadUnroll;  // 16-byte words per chunk
  const int lane = threadIdx.x & 63;
  const size_t nwaves = (size_t)gridDim.x * (kProbeThreads / 64);
  const size_t wave = (size_t)blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64;
  const size_t full = n16 / kChunk * kChunk;
  v4i acc = {0, 0, 0, 0};
  for (size_t base = wave * kChunk; base < full; base += nwaves * kChunk) {
    v4i v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + base + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (size_t i = full + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kProbeThreads)
    acc ^= __builtin_nontemporal_load(src + i);
  const int f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (f == kImprobable) sink[threadIdx.x & 3] = f;
}

// Each wavefront runs `iters` rounds of 32 MFMAs: 8 steps of four independent
// accumulator chains (fewer per round let the compiler's accumulator copies
// at the loop edge take a visible share of the issue slots).
// SHAPE 0: v_mfma_i32_16x16x64_i8 (16*16*64*2 = 32768 ops each);
// SHAPE 1: v_mfma_i32_32x32x32_i8 (32*32*32*2 = 65536 ops each).
template <int SHAPE>
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, int* sink) {
  typedef typename std::conditional<SHAPE == 0, v4i, v16i>::type Acc;
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane * 3 + 1, lane ^ 0x55, lane + 7};
  const v4i b = {lane * 5, lane + 11, lane ^ 0x33, lane * 7 + 2};
  Acc c0 = {}, c1 = {}, c2 = {}, c3 = {};
  c1[0] = 1;
  c2[0] = 2;
  c3[0] = 3;
  auto mfma = [&](const v4i& x, const v4i& y, const Acc& c) {
    if constexpr (SHAPE == 0)
      return __builtin_amdgcn_mfma_i32_16x16x64_i8(x, y, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_i32_32x32x32_i8(x, y, c, 0, 0, 0);
  };
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      c0 = mfma(a, b, c0);
      c1 = mfma(b, a, c1);
      c2 = mfma(a, a, c2);
      c3 = mfma(b, b, c3);
    }
  }
  int f = 0;
#pragma unroll
  for (int q = 0; q < (SHAPE == 0 ? 4 : 16); ++q) f ^= c0[q] ^ c1[q] ^ c2[q] ^ c3[q];
  if (f == kImprobable) sink[threadIdx.x & 3] = f;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, size_t bytes, int blocks, void* sink,
                             hipStream_t s) {
  moe_launch(probe_read_kernel, dim3(blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const v4i*>(buf), bytes / 16, static_cast<int*>(sink));
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int shape, int iters, int blocks, void* sink, hipStream_t s) {
  if (shape == 0)
    moe_launch(probe_mfma_kernel<0>, dim3(blocks), dim3(kProbeThreads), 0, s, iters,
                       static_cast<int*>(sink));
  else
    moe_launch(probe_mfma_kernel<1>, dim3(blocks), dim3(kProbeThreads), 0, s, iters,
                       static_cast<int*>(sink));
  return hipGetLastError();
}

}  // namespace moe
