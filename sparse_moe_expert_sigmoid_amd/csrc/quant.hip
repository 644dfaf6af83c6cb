// Weight quantizers: float weights (fp32 or bf16) -> the two quantised expert
// formats of this library.
//
//   int8 per output row: Kimi-Linear-48B-A3B-Instruct LiteRT-LM details,
//     "Conversion notes", quantization of the int8 file (one scale per output
//     row and expert, symmetric min-max): s = max|w_row| / 127,
//     q = round(w / s) in [-127, 127]; an all-zero row gets s = 0, codes 0.
//   int4 per block of 32 inputs: Qwen3-30B-A3B model card, file table (int4
//     blockwise, block 32, fp32 scales) and "Conversion Notes" (block scales
//     below 2^-14 raised to 2^-14): s = max(max|w_block| / 7, 2^-14),
//     q = round(w / s) in [-7, 7], two codes per byte, low nibble first; or
//     the same per block of 128 inputs.
//
// Arithmetic: the scale is an IEEE fp32 division (correctly rounded; the
// library is built without fast-math).  The quotient w / s must be the
// correctly rounded fp32 quotient, then rounded to an integer with halves away
// from zero (roundf) and clamped to the code range.  The divisor is fixed per
// row (block), so each element's quotient takes Markstein's correction step
// (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", IBM J. Res. Dev. 34(1), 1990; also the Handbook of
// Floating-Point Arithmetic, division by FMA): with y = RN(1/s) computed once,
// q0 = RN(w y), r = RN(w - s q0) (exact under an FMA) and q = RN(q0 + r y) =
// RN(w / s) as long as nothing underflows.  For s >= 2^-60 an underflow needs
// |w / s| far below 1/2, where the code is 0 either way; int4 scales are at
// least 2^-14, and int8 rows with a smaller scale divide element by element.
//
// Both kernels make one pass over HBM: the weights are read once (non-
// temporal), codes and scales written once.  Loads are 16 bytes per lane and
// neighbouring lanes read neighbouring bytes.
//   int8 rows: one wavefront per row; a lane owns 8-input units.  Rows of up
//     to 4096 inputs stay in registers between the maximum and the coding;
//     longer rows are read a second time for the coding (mostly from L2).
//   int4 blocks: a lane owns 16 inputs, a block of 32 is a lane pair, so the
//     grid streams over all rows flat.

#include "internal.h"

namespace moe {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kInF32 = 0;
constexpr int kInBf16 = 1;

// 8 consecutive inputs as loaded (non-temporal): bf16 stays packed in four
// dwords until it is used, fp32 is two float4.
template <int IN>
struct Raw8;

template <>
struct Raw8<kInBf16> {
  v4u r;
  __device__ inline void load(const void* __restrict__ w, size_t e) {
    r = __builtin_nontemporal_load(
        reinterpret_cast<const v4u*>(static_cast<const uint16_t*>(w) + e));
  }
  __device__ inline float at(int i) const {  // bf16 -> fp32 is exact
    const unsigned x = r[i >> 1];
    return __uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16));
  }
};

template <>
struct Raw8<kInF32> {
  v4f a, b;
  __device__ inline void load(const void* __restrict__ w, size_t e) {
    const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(w) + e);
    a = __builtin_nontemporal_load(p);
    b = __builtin_nontemporal_load(p + 1);
  }
  __device__ inline float at(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

// Largest magnitude of the 8 inputs.  bf16: on the packed bits (sign cleared,
// two halves per dword compared as unsigned 16-bit values, which orders
// non-negative floats), so the inputs are widened only for the coding.
__device__ inline float absmax8(const Raw8<kInBf16>& v) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v.r[k] & 0x7fff7fffu));
  const unsigned x = __builtin_bit_cast(unsigned, m);
  return fmaxf(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u));
}

__device__ inline float absmax8(const Raw8<kInF32>& v) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v.at(i)));
  return m;
}

__device__ inline float wave_max(float m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  return m;
}

constexpr float kFastDivMin = 0x1p-60f;  // scales at or above use the corrected product

// Nearest integer, halves away from zero: trunc(q + copysign(pred(1/2), q))
// with pred(1/2) the largest float below 1/2.  Adding 1/2 itself would turn
// pred(1/2) into 1; with pred(1/2) every sum rounds onto the right side of the
// next integer.  Equal to roundf(q) for every float with |q| <= 256 (checked
// over all of them); quotients here stay below 128 in magnitude.
__device__ inline int round_half_away(float q) {
  return (int)(q + copysignf(__uint_as_float(0x3EFFFFFFu), q));
}

// round(RN(x / s)) with y = RN(1 / s) (see the header).  No clamp is needed:
// s = RN(m / c) >= (m / c)(1 - 2^-24) for the largest magnitude m of the row
// (block) and c = 127 (7), so |x / s| <= c (1 + 2^-23), which rounds to at most
// c; a raised int4 scale only shrinks the quotient.
__device__ inline int code(float x, float s, float y) {
#pragma clang fp contract(off)
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, s, x);
  const float q = __builtin_fmaf(r, y, q0);
  return round_half_away(q);
}

__device__ inline int code_div(float x, float s) { return round_half_away(x / s); }

// Packing without masks: codes are summed as signed values at their byte
// (nibble) positions, then the offset 0x80 (0x8) is added to every byte
// (nibble) and xor-ed away again.  c + 0x80 lies in [1, 255] (c + 8 in
// [0, 15]), so no position carries into the next, and (c + 0x80) ^ 0x80 is
// the two's-complement byte (nibble) of c.

// 8 int8 codes as two dwords, input order = byte order.
template <int IN>
__device__ inline v2u codes_i8(const Raw8<IN>& v, float s, float y) {
  unsigned w[2] = {0u, 0u};
  if (s >= kFastDivMin) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i >> 2] += (unsigned)code(v.at(i), s, y) << (8 * (i & 3));
  } else if (s > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i >> 2] += (unsigned)code_div(v.at(i), s) << (8 * (i & 3));
  }
  return v2u{(w[0] + 0x80808080u) ^ 0x80808080u, (w[1] + 0x80808080u) ^ 0x80808080u};
}

// 8 int4 codes in one dword: byte i = code(2i) | code(2i+1) << 4.  s >= 2^-14.
template <int IN>
__device__ inline unsigned codes_i4(const Raw8<IN>& v, float s, float y) {
  unsigned w = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) w += (unsigned)code(v.at(i), s, y) << (4 * i);
  return (w + 0x88888888u) ^ 0x88888888u;
}

// RN(m / 7) by the same correction with the constant y7 = RN(1/7): equal to
// the correctly rounded quotient for every finite m >= 0 (checked over all of
// them).
__device__ inline float div7(float m) {
#pragma clang fp contract(off)
  const float y7 = 1.0f / 7.0f;
  const float q0 = m * y7;
  const float r = __builtin_fmaf(-q0, 7.0f, m);
  return __builtin_fmaf(r, y7, q0);
}

// ---------------------------------------------------------------- int8 rows
// One wavefront per row; a lane's units are u = lane + 64 j.  Lanes past the
// row end load the row's last unit again (a duplicate cannot change the
// maximum) and store its identical codes again, so every load and store is
// unconditional.
template <int IN, int J>
__device__ inline void load_row(Raw8<IN> (&b)[J], const void* __restrict__ w, long long row,
                                int K, int U, int lane) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int u = min(lane + kWave * j, U - 1);
    b[j].load(w, (size_t)row * (size_t)K + 8 * (size_t)u);
  }
}

template <int IN, int J>
__device__ inline void code_row(const Raw8<IN> (&b)[J], long long row, int K, int U, int lane,
                                int8_t* __restrict__ q, float* __restrict__ s) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) m = fmaxf(m, absmax8(b[j]));
  m = wave_max(m);
  const float sc = m / 127.0f;
  const float y = sc >= kFastDivMin ? 1.0f / sc : 0.0f;
  s[row] = sc;  // every lane writes the same value: no branch around the store
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int u = min(lane + kWave * j, U - 1);
    __builtin_nontemporal_store(
        codes_i8(b[j], sc, y),
        reinterpret_cast<v2u*>(q + (size_t)row * (size_t)K + 8 * (size_t)u));
  }
}

// Rows of up to 64*J units (4096 inputs at J = 8): the row stays in registers
// between the maximum and the coding.  One row per wavefront and no loop: the
// grid covers every row and occupancy overlaps them (measured faster than
// persistent wavefronts that prefetch their next row).
template <int IN, int J>
__global__ __launch_bounds__(256) void quant_i8_rows_kernel(const void* __restrict__ w,
                                                            long long rows, int K,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ s) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x / kWave);
  if (row >= rows) return;  // whole wavefronts leave; no workgroup barrier follows
  const int U = K >> 3;
  Raw8<IN> a[J];
  load_row<IN, J>(a, w, row, K, U, lane);
  code_row<IN, J>(a, row, K, U, lane, q, s);
}

// Longer rows: persistent wavefronts stream each row twice (maximum, then
// codes; the second read mostly from L2), rows strided by the grid.
template <int IN>
__global__ __launch_bounds__(256) void quant_i8_long_rows_kernel(const void* __restrict__ w,
                                                                 long long rows, int K,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ s) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long nw = (long long)gridDim.x * 4;
  const int U = K >> 3;
  for (long long row = (long long)blockIdx.x * 4 + (threadIdx.x / kWave); row < rows;
       row += nw) {
    const size_t base = (size_t)row * (size_t)K;
    float m = 0.0f;
    for (int u = lane; u < U; u += kWave) {
      Raw8<IN> v;
      v.load(w, base + 8 * (size_t)u);
      m = fmaxf(m, absmax8(v));
    }
    m = wave_max(m);
    const float sc = m / 127.0f;
    const float y = sc >= kFastDivMin ? 1.0f / sc : 0.0f;
    if (lane == 0) s[row] = sc;
    for (int u = lane; u < U; u += kWave) {
      Raw8<IN> v;
      v.load(w, base + 8 * (size_t)u);
      __builtin_nontemporal_store(codes_i8(v, sc, y),
                                  reinterpret_cast<v2u*>(q + base + 8 * (size_t)u));
    }
  }
}

// ---------------------------------------------------------------- int4 blocks
// Flat over all pairs of 8-input units of all rows: a lane owns 16 inputs
// (two units), a block of 32 (128) is LPB = 2 (8) neighbouring lanes, its
// maximum one (three) swizzles away.  A workgroup codes 256 * kI4Pairs pairs
// (kI4Pairs per lane, strided by 256 so that each load instruction reads
// contiguous bytes), all loaded before any is coded; the grid covers every
// pair.  Lanes past the end load the last block again (the pair count is a
// multiple of LPB; the lane's place in its block is kept) and store its
// identical codes and scale again, so no load or store is conditional.
constexpr int kI4Pairs = 8;

template <int IN>
struct Pair16 {
  Raw8<IN> lo, hi;
};

template <int IN, int LPB>
__global__ __launch_bounds__(256) void quant_i4_blocks_kernel(const void* __restrict__ w,
                                                              long long pairs,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ s) {
  const float floor_s = 1.0f / 16384.0f;  // 2^-14
  long long g[kI4Pairs];
  Pair16<IN> b[kI4Pairs];
#pragma unroll
  for (int n = 0; n < kI4Pairs; ++n) {
    const long long x = (long long)blockIdx.x * (256 * kI4Pairs) + 256 * n + threadIdx.x;
    g[n] = x < pairs ? x : pairs - LPB + (x & (LPB - 1));  // the last block
    b[n].lo.load(w, 16 * (size_t)g[n]);
    b[n].hi.load(w, 16 * (size_t)g[n] + 8);
  }
#pragma unroll
  for (int n = 0; n < kI4Pairs; ++n) {
    float m = fmaxf(absmax8(b[n].lo), absmax8(b[n].hi));
#pragma unroll
    for (int o = 1; o < LPB; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    const float sc = fmaxf(div7(m), floor_s);
    const float y = 1.0f / sc;
    s[g[n] / LPB] = sc;  // every lane of the block writes the same value
    __builtin_nontemporal_store(v2u{codes_i4(b[n].lo, sc, y), codes_i4(b[n].hi, sc, y)},
                                reinterpret_cast<v2u*>(q) + g[n]);
  }
}

// Workgroups of one kernel that fit on the device at once (occupancy x CUs),
// queried once per kernel: a persistent grid larger than this would leave a
// tail of workgroups that start only when the first ones finish.
template <typename Kern>
long long resident_blocks(Kern kern) {
  static const long long n = [&] {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256LL * 4;
    return (long long)(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 256);
  }();
  return n;
}

template <int IN, int J>
hipError_t launch_i8_j(const void* w, long long rows, int K, int8_t* q, float* s,
                       hipStream_t st) {
  const long long blocks = (rows + 3) / 4;  // rows <= 2^32: at most 2^30 workgroups
  moe_launch(quant_i8_rows_kernel<IN, J>, dim3((unsigned)blocks), dim3(256), 0, st, w, rows, K, q,
             s);
  return hipGetLastError();
}

template <int IN>
hipError_t launch_i8(const void* w, long long rows, int K, int8_t* q, float* s,
                     hipStream_t st) {
  switch ((K / 8 + kWave - 1) / kWave) {
    case 1: return launch_i8_j<IN, 1>(w, rows, K, q, s, st);
    case 2: return launch_i8_j<IN, 2>(w, rows, K, q, s, st);
    case 3: return launch_i8_j<IN, 3>(w, rows, K, q, s, st);
    case 4: return launch_i8_j<IN, 4>(w, rows, K, q, s, st);
    case 5: return launch_i8_j<IN, 5>(w, rows, K, q, s, st);
    case 6: return launch_i8_j<IN, 6>(w, rows, K, q, s, st);
    case 7: return launch_i8_j<IN, 7>(w, rows, K, q, s, st);
    case 8: return launch_i8_j<IN, 8>(w, rows, K, q, s, st);
    default: {
      const long long cap = resident_blocks(quant_i8_long_rows_kernel<IN>);
      long long blocks = (rows + 3) / 4;
      blocks = blocks < cap ? blocks : cap;
      moe_launch(quant_i8_long_rows_kernel<IN>, dim3((unsigned)blocks), dim3(256), 0, st, w,
                 rows, K, q, s);
      return hipGetLastError();
    }
  }
}

template <int IN, int LPB>
hipError_t launch_i4(const void* w, long long rows, int K, uint8_t* q, float* s,
                     hipStream_t st) {
  const long long pairs = rows * (long long)(K / 16);  // a multiple of LPB: K % (16 LPB) == 0
  const long long blocks = (pairs + 256 * kI4Pairs - 1) / (256 * kI4Pairs);
  moe_launch(quant_i4_blocks_kernel<IN, LPB>, dim3((unsigned)blocks), dim3(256), 0, st, w, pairs,
             q, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int fmt, int in_type, const void* w, long long rows, int K,
                           void* codes, float* scales, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (fmt == 1) {
    TimedLaunch t(K_QUANT_I8, st);
    return in_type == kInF32
               ? launch_i8<kInF32>(w, rows, K, static_cast<int8_t*>(codes), scales, st)
               : launch_i8<kInBf16>(w, rows, K, static_cast<int8_t*>(codes), scales, st);
  }
  TimedLaunch t(K_QUANT_I4, st);
  uint8_t* c = static_cast<uint8_t*>(codes);
  if (fmt == 3)
    return in_type == kInF32 ? launch_i4<kInF32, 8>(w, rows, K, c, scales, st)
                             : launch_i4<kInBf16, 8>(w, rows, K, c, scales, st);
  return in_type == kInF32 ? launch_i4<kInF32, 2>(w, rows, K, c, scales, st)
                           : launch_i4<kInBf16, 2>(w, rows, K, c, scales, st);
}

}  // namespace moe
