// Expert SwiGLU FFNs over grouped rows, weights dequantised in-kernel.
//
//   h[r]    = silu(Wg[e] x[tok(r)]) * (Wu[e] x[tok(r)])          (gate/up, K = d)
//   rows[r] = Wd[e] h[r]                                         (down,    K = I)
//
// The experts are SwiGLU FFNs with SiLU (Kimi-Linear LiteRT-LM DETAILS.md,
// Conversion notes, mixture-of-experts bullet; Qwen3-30B-A3B LiteRT card,
// Accuracy: activation 'silu').  Formats: int8 codes with one fp32 scale per
// output row and expert (same DETAILS.md bullet on the int8 file), int4 codes
// in blocks of 32 along the input with fp32 scales raised to 2^-14 (Qwen3
// card, Available Artifacts and Conversion Notes), and plain fp32.
//
// Quantised formats run on the int8 matrix cores.  The int8/int4 codes are
// the MFMA A operand as stored (no dequantisation to floating point at all);
// the fp32 activations are written as two int8 digits per element against a
// power-of-two scale per row, v = 2^-p (d0 + d1/256), so
//   sum_k q_k v_k = 2^-p (sum_k q_k d0_k + 2^-8 sum_k q_k d1_k)
// is two exact int32 MFMA accumulations.  The encoding error is below
// 2^-16 of the row's largest |v| (16-bit fixed point per row), far inside the
// fp32 tolerance of the layer; accumulation is exact integer arithmetic.
//
// Work split: a tile is up to 16 rows of one expert (the MFMA N side); a
// workgroup of 4 wavefronts owns 64 output columns of one tile, each
// wavefront 16 (the MFMA M side).  The tile's activation digits sit in LDS;
// the weight rows stream from HBM with 16-byte loads, each byte read once
// per tile.  Tiles are found on the device from the expert offsets, so no
// count is ever copied back to the host.
#include "internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kLdsPad = 16;  // bytes added per LDS row of digits

// ------------------------------------------------------------------ encode
// One wavefront per row: p = 7 - exponent(max|v|) (minus 1 if that overshoots
// 127), a = v * 2^p (exact), d0 = rint(a), d1 = rint((a - d0) * 256), both
// clamped to [-127, 127]; sig = 2^-p (0 for an all-zero row).
__global__ __launch_bounds__(256) void encode_rows_kernel(const float* __restrict__ v, int n,
                                                          int K, int8_t* __restrict__ q,
                                                          float* __restrict__ sig) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= n) return;
  const float* row = v + (size_t)r * K;
  float m = 0.0f;
  for (int c = lane; c < K / 4; c += kWave) {
    const float4 a = *reinterpret_cast<const float4*>(row + 4 * c);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  int p = 0;
  if (m > 0.0f) {
    int ex;
    frexpf(m, &ex);              // m = f * 2^ex, f in [0.5, 1)
    p = 7 - ex;
    if (ldexpf(m, p) > 127.0f) p -= 1;
  }
  int8_t* q0 = q + (size_t)r * 2 * K;
  int8_t* q1 = q0 + K;
  for (int c = lane; c < K / 4; c += kWave) {
    const float4 a = *reinterpret_cast<const float4*>(row + 4 * c);
    float av[4] = {a.x, a.y, a.z, a.w};
    char4 o0, o1;
    signed char d0v[4], d1v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float s = m > 0.0f ? ldexpf(av[u], p) : 0.0f;
      float d0 = rintf(s);
      d0 = fminf(fmaxf(d0, -127.0f), 127.0f);
      float d1 = rintf((s - d0) * 256.0f);
      d1 = fminf(fmaxf(d1, -127.0f), 127.0f);
      d0v[u] = (signed char)(int)d0;
      d1v[u] = (signed char)(int)d1;
    }
    o0 = make_char4(d0v[0], d0v[1], d0v[2], d0v[3]);
    o1 = make_char4(d1v[0], d1v[1], d1v[2], d1v[3]);
    *reinterpret_cast<char4*>(q0 + 4 * c) = o0;
    *reinterpret_cast<char4*>(q1 + 4 * c) = o1;
  }
  if (lane == 0) sig[r] = m > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
}

// Copy the tile's digit rows (2*K bytes each) into LDS rows of `ldr` bytes.
__device__ inline void stage_rows(int8_t* lds, int ldr, const int8_t* __restrict__ src, int K,
                                  const int32_t* __restrict__ row_token, int r0, int nr) {
  const int per_row = (2 * K) / 16;  // 16-byte chunks
  for (int q = threadIdx.x; q < nr * per_row; q += blockDim.x) {
    const int j = q / per_row, c = q % per_row;
    const int src_row = row_token ? row_token[r0 + j] : r0 + j;
    const v4i val = *reinterpret_cast<const v4i*>(src + (size_t)src_row * 2 * K + 16 * c);
    *reinterpret_cast<v4i*>(lds + j * ldr + 16 * c) = val;
  }
}

// ------------------------------------------------------------------ int8
// MODE 0: gate/up with SwiGLU epilogue -> h [R][I].
// MODE 1: down -> rows [R][d].
// K = reduction length; W points at expert 0's matrix [E][N][K] (N = 2I or d).
template <int MODE>
__global__ __launch_bounds__(256) void ffn_i8_kernel(const int8_t* __restrict__ W,
                                                     const float* __restrict__ S,
                                                     const int8_t* __restrict__ act_q,
                                                     const float* __restrict__ act_s,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int K, int N_out, int R,
                                                     float* __restrict__ out) {
  extern __shared__ int8_t lds[];
  Tile tl;
  if (!find_tile(offsets, E, R, kTileRows, blockIdx.y, tl)) return;
  const int ldr = 2 * K + kLdsPad;
  stage_rows(lds, ldr, act_q, K, MODE == 0 ? row_token : nullptr, tl.r0, tl.nr);
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int c0 = (blockIdx.x * (blockDim.x / kWave) + wave) * 16;  // output columns
  if (c0 >= N_out) return;
  const int i = lane & 15, g = lane >> 4;
  const size_t rows_per_expert = MODE == 0 ? (size_t)2 * N_out : (size_t)N_out;
  const int8_t* wa = W + ((size_t)tl.e * rows_per_expert + c0 + i) * K + 16 * g;
  const int8_t* wb = wa + (size_t)N_out * K;  // up rows (MODE 0 only)
  const bool jv = i < tl.nr;
  const int8_t* b0 = lds + i * ldr + 16 * g;
  const int8_t* b1 = b0 + K;

  v4i acc_a0 = {0, 0, 0, 0}, acc_a1 = {0, 0, 0, 0};
  v4i acc_b0 = {0, 0, 0, 0}, acc_b1 = {0, 0, 0, 0};
  constexpr int U = 4;
  int k = 0;
  for (; k + U * kKStep <= K; k += U * kKStep) {
    v4i ra[U], rb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ra[u] = *reinterpret_cast<const v4i*>(wa + k + u * kKStep);
      if (MODE == 0) rb[u] = *reinterpret_cast<const v4i*>(wb + k + u * kKStep);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v4i x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
      if (jv) {
        x0 = *reinterpret_cast<const v4i*>(b0 + k + u * kKStep);
        x1 = *reinterpret_cast<const v4i*>(b1 + k + u * kKStep);
      }
      acc_a0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra[u], x0, acc_a0, 0, 0, 0);
      acc_a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra[u], x1, acc_a1, 0, 0, 0);
      if (MODE == 0) {
        acc_b0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(rb[u], x0, acc_b0, 0, 0, 0);
        acc_b1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(rb[u], x1, acc_b1, 0, 0, 0);
      }
    }
  }
  for (; k < K; k += kKStep) {
    const v4i ra = *reinterpret_cast<const v4i*>(wa + k);
    v4i rb = {0, 0, 0, 0};
    if (MODE == 0) rb = *reinterpret_cast<const v4i*>(wb + k);
    v4i x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
    if (jv) {
      x0 = *reinterpret_cast<const v4i*>(b0 + k);
      x1 = *reinterpret_cast<const v4i*>(b1 + k);
    }
    acc_a0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra, x0, acc_a0, 0, 0, 0);
    acc_a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra, x1, acc_a1, 0, 0, 0);
    if (MODE == 0) {
      acc_b0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(rb, x0, acc_b0, 0, 0, 0);
      acc_b1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(rb, x1, acc_b1, 0, 0, 0);
    }
  }

  // D layout (16x16): lane holds rows 4g..4g+3 (weight rows) of column i (tile row).
  if (!jv) return;
  const int r = tl.r0 + i;
  const int src = (MODE == 0 && row_token) ? row_token[r] : r;
  const float sig = act_s[MODE == 0 ? src : r];
  float res[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int n = c0 + 4 * g + c;
    const float va = (float)acc_a0[c] + (float)acc_a1[c] * (1.0f / 256.0f);
    if (MODE == 0) {
      const float* se = S + (size_t)tl.e * 2 * N_out;
      const float gate = se[n] * sig * va;
      const float vb = (float)acc_b0[c] + (float)acc_b1[c] * (1.0f / 256.0f);
      const float up = se[N_out + n] * sig * vb;
      res[c] = silu_f(gate) * up;
    } else {
      res[c] = S[(size_t)tl.e * N_out + n] * sig * va;
    }
  }
  *reinterpret_cast<float4*>(out + (size_t)r * N_out + c0 + 4 * g) =
      make_float4(res[0], res[1], res[2], res[3]);
}

// ------------------------------------------------------------------ int4
// Codes packed two per byte (element 2i low nibble).  One 16x16x32 MFMA per
// block of 32 inputs, so each block's integer sum gets its own scale
// max(s, 2^-14) before it joins the fp32 accumulator.
__device__ inline long unpack8_int4(unsigned w) {
  // nibbles -> sign-extended bytes, element order kept
  const unsigned lo = w & 0x0F0F0F0Fu;          // elements 0,2,4,6
  const unsigned hi = (w >> 4) & 0x0F0F0F0Fu;   // elements 1,3,5,7
  const unsigned slo = ((lo ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
  const unsigned shi = ((hi ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
  const unsigned o0 = __builtin_amdgcn_perm(shi, slo, 0x05010400u);  // e0 e1 e2 e3
  const unsigned o1 = __builtin_amdgcn_perm(shi, slo, 0x07030602u);  // e4 e5 e6 e7
  return (long)(((unsigned long)o1 << 32) | o0);
}

template <int MODE>
__global__ __launch_bounds__(256) void ffn_i4_kernel(const uint8_t* __restrict__ W,
                                                     const float* __restrict__ S,
                                                     const int8_t* __restrict__ act_q,
                                                     const float* __restrict__ act_s,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int K, int N_out, int R,
                                                     float* __restrict__ out) {
  extern __shared__ int8_t lds[];
  Tile tl;
  if (!find_tile(offsets, E, R, kTileRows, blockIdx.y, tl)) return;
  const int ldr = 2 * K + kLdsPad;
  stage_rows(lds, ldr, act_q, K, MODE == 0 ? row_token : nullptr, tl.r0, tl.nr);
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int c0 = (blockIdx.x * (blockDim.x / kWave) + wave) * 16;
  if (c0 >= N_out) return;
  const int i = lane & 15, g = lane >> 4;
  const int nblk = K / 32;
  const size_t rows_per_expert = MODE == 0 ? (size_t)2 * N_out : (size_t)N_out;
  const size_t row_a = (size_t)tl.e * rows_per_expert + c0 + i;
  const uint8_t* wa = W + row_a * (K / 2) + 4 * g;
  const uint8_t* wb = wa + (size_t)N_out * (K / 2);
  // scales of this lane's four output rows 4g..4g+3
  const float* sa = S + ((size_t)tl.e * rows_per_expert + c0 + 4 * g) * nblk;
  const float* sb = sa + (size_t)N_out * nblk;
  const bool jv = i < tl.nr;
  const int8_t* b0 = lds + i * ldr + 8 * g;
  const int8_t* b1 = b0 + K;
  const float floor_s = 1.0f / 16384.0f;  // 2^-14

  float fa[4] = {0.f, 0.f, 0.f, 0.f}, fb[4] = {0.f, 0.f, 0.f, 0.f};
  const v4i zero = {0, 0, 0, 0};
  for (int b = 0; b < nblk; ++b) {
    const long a = unpack8_int4(*reinterpret_cast<const unsigned*>(wa + 16 * b));
    long bb = 0;
    if (MODE == 0) bb = unpack8_int4(*reinterpret_cast<const unsigned*>(wb + 16 * b));
    long x0 = 0, x1 = 0;
    if (jv) {
      x0 = *reinterpret_cast<const long*>(b0 + 32 * b);
      x1 = *reinterpret_cast<const long*>(b1 + 32 * b);
    }
    const v4i pa0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, x0, zero, 0, 0, 0);
    const v4i pa1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, x1, zero, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float s = fmaxf(sa[(size_t)c * nblk + b], floor_s);
      fa[c] = fmaf(s, (float)(pa0[c] * 256 + pa1[c]), fa[c]);
    }
    if (MODE == 0) {
      const v4i pb0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(bb, x0, zero, 0, 0, 0);
      const v4i pb1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(bb, x1, zero, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float s = fmaxf(sb[(size_t)c * nblk + b], floor_s);
        fb[c] = fmaf(s, (float)(pb0[c] * 256 + pb1[c]), fb[c]);
      }
    }
  }

  if (!jv) return;
  const int r = tl.r0 + i;
  const int src = (MODE == 0 && row_token) ? row_token[r] : r;
  const float sig = act_s[MODE == 0 ? src : r] * (1.0f / 256.0f);
  float res[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (MODE == 0) res[c] = silu_f(fa[c] * sig) * (fb[c] * sig);
    else res[c] = fa[c] * sig;
  }
  *reinterpret_cast<float4*>(out + (size_t)r * N_out + c0 + 4 * g) =
      make_float4(res[0], res[1], res[2], res[3]);
}

// ------------------------------------------------------------------ fp32
// Plain fp32 weights: one wavefront per output column, lanes split the
// reduction, a fixed butterfly adds the lanes.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ W,
                                                      const float* __restrict__ act,
                                                      const int32_t* __restrict__ row_token,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int K, int N_out, int R,
                                                      float* __restrict__ out) {
  Tile tl;
  if (!find_tile(offsets, E, R, kTileRows, blockIdx.y, tl)) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * (blockDim.x / kWave) + wave;
  if (n >= N_out) return;
  const size_t rows_per_expert = MODE == 0 ? (size_t)2 * N_out : (size_t)N_out;
  const float* wa = W + ((size_t)tl.e * rows_per_expert + n) * K;
  const float* wb = wa + (size_t)N_out * K;
  for (int j = 0; j < tl.nr; ++j) {
    const int r = tl.r0 + j;
    const int src = (MODE == 0 && row_token) ? row_token[r] : r;
    const float* a = act + (size_t)src * K;
    float sa = 0.f, sb = 0.f;
    for (int c = lane; c < K / 4; c += kWave) {
      const float4 av = *reinterpret_cast<const float4*>(a + 4 * c);
      const float4 w1 = *reinterpret_cast<const float4*>(wa + 4 * c);
      sa = fmaf(w1.x, av.x, sa); sa = fmaf(w1.y, av.y, sa);
      sa = fmaf(w1.z, av.z, sa); sa = fmaf(w1.w, av.w, sa);
      if (MODE == 0) {
        const float4 w2 = *reinterpret_cast<const float4*>(wb + 4 * c);
        sb = fmaf(w2.x, av.x, sb); sb = fmaf(w2.y, av.y, sb);
        sb = fmaf(w2.z, av.z, sb); sb = fmaf(w2.w, av.w, sb);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      sa += __shfl_xor(sa, o, kWave);
      sb += __shfl_xor(sb, o, kWave);
    }
    if (lane == 0) out[(size_t)r * N_out + n] = MODE == 0 ? silu_f(sa) * sb : sa;
  }
}

int g_max_lds = 64 * 1024;

}  // namespace

void set_max_lds(int bytes) { g_max_lds = bytes; }

hipError_t launch_encode_rows(const float* v, int n, int K, int8_t* q, float* sig,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(encode_rows_kernel, dim3((n + 3) / 4), dim3(256), 0, s, v, n, K, q, sig);
  return hipGetLastError();
}

hipError_t launch_ffn_quant(int fmt, const void* wgu, const float* sgu, const void* wdn,
                            const float* sdn, int E, int d, int inter, const float* x, int T,
                            const int32_t* row_token, const int32_t* offsets, int R,
                            float* rows_out, const FfnWs& ws, hipStream_t s) {
  hipError_t err = launch_encode_rows(x, T, d, ws.xq, ws.xs, s);
  if (err != hipSuccess) return err;
  const int tiles = offsets ? max_tiles(R, E, kTileRows) : (R + kTileRows - 1) / kTileRows;
  const size_t lds_gu = (size_t)kTileRows * (2 * d + kLdsPad);
  const size_t lds_dn = (size_t)kTileRows * (2 * inter + kLdsPad);
  if ((int)lds_gu > g_max_lds || (int)lds_dn > g_max_lds) return hipErrorInvalidValue;
  dim3 grid_gu((inter + 63) / 64, tiles), grid_dn((d + 63) / 64, tiles);
  if (fmt == 1) {
    hipLaunchKernelGGL(ffn_i8_kernel<0>, grid_gu, dim3(256), lds_gu, s,
                       static_cast<const int8_t*>(wgu), sgu, ws.xq, ws.xs, row_token, offsets,
                       E, d, inter, R, ws.h);
  } else {
    hipLaunchKernelGGL(ffn_i4_kernel<0>, grid_gu, dim3(256), lds_gu, s,
                       static_cast<const uint8_t*>(wgu), sgu, ws.xq, ws.xs, row_token, offsets,
                       E, d, inter, R, ws.h);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_encode_rows(ws.h, R, inter, ws.hq, ws.hs, s);
  if (err != hipSuccess) return err;
  if (fmt == 1) {
    hipLaunchKernelGGL(ffn_i8_kernel<1>, grid_dn, dim3(256), lds_dn, s,
                       static_cast<const int8_t*>(wdn), sdn, ws.hq, ws.hs, row_token, offsets,
                       E, inter, d, R, rows_out);
  } else {
    hipLaunchKernelGGL(ffn_i4_kernel<1>, grid_dn, dim3(256), lds_dn, s,
                       static_cast<const uint8_t*>(wdn), sdn, ws.hq, ws.hs, row_token, offsets,
                       E, inter, d, R, rows_out);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_f32(const float* wgu, const float* wdn, int E, int d, int inter,
                          const float* x, int T, const int32_t* row_token,
                          const int32_t* offsets, int R, float* rows_out, float* h,
                          hipStream_t s) {
  (void)T;
  const int tiles = offsets ? max_tiles(R, E, kTileRows) : (R + kTileRows - 1) / kTileRows;
  hipLaunchKernelGGL(ffn_f32_kernel<0>, dim3((inter + 3) / 4, tiles), dim3(256), 0, s, wgu, x,
                     row_token, offsets, E, d, inter, R, h);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ffn_f32_kernel<1>, dim3((d + 3) / 4, tiles), dim3(256), 0, s, wdn, h,
                     row_token, offsets, E, inter, d, R, rows_out);
  return hipGetLastError();
}

}  // namespace moe
