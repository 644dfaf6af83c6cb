// Internal declarations shared by the HIP translation units of the MoE
// library (kernel launchers and small device helpers).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- sizes
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kRouterChunk = 256;      // router logits are summed in fixed 256-input chunks
constexpr int kMaxK = 16;              // top-k limit
constexpr int kMaxE = 1024;            // experts per layer limit
constexpr int kKStep = 64;             // K of one int8 MFMA (16x16x64)
constexpr int kTileRows = 16;          // routed rows per FFN tile (MFMA N)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- workspace layout
// Router: fp32 partial logits [ceil(d/256)][T][E].
inline size_t route_ws_bytes(int T, int d, int E) {
  size_t chunks = (size_t)((d + kRouterChunk - 1) / kRouterChunk);
  return align_up(chunks * (size_t)T * (size_t)E * sizeof(float), 256);
}

// Expert FFN, quantised formats:
//   xq   [T][2][d] int8   activations as two int8 digits (see encode_rows)
//   xs   [T] fp32         per-row power-of-two scale of xq
//   h    [R][I] fp32      silu(gate) * up
//   hq   [R][2][I] int8   h as two digits
//   hs   [R] fp32
// fp32 format: only h.
struct FfnWs {
  int8_t* xq;
  float* xs;
  float* h;
  int8_t* hq;
  float* hs;
  size_t bytes;
};

inline FfnWs ffn_ws_layout(void* base, int T, int R, int d, int inter, bool quantised) {
  FfnWs w{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t n) {
    char* p = b ? b + off : nullptr;
    off = align_up(off + n, 256);
    return p;
  };
  w.h = reinterpret_cast<float*>(take((size_t)R * inter * sizeof(float)));
  if (quantised) {
    w.xq = reinterpret_cast<int8_t*>(take((size_t)T * 2 * d));
    w.xs = reinterpret_cast<float*>(take((size_t)T * sizeof(float)));
    w.hq = reinterpret_cast<int8_t*>(take((size_t)R * 2 * inter));
    w.hs = reinterpret_cast<float*>(take((size_t)R * sizeof(float)));
  }
  w.bytes = off;
  return w;
}

// Upper bound on the number of FFN tiles (kTileRows rows of one expert each)
// for R rows spread over E experts: sum_e ceil(c_e/MT) <= n + (R - n)/MT with
// n = min(E, R) non-empty experts at most.
inline int max_tiles(int R, int E, int mt) {
  int n = R < E ? R : E;
  return n + (R - n + mt - 1) / mt;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.
hipError_t launch_router(int router, const float* x, const float* wr, const float* bias, int T,
                         int d, int E, int k, float scale, int32_t* idx, float* w,
                         float* partial, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* row_token, int32_t* token_row, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);
hipError_t launch_encode_rows(const float* v, int n, int K, int8_t* q, float* sig,
                              hipStream_t s);
hipError_t launch_ffn_quant(int fmt, const void* wgu, const float* sgu, const void* wdn,
                            const float* sdn, int E, int d, int inter, const float* x, int T,
                            const int32_t* row_token, const int32_t* offsets, int R,
                            float* rows_out, const FfnWs& ws, hipStream_t s);
hipError_t launch_ffn_f32(const float* wgu, const float* wdn, int E, int d, int inter,
                          const float* x, int T, const int32_t* row_token,
                          const int32_t* offsets, int R, float* rows_out, float* h,
                          hipStream_t s);
hipError_t launch_combine(const float* rows, const int32_t* token_row, const float* w,
                          const float* shared, const float* residual, int T, int k, int d,
                          float* y, hipStream_t s);

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)

// A tile is up to `mt` consecutive rows of one expert.  Tiles are numbered
// expert by expert; every lane of the calling wave gets the same answer.
struct Tile {
  int e, r0, nr;
};

__device__ inline bool find_tile(const int32_t* __restrict__ offsets, int E, int R, int mt,
                                 int tile, Tile& out) {
  if (offsets == nullptr) {  // one expert over rows [0, R)
    int r0 = tile * mt;
    if (r0 >= R) return false;
    out.e = 0;
    out.r0 = r0;
    out.nr = min(mt, R - r0);
    return true;
  }
  const int lane = threadIdx.x & (kWave - 1);
  int base = 0;
  for (int c0 = 0; c0 < E; c0 += kWave) {
    const int e = c0 + lane;
    int start = 0, cnt = 0;
    if (e < E) {
      start = offsets[e];
      cnt = offsets[e + 1] - start;
      if (cnt < 0) cnt = 0;
    }
    const int nt = (cnt + mt - 1) / mt;
    int incl = nt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    if (tile < base + total) {
      const unsigned long long m = __ballot(base + incl > tile);
      const int L = __ffsll((long long)m) - 1;
      const int excl = __shfl(incl - nt, L, kWave);
      const int st = __shfl(start, L, kWave);
      const int ct = __shfl(cnt, L, kWave);
      const int sub = tile - base - excl;
      out.e = c0 + L;
      out.r0 = st + sub * mt;
      out.nr = min(mt, ct - sub * mt);
      return out.r0 >= 0 && out.r0 + out.nr <= R;
    }
    base += total;
  }
  return false;
}

__device__ inline float silu_f(float z) { return z / (1.0f + expf(-z)); }

#endif

}  // namespace moe
