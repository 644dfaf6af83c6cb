// Internal declarations shared by the HIP translation units of the MoE
// library (kernel launchers and small device helpers).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace moe {

// sizes, limits and the workspace layouts: layout.h (plain host C++)
constexpr int kWave = 64;              // CDNA wavefront width
constexpr size_t kLdsBytes = kPlanLdsBytes;  // LDS per workgroup (gfx950)
constexpr int kKStep = kPlanKStep;     // K of one int8 MFMA (16x16x64)
constexpr int kTileRows = kPlanTileRows;  // routed rows per FFN tile (MFMA N)

// One expert set for the quantised FFN launchers.
struct FfnSet {
  int fmt;                   // 1 = int8 rows, 2 = int4 blocks of 32, 3 = int4 blocks of 128
  int layout;                // 0 = rows, 1 = tiled (both sets of one launch alike)
  int E, inter, R;
  const void* wgu;
  const float* sgu;
  const void* wdn;
  const float* sdn;
  const int32_t* row_token;  // NULL = identity
  const int32_t* offsets;    // NULL = one expert over R rows
  int8_t* hq;
  float* hs;
  float* out;                // [R][d]
  const int32_t* pairs_idx;  // non-NULL: rows are the R = T*k pairs of topk_idx, grouped in-kernel
  int k;
  int act;                   // gate activation: 0 silu, 1 gelu_tanh
};

// ---------------------------------------------------------------- kernel timer
// Measurement aid (off unless a context turns it on): each launch is
// bracketed by a pair of HIP events on its own stream.
enum KernelId {
  K_ROUTER_LOGITS, K_ROUTER_TOPK, K_PERMUTE, K_FILL, K_ENCODE_ROWS,
  K_FFN_I8_GATE_UP, K_FFN_I8_DOWN, K_FFN_I4_GATE_UP, K_FFN_I4_DOWN,
  K_FFN_F32_GATE_UP, K_FFN_F32_DOWN, K_COMBINE, K_ROUTER_TAIL, K_FFN_I8_GATE_UP_GEMM,
  K_FFN_I8_DOWN_GEMM, K_QUANT_I8, K_QUANT_I4, K_FFN_I4_GATE_UP_GEMM, K_FFN_I4_DOWN_GEMM,
  K_COUNT
};
extern const char* const kKernelNames[K_COUNT];

struct KernelTimer;
extern thread_local KernelTimer* g_timer;  // set by the API for the duration of a call
// A TimedLaunch scope names the kernel of the one launch inside it.  With a
// timer on, that launch (moe_launch) has the runtime record the kernel's own
// start and stop on a pair of the timer's events (hipExtLaunchKernel: the
// dispatch's timestamps, no event packets queued between kernels), so a
// kernel's time excludes its dispatch and the kernels around it overlap as
// they do untimed.
void timer_open(int id);
void timer_close();
bool timer_take(hipEvent_t* start, hipEvent_t* stop);  // the open scope's pair, once

struct TimedLaunch {
  TimedLaunch(int id, hipStream_t) {
    if (g_timer) timer_open(id);
  }
  ~TimedLaunch() {
    if (g_timer) timer_close();
  }
};

// Every kernel launch of the library.
template <typename... Args, typename F = void (*)(Args...)>
inline void moe_launch(F kernel, const dim3& grid, const dim3& block, uint32_t shmem,
                       hipStream_t s, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_timer && timer_take(&a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, a, b, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.
// mask: [E] uint8 device array (nonzero = the expert may be selected) or NULL
hipError_t launch_router(int router, const float* x, const float* wr, const float* bias,
                         const uint8_t* mask, int T,
                         int d, int E, int k, float scale, int32_t* idx, float* w,
                         float* partial, hipStream_t s);
// The previous layer's pending output (moe_forward_chained) that the logits
// launch sums into this layer's input x_out before multiplying it.
struct ChainIn {
  const float* rows;      // [T*k][d], (token, slot) order
  const float* shared;    // [T][d] or NULL
  const float* w;         // [T][k]
  const float* residual;  // [T][d] or NULL
  int k;
  float* x_out;           // [T][d]
};
// Logits, then one launch for the selection and the x encoding (xq/xs, see
// the FFN workspace), which replaces the FFN's own encoding when every expert
// set of the layer reads the same digits.  No permutation: up to kSmallT
// tokens the FFN groups the pairs itself (FfnSet::pairs_idx), beyond that
// launch_permute follows.  chain non-NULL (T <= 16): the logits launch first
// forms x, the previous layer's pending output, into chain->x_out, and x is
// ignored (hipErrorInvalidValue for T > 16 or chain->k outside [1, 16]).
// logits_only: the logits launch alone, which then clears split_cnt; the
// one-token FFN launch selects and encodes for itself (SelIn).
hipError_t launch_router_encode(int router, const float* x, const float* wr, const float* bias,
                                const uint8_t* mask,
                                int T, int d, int E, int k, float scale, int32_t* idx, float* w,
                                float* partial, int8_t* xq, float* xs, bool perm,
                                int* split_cnt, hipStream_t s, const ChainIn* chain = nullptr,
                                bool logits_only = false);
// One token whose selection and x digits the gate/up launch makes itself
// (launch_ffn_quant, sel non-NULL): every workgroup of the routed set ranks
// the experts from the logit slices as the router's selection kernel does,
// the launch's first workgroup stores topk_idx and topk_w for the down launch
// and the combine, and every workgroup encodes the token's row of x into LDS.
struct SelIn {
  const float* partial;  // logit slices [nchunk][1][E]
  int nchunk;
  const float* bias;     // selection bias [E] or NULL
  const uint8_t* mask;   // allowed experts [E] or NULL
  int E, k, router;
  float scale;
  const float* x;        // the token's row [d]
  int32_t* idx;          // [k] out
  float* w;              // [k] out
  bool perm;             // int4 digit order
};
// counts[e] += number of topk_idx entries equal to e (entries outside [0, E) skipped)
hipError_t launch_expert_counts(const int32_t* idx, long long n, int E, unsigned long long* counts,
                                hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* row_token, int32_t* token_row, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);
// (split_cnt, if not NULL: the kSplitSlots split-K counters, cleared here so
// that the FFN launches after this one find them zero)
hipError_t launch_encode_rows(const float* v, int n, int K, int8_t* q, float* sig, bool perm,
                              int* split_cnt, hipStream_t s);
// Encodes x (unless x_encoded) and runs gate/up then down for 1 or 2 expert
// sets (same format) in one pair of launches.
hipError_t launch_ffn_quant(const FfnSet* sets, int nsets, int d, const float* x, int T,
                            const FfnWs& ws, bool x_encoded, hipStream_t s,
                            const SelIn* sel = nullptr);
void set_device_info(int cu_count);
int device_cu_count();

// Attainable-peak probes (probe.hip): a streaming read of `bytes` (a multiple
// of 16) and `iters` rounds of 32 int8 MFMAs per wavefront (shape 0: 16x16x64,
// 1: 32x32x32), each over `blocks` workgroups of 256 threads; sink >= 16 bytes.
hipError_t launch_probe_read(const void* buf, size_t bytes, int blocks, void* sink,
                             hipStream_t s);
// Expert restriction (restrict.hip): kept ids ascending in keep[0..n-1], -1
// after, n in *n_keep; E <= kMaxE.
hipError_t launch_coverage_set(const unsigned long long* counts, int E, double cover, int k,
                               int32_t* keep, int32_t* n_keep, hipStream_t s);
hipError_t launch_probe_mfma(int shape, int iters, int blocks, void* sink, hipStream_t s);
// Row-major codes [nrows][K] (int4: K/2 bytes per row) -> tiled layout.
hipError_t launch_tile_weights(int fmt, const void* src, void* dst, long long nrows, int K,
                               hipStream_t s);
hipError_t launch_ffn_f32(const float* wgu, const float* wdn, int E, int d, int inter,
                          const float* x, int T, const int32_t* row_token,
                          const int32_t* offsets, int R, float* rows_out, float* h, int act,
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

// PREFETCH: load every offset (E <= 512) before the scan (see below); kernels
// whose registers are tight and that rarely scan leave it off.
template <bool PREFETCH = true>
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
  // Up to kFastChunks chunks of 64 experts, every offset is loaded before the
  // scan starts (unconditionally, indices clamped to the E + 1 offsets): one
  // trip to memory instead of one per chunk.
  constexpr int kFastChunks = 8;
  int pre_st[kFastChunks], pre_en[kFastChunks];
  const bool fast = PREFETCH && E <= kFastChunks * kWave;
  if (fast) {
#pragma unroll
    for (int c = 0; c < kFastChunks; ++c) {
      const int e = c * kWave + lane;
      pre_st[c] = offsets[e < E ? e : E];
      pre_en[c] = offsets[e + 1 < E ? e + 1 : E];
    }
  }
  int base = 0;
  for (int c0 = 0; c0 < E; c0 += kWave) {
    const int e = c0 + lane;
    int start = 0, cnt = 0;
    if (fast) {
      int st = 0, en = 0;
#pragma unroll
      for (int c = 0; c < kFastChunks; ++c)
        if (c * kWave == c0) {
          st = pre_st[c];
          en = pre_en[c];
        }
      start = st;
      cnt = e < E ? en - st : 0;
    } else if (e < E) {
      start = offsets[e];
      cnt = offsets[e + 1] - start;
    }
    if (cnt < 0) cnt = 0;
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

// The activations use the hardware's single-instruction exp2 and reciprocal
// (v_exp_f32, v_rcp_f32, about 1 ulp each): a few instructions per value
// where the library exp and an IEEE division take about thirty, which
// dominated the epilogues of the FFN kernels.  Relative error about 3e-7.
constexpr float kLog2e = 1.4426950408889634f;
__device__ inline float exp_approx(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// SiLU: z / (1 + e^-z)
__device__ inline float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + exp_approx(-z)); }
// GELU, tanh form: z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))), with
// tanh u = 1 - 2 / (1 + e^(2u)) (exact at both tails: e^(2u) -> 0 or inf).
__device__ inline float gelu_tanh_f(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float u = c * (z + 0.044715f * z * z * z);
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + exp_approx(2.0f * u));
  return 0.5f * z * (1.0f + t);
}
// Gate activation of the SwiGLU-style FFN: 0 = silu, 1 = gelu_tanh.
__device__ inline float act_f(int act, float z) { return act == 1 ? gelu_tanh_f(z) : silu_f(z); }

// ---- two-digit int8 encoding of fp32 activations (used by the FFN kernels)
// v = 2^-p (d0 + d1/256) + e, |e| <= 2^-p / 512, d0, d1 in [-127, 127], with p
// chosen per set of values so that max|v| * 2^p lies in (63.5, 127].
// p such that max|v| * 2^p lies in (63.5, 127]; 0 for an all-zero set.
__device__ inline int digit_exponent(float m) {
  if (!(m > 0.0f)) return 0;
  int ex;
  frexpf(m, &ex);  // m = f * 2^ex, f in [0.5, 1)
  int p = 7 - ex;
  if (ldexpf(m, p) > 127.0f) p -= 1;
  return p;
}

__device__ inline void two_digits(float v, int p, int& d0, int& d1) {
  const float a = ldexpf(v, p);
  const float f0 = fminf(fmaxf(rintf(a), -127.0f), 127.0f);
  const float f1 = fminf(fmaxf(rintf((a - f0) * 256.0f), -127.0f), 127.0f);
  d0 = (int)f0;
  d1 = (int)f1;
}

__device__ inline unsigned pack4(int a, int b, int c, int d) {
  return (unsigned)(a & 0xff) | ((unsigned)(b & 0xff) << 8) | ((unsigned)(c & 0xff) << 16) |
         ((unsigned)(d & 0xff) << 24);
}

// Digit bytes of 8 consecutive values v[0..7] (two float4), as two 8-byte
// words (d0 digits, d1 digits).  perm = false: natural order.  perm = true:
// (0, 2, 4, 6, 1, 3, 5, 7), the order within each group of 8 that the int4
// FFN kernels read: their weight unpacking leaves even and odd codes in
// separate words, and the activations must line up with them (ffn.hip,
// int4).  The int4 order also moves the groups inside each 128-wide span
// (int4_digit_chunk), so that a lane's four groups of a span are contiguous.
__device__ inline void encode8(const float4& a, const float4& b, int p, bool perm, uint2& w0,
                               uint2& w1) {
  int x[8], y[8];
  two_digits(a.x, p, x[0], y[0]);
  two_digits(a.y, p, x[1], y[1]);
  two_digits(a.z, p, x[2], y[2]);
  two_digits(a.w, p, x[3], y[3]);
  two_digits(b.x, p, x[4], y[4]);
  two_digits(b.y, p, x[5], y[5]);
  two_digits(b.z, p, x[6], y[6]);
  two_digits(b.w, p, x[7], y[7]);
  if (perm) {
    w0 = make_uint2(pack4(x[0], x[2], x[4], x[6]), pack4(x[1], x[3], x[5], x[7]));
    w1 = make_uint2(pack4(y[0], y[2], y[4], y[6]), pack4(y[1], y[3], y[5], y[7]));
  } else {
    w0 = make_uint2(pack4(x[0], x[1], x[2], x[3]), pack4(x[4], x[5], x[6], x[7]));
    w1 = make_uint2(pack4(y[0], y[1], y[2], y[3]), pack4(y[4], y[5], y[6], y[7]));
  }
}

// The int4 digit order of a row: group c (elements 8c..8c+7) of span c / 16
// is group j = 4q + g of its span (q = block of 32, g = group within the
// block); it moves to place 4g + q, so that lane group g of an MFMA finds its
// four blocks' groups in 32 contiguous bytes; inside the group the order is
// encode8's.  int4_digit_chunk gives the group's new index, int4_digit_pos an
// element's new byte position.
__device__ inline int int4_digit_chunk(int c) {
  return (c & ~15) | ((c & 3) << 2) | ((c >> 2) & 3);
}
__device__ inline int int4_digit_pos(int k) {
  return 8 * int4_digit_chunk(k >> 3) | ((k & 7) >> 1) | ((k & 1) << 2);
}

// One wavefront encodes one row of K values (K % 8 == 0; K % 128 == 0 with
// perm): q = [d0 x K | d1 x K], *sig = 2^-p (0 for an all-zero row); perm: the
// int4 digit order (encode8, int4_digit_chunk).
__device__ inline void encode_row(const float* __restrict__ row, int K, int8_t* __restrict__ q,
                                  float* __restrict__ sig, bool perm) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = 0.0f;
  for (int c = lane; c < K / 4; c += kWave) {
    const float4 a = *reinterpret_cast<const float4*>(row + 4 * c);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  const int p = digit_exponent(m);
  uint2* q0 = reinterpret_cast<uint2*>(q);
  uint2* q1 = reinterpret_cast<uint2*>(q + K);
  for (int c = lane; c < K / 8; c += kWave) {
    const float4 a = *reinterpret_cast<const float4*>(row + 8 * c);
    const float4 b = *reinterpret_cast<const float4*>(row + 8 * c + 4);
    uint2 w0, w1;
    encode8(a, b, p, perm, w0, w1);
    const int dst = perm ? int4_digit_chunk(c) : c;
    q0[dst] = w0;
    q1[dst] = w1;
  }
  if (lane == 0) *sig = m > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
}

#endif

// ---------------------------------------------------------------- weight quantizers (quant.hip)
// fmt 1 = int8 per row, 2 = int4 blocks of 32; in_type 0 = fp32, 1 = bf16.
hipError_t launch_quantize(int fmt, int in_type, const void* w, long long rows, int K,
                           void* codes, float* scales, hipStream_t st);

}  // namespace moe
