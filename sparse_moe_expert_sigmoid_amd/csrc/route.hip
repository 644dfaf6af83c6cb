// Router: logits, selection and weights for every token.
//
// Sigmoid router (Kimi-Linear LiteRT-LM DETAILS.md, Conversion notes, the
// mixture-of-experts bullet): s = sigmoid(l), top k on s + bias, weights
// s / sum(s) times a scale (2.446).  Softmax router (Qwen3-30B-A3B LiteRT card,
// Conversion Notes): p = softmax(l), top k on p, weights p / sum(p).
//
// Two kernels.  The first writes partial logits, each a sum over a fixed
// 256-wide slice of the input on the matrix cores in one fixed order; the
// second adds the slices in order, so a token's logits never depend on T or on
// the launch shape.
// The second kernel runs one workgroup per token and ranks the selection keys
// by counting in two rounds (no sequential arg-max rounds; select.h).  For one
// token whose expert sets all read digits, the gate/up launch runs that
// selection itself and only the first kernel runs here (logits_only).
#include "internal.h"
#include "select.h"

namespace moe {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// partial[c][t][e] = sum over i in [256c, 256c + 256) of Wr[e][i] * x[t][i] on
// the fp32 matrix cores (v_mfma_f32_16x16x4_f32, 16 experts x 16 tokens x 4
// inputs per instruction).  Step s of a slice multiplies inputs 4s .. 4s + 3:
// lane quarter q (lane / 16) carries input 4s + q of weight row lane % 16 (A)
// and of token lane % 16 (B).  Step s goes to accumulator chain s % 4 and the
// slice's value is (chain 0 + chain 1) + (chain 2 + chain 3).  Both kernels
// below run exactly this sequence for every output, and a product of the
// instruction depends only on its own row and column, so a token's logits do
// not depend on T or on where its row and expert sit in a tile.  d is a
// multiple of 64 (checked on the host), so a slice has a multiple of 16 steps.
__device__ inline void logit_steps4(const float4& a, const float4& b, v4f acc[4]) {
  acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc[0], 0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc[1], 0, 0, 0);
  acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc[2], 0, 0, 0);
  acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc[3], 0, 0, 0);
}

// Store one 16x16 block: lane l holds experts eb + 4 (l / 16) + r (r = 0..3)
// of token tb + l % 16.
__device__ inline void logit_store(const v4f& v, int eb, int tb, int lane, int c, int T, int E,
                                   float* __restrict__ partial) {
  const int t = tb + (lane & 15);
  const int e = eb + 4 * (lane >> 4);
  if (t >= T) return;
  float* dst = partial + ((size_t)c * T + t) * E + e;
  if ((E & 3) == 0 && e + 3 < E) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e + r < E) dst[r] = v[r];
  }
}

// One chain of N steps on operands already in registers.
template <int N>
__device__ __forceinline__ v4f logit_chain(const float* a, const float* b) {
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < N; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], acc, 0, 0, 0);
  return acc;
}

// Small batches (T <= 32): one workgroup per 16 experts x 16 tokens x slice,
// wavefront h running chain h (steps h, h + 4, ...), its operands loaded
// straight into registers (one trip to memory); the chains meet in LDS.
__global__ __launch_bounds__(256) void router_logits_small_kernel(const float* __restrict__ x,
                                                                  const float* __restrict__ wr,
                                                                  int T, int d, int E,
                                                                  float* __restrict__ partial,
                                                                  int* __restrict__ split_cnt) {
  if (split_cnt) {  // (logits-only launches) the FFN launches that follow start from zero counters
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    const int b = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    for (int q = b * blockDim.x + threadIdx.x; q < kSplitSlots; q += nb * blockDim.x) split_cnt[q] = 0;
  }
  constexpr int kChainSteps = kRouterChunk / 16;  // steps per chain in a whole slice
  __shared__ v4f chain_sm[4][kWave];
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16, c = blockIdx.z;
  const int kbeg = c * kRouterChunk;
  const int nm = min(kRouterChunk, d - kbeg) / 16;  // steps per chain in this slice
  const int h = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, q = lane >> 4;
  // step s = h + 4m multiplies input 4s + q = 4h + 16m + q
  const float* wa = wr + (size_t)min(e0 + i, E - 1) * d + kbeg + 4 * h + q;
  const float* xb = x + (size_t)min(t0 + i, T - 1) * d + kbeg + 4 * h + q;
  float a[kChainSteps], b[kChainSteps];
#pragma unroll
  for (int m = 0; m < kChainSteps; ++m) {
    const int mc = min(m, nm - 1);
    a[m] = wa[16 * mc];
    b[m] = xb[16 * mc];
  }
  // a slice holds 4, 8, 12 or 16 steps per chain (d is a multiple of 64)
  const v4f acc = nm == 16  ? logit_chain<16>(a, b)
                  : nm == 12 ? logit_chain<12>(a, b)
                  : nm == 8  ? logit_chain<8>(a, b)
                             : logit_chain<4>(a, b);
  chain_sm[h][lane] = acc;
  __syncthreads();
  if (h != 0) return;
  const v4f c0 = chain_sm[0][lane], c1 = chain_sm[1][lane];
  const v4f c2 = chain_sm[2][lane], c3 = chain_sm[3][lane];
  v4f v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = (c0[r] + c1[r]) + (c2[r] + c3[r]);
  logit_store(v, e0, t0, lane, c, T, E, partial);
}

// Chained layers (T <= 16, moe_forward_chained): the previous layer's output
// is still pending as its rows, and this launch forms the x slice it needs as
// the combine would (the k weighted rows in slot order by fused
// multiply-adds, then the shared row, then the residual), one element per
// thread with all of its loads in flight, into LDS; the workgroups of expert
// block 0 also store the slice as the layer's input.  The logits then follow
// the small kernel's chains exactly, with the x operand read from LDS, so
// they equal an unchained call's bit for bit.
template <int KMAX>
__global__ __launch_bounds__(256) void router_logits_chain_kernel(ChainIn ch,
                                                                  const float* __restrict__ wr,
                                                                  int T, int d, int E,
                                                                  float* __restrict__ partial,
                                                                  int* __restrict__ split_cnt) {
  if (split_cnt) {  // (logits-only launches) the FFN launches that follow start from zero counters
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    const int b = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    for (int q = b * blockDim.x + threadIdx.x; q < kSplitSlots; q += nb * blockDim.x) split_cnt[q] = 0;
  }
  constexpr int kChainSteps = kRouterChunk / 16;
  __shared__ float x_sm[16][kRouterChunk];
  __shared__ v4f chain_sm[4][kWave];
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16, c = blockIdx.z;
  const int kbeg = c * kRouterChunk;
  const int width = min(kRouterChunk, d - kbeg);
  const int nt = min(16, T - t0);
  const int nm = width / 16;  // steps per chain in this slice
  const int h = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, q4 = lane >> 4;
  // the router rows do not depend on x: their loads go out first, and their
  // latency overlaps the sum below
  const float* wa = wr + (size_t)min(e0 + i, E - 1) * d + kbeg + 4 * h + q4;
  float a[kChainSteps], b[kChainSteps];
#pragma unroll
  for (int m = 0; m < kChainSteps; ++m) a[m] = wa[16 * min(m, nm - 1)];
  for (int q = threadIdx.x; q < nt * width; q += blockDim.x) {
    const int tl = q / width, col = kbeg + q % width, t = t0 + tl;
    const size_t o = (size_t)t * d + col;
    float v[KMAX], wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int jj = j < ch.k ? j : 0;
      v[j] = ch.rows[(size_t)(t * ch.k + jj) * d + col];
      wj[j] = ch.w[(size_t)t * ch.k + jj];
    }
    const float shv = ch.shared ? ch.shared[o] : 0.0f;
    const float rsv = ch.residual ? ch.residual[o] : 0.0f;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) acc = fmaf(j < ch.k ? wj[j] : 0.0f, v[j], acc);
    if (ch.shared) acc += shv;
    if (ch.residual) acc += rsv;
    x_sm[tl][q % width] = acc;
    if (blockIdx.x == 0) ch.x_out[o] = acc;
  }
  __syncthreads();
  const float* xb = &x_sm[min(i, nt - 1)][4 * h + q4];
#pragma unroll
  for (int m = 0; m < kChainSteps; ++m) b[m] = xb[16 * min(m, nm - 1)];
  const v4f acc = nm == 16  ? logit_chain<16>(a, b)
                  : nm == 12 ? logit_chain<12>(a, b)
                  : nm == 8  ? logit_chain<8>(a, b)
                             : logit_chain<4>(a, b);
  chain_sm[h][lane] = acc;
  __syncthreads();
  if (h != 0) return;
  const v4f c0 = chain_sm[0][lane], c1 = chain_sm[1][lane];
  const v4f c2 = chain_sm[2][lane], c3 = chain_sm[3][lane];
  v4f v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = (c0[r] + c1[r]) + (c2[r] + c3[r]);
  logit_store(v, e0, t0, lane, c, T, E, partial);
}

// Larger batches: 64 experts x 64 tokens per workgroup, wavefront w owning
// experts 32 (w & 1) .. + 31 and tokens 32 (w >> 1) .. + 31 (2 x 2 blocks, 4
// chains each).  The slice moves through LDS 16 steps (64 inputs) at a time
// as planes [q][row][step]: one 16-byte read gives a lane 4 consecutive steps.
// Two groups of 64 inputs are in flight in registers while the current one is
// multiplied (one group ahead left the loads about one MFMA phase to land).
constexpr int kLtSteps = 16;           // steps staged at a time
constexpr int kLtLd = kLtSteps + 4;    // row stride in floats (16-byte aligned, conflict-free)

__global__ __launch_bounds__(256) void router_logits_tile_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ wr,
                                                                 int T, int d, int E,
                                                                 float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) float wl[4][64][kLtLd];
  __shared__ __attribute__((aligned(16))) float xl[4][64][kLtLd];
  const int e0 = blockIdx.x * 64, t0 = blockIdx.y * 64, c = blockIdx.z;
  const int kbeg = c * kRouterChunk;
  const int nsub = min(kRouterChunk, d - kbeg) / (4 * kLtSteps);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, q = lane >> 4;
  const int er = 32 * (wave & 1), tr = 32 * (wave >> 1);
  // this thread's loads: rows (threadIdx.x + 256 u) / 16, step (threadIdx.x % 16)
  const float* wsrc[4];
  const float* xsrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int f = threadIdx.x + 256 * u, row = f >> 4, st = f & 15;
    wsrc[u] = wr + (size_t)min(e0 + row, E - 1) * d + kbeg + 4 * st;
    xsrc[u] = x + (size_t)min(t0 + row, T - 1) * d + kbeg + 4 * st;
  }
  // two groups of 64 inputs in flight in registers (wv[g], xv[g] hold group
  // sub with sub % 2 == g); a slice has at most 4 groups, so the loop unrolls
  float4 wv[2][4], xv[2][4];
  constexpr int kGrp = 4 * kLtSteps;  // inputs per group
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int nx = (g < nsub ? g : nsub - 1) * kGrp;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wv[g][u] = *reinterpret_cast<const float4*>(wsrc[u] + nx);
      xv[g][u] = *reinterpret_cast<const float4*>(xsrc[u] + nx);
    }
  }
  v4f acc[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int h = 0; h < 4; ++h) acc[a][b][h] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int sub = 0; sub < kRouterChunk / kGrp; ++sub) {
    if (sub < nsub) {
      const int g = sub & 1;
      if (sub > 0) __syncthreads();  // every read of the previous 16 steps is done
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = threadIdx.x + 256 * u, row = f >> 4, st = f & 15;
        wl[0][row][st] = wv[g][u].x;
        wl[1][row][st] = wv[g][u].y;
        wl[2][row][st] = wv[g][u].z;
        wl[3][row][st] = wv[g][u].w;
        xl[0][row][st] = xv[g][u].x;
        xl[1][row][st] = xv[g][u].y;
        xl[2][row][st] = xv[g][u].z;
        xl[3][row][st] = xv[g][u].w;
      }
      __syncthreads();
      {  // the group after next (past the end: the last group again, unused)
        const int nx = (sub + 2 < nsub ? sub + 2 : nsub - 1) * kGrp;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wv[g][u] = *reinterpret_cast<const float4*>(wsrc[u] + nx);
          xv[g][u] = *reinterpret_cast<const float4*>(xsrc[u] + nx);
        }
      }
#pragma unroll
      for (int s4 = 0; s4 < kLtSteps / 4; ++s4) {
        float4 av[2], bv[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
          av[a] = *reinterpret_cast<const float4*>(&wl[q][er + 16 * a + i][4 * s4]);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          bv[b] = *reinterpret_cast<const float4*>(&xl[q][tr + 16 * b + i][4 * s4]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) logit_steps4(av[a], bv[b], acc[a][b]);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      v4f v;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[r] = (acc[a][b][0][r] + acc[a][b][1][r]) + (acc[a][b][2][r] + acc[a][b][3][r]);
      logit_store(v, e0 + er + 16 * a, t0 + tr + 16 * b, lane, c, T, E, partial);
    }
}

// One workgroup per token.
template <int EPT>
__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ partial,
                                                            int nchunk,
                                                            const float* __restrict__ bias,
                                                            const uint8_t* __restrict__ mask,
                                                            int T, int E, int k, int router,
                                                            float scale,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ w) {
  __shared__ unsigned long long keys[256 * EPT];
  __shared__ float red[4];
  __shared__ float sel_s[kMaxK];
  select_token<EPT>(partial, nchunk, bias, mask, T, E, k, router, scale, blockIdx.x, true,
                    threadIdx.x,
                    keys, red, sel_s, idx, w, nullptr);
}

template <int EPT>
hipError_t launch_select(const float* partial, int nchunk, const float* bias,
                         const uint8_t* mask, int T, int E, int k,
                         int router, float scale, int32_t* idx, float* w, hipStream_t s) {
  TimedLaunch tl(K_ROUTER_TOPK, s);
  moe_launch(router_select_kernel<EPT>, dim3(T), dim3(256), 0, s, partial, nchunk, bias,
                     mask,
                     T, E, k, router, scale, idx, w);
  return hipGetLastError();
}

// ------------------------------------------------------------------ selection + encoding
// After the logits kernel, one workgroup per token selects that token's
// experts (select_token) and encodes its row of x as two-digit int8 for the
// FFN kernels (which, for small batches, then group the (token, slot) pairs
// themselves; larger batches are permuted first).
template <int EPT>
__global__ __launch_bounds__(256) void router_tail_kernel(
    const float* __restrict__ partial, int nchunk, const float* __restrict__ x, int d,
    const float* __restrict__ bias, const uint8_t* __restrict__ mask, int T, int E, int k,
    int router, float scale,
    int32_t* __restrict__ idx, float* __restrict__ w, int8_t* __restrict__ xq,
    float* __restrict__ xs, bool perm, int* __restrict__ split_cnt) {
  __shared__ unsigned long long keys[256 * EPT];
  if (split_cnt)  // the FFN launches that follow start from zero counters
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < kSplitSlots; q += gridDim.x * blockDim.x)
      split_cnt[q] = 0;
  __shared__ float red[4];
  __shared__ float xred[4];
  __shared__ float sel_s[kMaxK];
  const int t = blockIdx.x;
  const float* row = x + (size_t)t * d;
  // the token's row of x (up to 4096 values, in groups of 8 per thread) goes
  // into registers first, so its loads are in flight during the selection
  constexpr int kXPer = 2;
  const int n8 = d / 8;
  const bool in_regs = n8 <= kXPer * 256;
  float4 xv[kXPer][2];
#pragma unroll
  for (int m = 0; m < kXPer; ++m) {
    const int c = threadIdx.x + 256 * m;
    const bool ok = in_regs && c < n8;
    xv[m][0] = ok ? *reinterpret_cast<const float4*>(row + 8 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    xv[m][1] = ok ? *reinterpret_cast<const float4*>(row + 8 * c + 4)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  select_token<EPT>(partial, nchunk, bias, mask, T, E, k, router, scale, t, true, threadIdx.x,
                    keys,
                    red, sel_s, idx, w, nullptr);
  if (!in_regs) {
    if (threadIdx.x < kWave) encode_row(row, d, xq + (size_t)t * 2 * d, xs + t, perm);
    return;
  }
  // two-digit encoding of the row with one scale (as encode_row), by all threads
  float mx = 0.0f;
#pragma unroll
  for (int m = 0; m < kXPer; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[m][h].x), fabsf(xv[m][h].y)),
                           fmaxf(fabsf(xv[m][h].z), fabsf(xv[m][h].w))));
  mx = wave_max_f(mx);
  if ((threadIdx.x & (kWave - 1)) == 0) xred[threadIdx.x / kWave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(xred[0], xred[1]), fmaxf(xred[2], xred[3]));
  const int p = digit_exponent(mx);
  uint2* q0 = reinterpret_cast<uint2*>(xq + (size_t)t * 2 * d);
  uint2* q1 = reinterpret_cast<uint2*>(xq + (size_t)t * 2 * d + d);
#pragma unroll
  for (int m = 0; m < kXPer; ++m) {
    const int c = threadIdx.x + 256 * m;
    if (c >= n8) continue;
    uint2 w0, w1;
    encode8(xv[m][0], xv[m][1], p, perm, w0, w1);
    const int dst = perm ? int4_digit_chunk(c) : c;
    q0[dst] = w0;
    q1[dst] = w1;
  }
  if (threadIdx.x == 0) xs[t] = mx > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
}

template <int EPT>
hipError_t launch_tail(const float* partial, int nchunk, const float* x, int d, const float* bias,
                       const uint8_t* mask,
                       int T, int E, int k, int router, float scale, int32_t* idx, float* w,
                       int8_t* xq, float* xs, bool perm, int* split_cnt, hipStream_t s) {
  TimedLaunch tl(K_ROUTER_TAIL, s);
  moe_launch(router_tail_kernel<EPT>, dim3(T), dim3(256), 0, s, partial, nchunk, x, d,
                     bias, mask, T, E, k, router, scale, idx, w, xq, xs, perm, split_cnt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(int router, const float* x, const float* wr, const float* bias,
                         const uint8_t* mask, int T,
                         int d, int E, int k, float scale, int32_t* idx, float* w,
                         float* partial, hipStream_t s) {
  const int nchunk = (d + kRouterChunk - 1) / kRouterChunk;
  {
  TimedLaunch tl(K_ROUTER_LOGITS, s);
  if (T <= 32) {
    dim3 grid((E + 15) / 16, (T + 15) / 16, nchunk);
    moe_launch(router_logits_small_kernel, grid, dim3(256), 0, s, x, wr, T, d, E,
                       partial, nullptr);
  } else {
    dim3 grid((E + 63) / 64, (T + 63) / 64, nchunk);
    moe_launch(router_logits_tile_kernel, grid, dim3(256), 0, s, x, wr, T, d, E,
                       partial);
  }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (E <= 256)
    return launch_select<1>(partial, nchunk, bias, mask, T, E, k, router, scale, idx, w, s);
  if (E <= 512)
    return launch_select<2>(partial, nchunk, bias, mask, T, E, k, router, scale, idx, w, s);
  return launch_select<4>(partial, nchunk, bias, mask, T, E, k, router, scale, idx, w, s);
}

hipError_t launch_router_encode(int router, const float* x, const float* wr, const float* bias,
                                const uint8_t* mask,
                                int T, int d, int E, int k, float scale, int32_t* idx, float* w,
                                float* partial, int8_t* xq, float* xs, bool perm,
                                int* split_cnt, hipStream_t s, const ChainIn* chain,
                                bool logits_only) {
  const int nchunk = (d + kRouterChunk - 1) / kRouterChunk;
  if (chain) {
    if (T > 16 || chain->k < 1 || chain->k > kMaxK) return hipErrorInvalidValue;
    x = chain->x_out;  // the selection encodes the formed input
  }
  {
    TimedLaunch tl(K_ROUTER_LOGITS, s);
    if (chain) {
      dim3 grid((E + 15) / 16, 1, nchunk);
      int* cnt = logits_only ? split_cnt : nullptr;
      if (chain->k <= 8)
        moe_launch(router_logits_chain_kernel<8>, grid, dim3(256), 0, s, *chain, wr, T, d, E,
                   partial, cnt);
      else
        moe_launch(router_logits_chain_kernel<kMaxK>, grid, dim3(256), 0, s, *chain, wr, T, d,
                   E, partial, cnt);
    } else if (T <= 32) {
      dim3 grid((E + 15) / 16, (T + 15) / 16, nchunk);
      moe_launch(router_logits_small_kernel, grid, dim3(256), 0, s, x, wr, T, d, E,
                         partial, logits_only ? split_cnt : nullptr);
    } else {
      if (logits_only) return hipErrorInvalidValue;  // (one token only)
      dim3 grid((E + 63) / 64, (T + 63) / 64, nchunk);
      moe_launch(router_logits_tile_kernel, grid, dim3(256), 0, s, x, wr, T, d, E,
                         partial);
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || logits_only) return err;
  if (E <= 256)
    return launch_tail<1>(partial, nchunk, x, d, bias, mask, T, E, k, router, scale, idx, w, xq,
                          xs, perm, split_cnt, s);
  if (E <= 512)
    return launch_tail<2>(partial, nchunk, x, d, bias, mask, T, E, k, router, scale, idx, w, xq,
                          xs, perm, split_cnt, s);
  return launch_tail<4>(partial, nchunk, x, d, bias, mask, T, E, k, router, scale, idx, w, xq,
                          xs, perm, split_cnt, s);
}

}  // namespace moe
