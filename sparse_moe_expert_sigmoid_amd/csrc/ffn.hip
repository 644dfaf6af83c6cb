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
// the MFMA A operand as stored (no dequantisation to floating point); the
// fp32 activations are written as two int8 digits against a power-of-two
// scale, v = 2^-p (d0 + d1/256), so that
//   sum_k q_k v_k = 2^-p (sum_k q_k d0_k + 2^-8 sum_k q_k d1_k)
// is two exact int32 MFMA accumulations.  The encoding error is at most
// 2^-16 of the largest |v| sharing the scale.  x uses one scale per row; h
// uses one scale per row and 64-column block (128-column block on the
// prefill GEMM path), chosen in the gate/up epilogue (so h never exists in
// fp32 memory and no separate pass is needed); the down projection folds each
// block's int32 sums into fp32 with that block's scale.
//
// Work split: a tile is up to 16 rows of one expert (the MFMA N side); a
// workgroup owns 64 output columns of one tile, one wavefront per 16 columns
// (the MFMA M side), optionally KS wavefronts per 16 columns each taking a
// K slice (int32 partial sums are added exactly).  Weight rows stream from
// HBM with 16-byte loads, each byte read once per tile; activation digits are
// read straight from L2 (no LDS staging, so occupancy is set by registers
// only).  Tiles are found on the device from the expert offsets, so no count
// is copied back to the host; the routed and the shared expert can share one
// launch (group 0 and group 1 below).
#include <algorithm>

#include "internal.h"
#include "select.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef long v2l __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// A load through a pointer the compiler knows to be global.  Where a kernel
// mixes LDS and global pointers the address-space inference can give up and
// emit flat loads, which also count against the LDS wait counter: every wait
// for an LDS read then waits for the weight stream as well.
template <class T>
__device__ inline T gload(const void* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ inline T gload_nt(const void* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)p);
}

// One wavefront per row (see encode_row).
__global__ __launch_bounds__(256) void encode_rows_kernel(const float* __restrict__ v, int n,
                                                          int K, int8_t* __restrict__ q,
                                                          float* __restrict__ sig, bool perm,
                                                          int* __restrict__ split_cnt) {
  if (split_cnt)  // the FFN launches that follow start from zero counters
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < kSplitSlots; c += gridDim.x * blockDim.x)
      split_cnt[c] = 0;
  const int r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= n) return;
  encode_row(v + (size_t)r * K, K, q + (size_t)r * 2 * K, sig + r, perm);
}

// ------------------------------------------------------------------ work items
// Group 0: routed experts (rows grouped by `offsets`, rows read token
// row_token[r]); group 1: optional second expert set, e.g. the shared expert
// (one expert, identity rows).  Tiles of group 1 follow group 0's.
struct Group {
  int E, inter, R, tiles;
  const void* wgu;
  const float* sgu;
  const void* wdn;
  const float* sdn;
  const int32_t* row_token;  // NULL = identity
  const int32_t* offsets;    // NULL = one expert over R rows
  int8_t* hq;                // [R][2][inter]
  float* hs;                 // [R][inter/64]
  float* out;                // [R][d]
  const int32_t* pairs_idx;  // non-NULL: group the R = T*k pairs of topk_idx [T][k] on the fly
  int k;
  int act;                   // gate activation: 0 silu, 1 gelu (tanh form)
};

struct Job {
  int g, e, r0, nr;
};

// K split across the workgroups of one work unit.  Each writes its partial
// sums to its slot; the last to arrive (by an atomic count) adds every slot in
// workgroup order, so the result does not depend on arrival order, clears the
// count for the next launch and goes on to the epilogue.  The two expert sets
// of a launch split n0 and n1 ways: the grid's y range holds group 0's tiles
// n0 times each, then group 1's n1 times each (virtual tiles).
struct SplitK {
  int n0, n1;  // workgroups per unit of group 0 / group 1 (1: no split)
  int* cnt;    // one arrival count per unit, zero before the launch
  float* part; // kSplitSlotBytes per (unit, workgroup) of the units that split
};

// Where virtual tile v (unit column x of gx) sits: its real tile, its K-split
// index and count, and its unit's first join slot (group 0's units take slots
// first when they split, then group 1's).
struct SplitPos {
  int tile, kw, n, slot0;
};
__device__ inline SplitPos split_pos(const SplitK& sk, int v, int t0, int gx, int x) {
  SplitPos p;
  const int v0 = t0 * sk.n0;
  if (v < v0) {
    p.tile = v / sk.n0;
    p.kw = v % sk.n0;
    p.n = sk.n0;
    p.slot0 = (p.tile * gx + x) * sk.n0;
  } else {
    const int v1 = v - v0;
    p.tile = t0 + v1 / sk.n1;
    p.kw = v1 % sk.n1;
    p.n = sk.n1;
    p.slot0 = (sk.n0 > 1 ? t0 * gx * sk.n0 : 0) + ((p.tile - t0) * gx + x) * sk.n1;
  }
  return p;
}

// holder lanes carry N values of type V (int32 digit sums or fp32 partials);
// grp is the wavefront's index among the holders.  Returns false in every workgroup but
// the last of its unit (uniform over the workgroup); the last one returns
// with the total in v.  The slots and the count are accessed with relaxed
// device-scope atomics, which stay coherent across the XCDs' separate L2
// caches without the whole-L2 write-back and invalidation that a device-scope
// fence costs: each thread waits for its own slot stores to complete
// (vmcnt 0) before the barrier, and the count is taken after the barrier.
template <typename V, int N>
__device__ inline bool split_join(const SplitK& sk, int unit, int slot0, int kw, int n, int grp,
                                  bool holder, V* v, int* flag_sm) {
  // slot layout [grp][c][lane]: each store and load of a value is 256
  // contiguous bytes over the wavefront; grp < 4 (the column groups)
  static_assert(4 * N * kWave * sizeof(V) <= kSplitSlotBytes, "a slot holds 4 groups");
  V* base = reinterpret_cast<V*>(sk.part);
  constexpr size_t kPer = kSplitSlotBytes / sizeof(V);
  const int lane = threadIdx.x & (kWave - 1);
  const size_t at = (size_t)grp * N * kWave + lane;
  if (holder) {
    V* dst = base + (size_t)(slot0 + kw) * kPer + at;
#pragma unroll
    for (int c = 0; c < N; ++c)
      __hip_atomic_store(dst + c * kWave, v[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70 & ~0x0F70u);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    *flag_sm = __hip_atomic_fetch_add(sk.cnt + unit, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == n - 1;
  __syncthreads();
  if (!*flag_sm) return false;
  if (holder) {
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = V(0);
    for (int q = 0; q < n; ++q) {
      V* src = base + (size_t)(slot0 + q) * kPer + at;
#pragma unroll
      for (int c = 0; c < N; ++c)
        v[c] += __hip_atomic_load(src + c * kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(sk.cnt + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

__device__ inline bool find_job(const Group& g0, const Group& g1, int mt, int tile, Job& j) {
  const Group& G = tile < g0.tiles ? g0 : g1;
  const int t = tile < g0.tiles ? tile : tile - g0.tiles;
  if (tile >= g0.tiles && t >= g1.tiles) return false;
  Tile tl;
  if (!find_tile(G.offsets, G.E, G.R, mt, t, tl)) return false;
  j.g = tile < g0.tiles ? 0 : 1;
  j.e = tl.e;
  j.r0 = tl.r0;
  j.nr = tl.nr;
  return true;
}

// Workgroup-level tile lookup for the decode kernels: rows[j] is the row of
// the group's h / out arrays and toks[j] the row of x for tile row j < nr.
// Groups with pairs_idx group the T*k (token, slot) pairs of topk_idx on the
// fly (no permutation pass): per-expert counts by an LDS histogram, the tile
// by a scan over experts, its pairs by ballots in (t, j) order; the row of a
// pair is its index t*k + j, so outputs land in (token, slot) order.
__device__ inline bool find_rows(const Group& g0, const Group& g1, int mt, int tile, Job& job,
                                 int* rows, int* toks, int* hist, int* sh, bool need_toks) {
  const bool first = tile < g0.tiles;
  if (!first && tile - g0.tiles >= g1.tiles) return false;
  const Group G = first ? g0 : g1;
  const int t = first ? tile : tile - g0.tiles;
  job.g = first ? 0 : 1;
  if (G.pairs_idx == nullptr) {
    Tile tl;
    if (!find_tile<false>(G.offsets, G.E, G.R, mt, t, tl)) return false;
    job.e = tl.e;
    job.r0 = tl.r0;
    job.nr = tl.nr;
    for (int j = threadIdx.x; j < tl.nr; j += blockDim.x) {
      rows[j] = tl.r0 + j;
      if (need_toks) toks[j] = G.row_token ? G.row_token[tl.r0 + j] : tl.r0 + j;
    }
    __syncthreads();
    return true;
  }
  if (G.R == G.k && mt == 1) {
    // one token: its k experts are distinct, so tile t is slot t alone (the
    // same rows, in another tile order, as the histogram path below)
    const int e = G.pairs_idx[t];
    if (e < 0 || e >= G.E) return false;
    job.e = e;
    job.r0 = 0;
    job.nr = 1;
    if (threadIdx.x == 0) {
      rows[0] = t;
      if (need_toks) toks[0] = 0;
    }
    __syncthreads();
    return true;
  }
  const int n = G.R, E = G.E, lane = threadIdx.x & (kWave - 1);
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < n; q += blockDim.x) {
    const int e = G.pairs_idx[q];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    int base = 0, found = -1, lo = 0, cnt = 0;
    for (int c0 = 0; c0 < E && found < 0; c0 += kWave) {
      const int e = c0 + lane;
      const int ce = e < E ? hist[e] : 0;
      const int nt = (ce + mt - 1) / mt;
      int incl = nt;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      const int total = __shfl(incl, kWave - 1, kWave);
      if (t < base + total) {
        const unsigned long long m = __ballot(base + incl > t);
        const int L = __ffsll((long long)m) - 1;
        found = c0 + L;
        lo = (t - base - __shfl(incl - nt, L, kWave)) * mt;
        cnt = __shfl(ce, L, kWave);
      }
      base += total;
    }
    if (lane == 0) {
      sh[0] = found;
      sh[1] = lo;
      sh[2] = found < 0 ? 0 : min(mt, cnt - lo);
    }
  }
  __syncthreads();
  if (sh[0] < 0) return false;
  job.e = sh[0];
  job.r0 = sh[1];
  job.nr = sh[2];
  if (threadIdx.x < kWave) {
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    int rank0 = 0;
    for (int q0 = 0; q0 < n; q0 += kWave) {
      const int q = q0 + lane;
      const bool hit = q < n && G.pairs_idx[q] == job.e;
      const unsigned long long m = __ballot(hit);
      const int rk = rank0 + __popcll(m & below) - job.r0;
      if (hit && rk >= 0 && rk < job.nr) {
        rows[rk] = q;
        if (need_toks) toks[rk] = q / G.k;
      }
      rank0 += __popcll(m);
    }
  }
  __syncthreads();
  return true;
}

// ------------------------------------------------------------------ weight layouts
// kRows:  [E][N][K] int8 (int4: [E][N][K/2] bytes), input axis contiguous.
// kTiled: the same bytes arranged as MFMA A operands.  int8: for each group of
//   16 rows and each 64-wide K step one 1 KB block in lane order, lane
//   l = row%16 + 16*((k%64)/16) holding k%16 = 0..15.  int4: for each group of
//   16 rows and each 128-wide K span one 1 KB block, lane l = row%16 +
//   16*((k%32)/8) holding 4 bytes per block of 32 (elements 8g..8g+7, two per
//   byte, low nibble first) for the span's 4 blocks in order.
// A wavefront streaming one row group then reads whole 1 KB blocks per
// instruction.
constexpr int kRows = 0, kTiled = 1;

template <int LAY>
__device__ inline const int8_t* i8_operand_base(const int8_t* W, size_t row0, int K, int i,
                                                int g, int lane) {
  return LAY == kRows ? W + (row0 + i) * K + 16 * g : W + row0 * K + 16 * lane;
}
template <int LAY>
__device__ inline v4i i8_load(const int8_t* base, int step) {
  return gload_nt<v4i>(base + (LAY == kRows ? 64 : 1024) * step);
}
// Ordinary (cached) load: for weights that several tiles of one expert read.
template <int LAY>
__device__ inline v4i i8_load_cached(const int8_t* base, int step) {
  return gload<v4i>(base + (LAY == kRows ? 64 : 1024) * step);
}

template <int LAY>
__device__ inline const uint8_t* i4_operand_base(const uint8_t* W, size_t row0, int K, int i,
                                                 int g, int lane) {
  return LAY == kRows ? W + (row0 + i) * (K / 2) + 4 * g : W + row0 * (K / 2) + 16 * lane;
}
// the 4 words (one per block of 32) of span m
template <int LAY>
__device__ inline v4i i4_load(const uint8_t* base, int m) {
  if (LAY == kTiled) return gload_nt<v4i>(base + 1024 * m);
  const uint8_t* p = base + 64 * m;
  return v4i{gload<int>(p), gload<int>(p + 16), gload<int>(p + 32), gload<int>(p + 48)};
}

// ------------------------------------------------------------------ int4
// 8 codes of one 4-byte word (code 2b in the low nibble of byte b, code 2b+1
// in the high nibble) -> 8 bytes holding 16 * code, in the order
// (0, 2, 4, 6, 1, 3, 5, 7): the low nibbles shifted into the high half of each
// byte, the high nibbles masked in place.  A nibble in the high half of a byte
// reads as the signed byte 16 * code (two's complement), so three operations
// unpack 8 codes; the activation digits are stored in the same order (encode8)
// and the factor 16 goes into the block scale.
__device__ inline long unpack8_int4_x16(unsigned w) {
  const unsigned even = (w << 4) & 0xF0F0F0F0u;  // codes 0, 2, 4, 6
  const unsigned odd = w & 0xF0F0F0F0u;          // codes 1, 3, 5, 7
  return (long)(((unsigned long)odd << 32) | even);
}

constexpr float kScaleFloor = 1.0f / 16384.0f;  // int4 block scales are raised to 2^-14
constexpr float kInv16 = 1.0f / 16.0f;          // the unpacked codes carry a factor 16

// ------------------------------------------------------------------ gate/up
// FMT 1: int8 rows; FMT 2: int4 blocks of 32.  Block = 4*KS wavefronts:
// column group cg = wave % 4 (16 h-columns each), K slice kp = wave / 4.
// PAIRS (small batches): rows are the (token, slot) pairs grouped in-kernel.
// The tile's activation digit rows are staged in LDS (mt rows of 2d bytes); a
// workgroup covers NCB column blocks of 64 in turn.
// SEL (one token, SelIn): the launch selects the token's experts and encodes
// its row of x itself, in front of the weight loads, instead of a selection
// launch before it.  The x row's loads go out first, so that they overlap
// the selection; every routed workgroup ranks the experts from the logit
// slices with the router's own select_token (the same keys, order and
// weights), keeps the indices in LDS and takes tile t's expert from slot t;
// the launch's first workgroup also stores the indices and weights.  Every
// workgroup encodes the row into LDS as two-digit int8 with one scale, as the
// router's selection launch does, and the K loop reads the digits from there.
template <int FMT, int LAY, int KS, bool PAIRS, int NCB, bool SPLIT, bool SEL = false>
__global__ __launch_bounds__(256 * KS) void gate_up_kernel(Group g0, Group g1, int d, int mt,
                                                           const int8_t* __restrict__ xq,
                                                           const float* __restrict__ xs,
                                                           SplitK sk, SelIn sel) {
  extern __shared__ int8_t lds[];
  __shared__ float red_max[4][16];
  // K-slice partials: int8 path 16 ints per lane, int4 path 8 floats per lane
  __shared__ float red_acc[KS > 1 ? (KS - 1) * 4 * 64 * 16 : 1];
  __shared__ int rows_sm[kTileRows], toks_sm[kTileRows], sh_sm[3], last_sm;
  int vtile = blockIdx.y, kw = 0, nsplit = 1, slot0 = 0;  // (see SplitK)
  if constexpr (SPLIT) {
    const SplitPos sp = split_pos(sk, blockIdx.y, g0.tiles, gridDim.x, blockIdx.x);
    vtile = sp.tile;
    kw = sp.kw;
    nsplit = sp.n;
    slot0 = sp.slot0;
  }
  {
    const bool first = vtile < g0.tiles;
    if ((int)blockIdx.x * 64 * NCB >= (first ? g0.inter : g1.inter)) return;
  }
  float sel_xs = 0.0f;  // SEL: the x row's scale
  __shared__ int sel_idx[SEL ? kMaxK : 1];
  if constexpr (SEL) {
    __shared__ unsigned long long sel_keys[KS][256];
    __shared__ float sel_red[KS][4], sel_s[KS][kMaxK], sel_w[kMaxK], sel_xred[4 * KS];
    const int tid = threadIdx.x, n8 = d / 8;
    float4 xv[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int c = tid + 256 * KS * m;
      const bool ok = c < n8;
      const float* src = sel.x + 8 * (ok ? c : 0);
      xv[m][0] = ok ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
      xv[m][1] = ok ? *reinterpret_cast<const float4*>(src + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (vtile < g0.tiles) {  // routed workgroups (the whole workgroup takes part)
      const int grp = tid >> 8;
      const bool lead = blockIdx.x == 0 && blockIdx.y == 0;
      select_token<1>(sel.partial, sel.nchunk, sel.bias, sel.mask, 1, sel.E, sel.k, sel.router,
                      sel.scale, 0, grp == 0, tid & 255, sel_keys[grp], sel_red[grp],
                      sel_s[grp], lead ? sel.idx : sel_idx, lead ? sel.w : sel_w, sel_idx);
    }
    float mx = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[m][h].x), fabsf(xv[m][h].y)),
                             fmaxf(fabsf(xv[m][h].z), fabsf(xv[m][h].w))));
    mx = wave_max_f(mx);
    if ((tid & (kWave - 1)) == 0) sel_xred[tid / kWave] = mx;
    __syncthreads();
    mx = 0.0f;
    for (int q = 0; q < 4 * KS; ++q) mx = fmaxf(mx, sel_xred[q]);
    const int p = digit_exponent(mx);
    uint2* q0 = reinterpret_cast<uint2*>(lds);
    uint2* q1 = reinterpret_cast<uint2*>(lds + d);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int c = tid + 256 * KS * m;
      if (c >= n8) continue;
      uint2 w0, w1;
      encode8(xv[m][0], xv[m][1], p, sel.perm, w0, w1);
      const int dst = sel.perm ? int4_digit_chunk(c) : c;
      q0[dst] = w0;
      q1[dst] = w1;
    }
    sel_xs = mx > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
    __syncthreads();
  }
  Job job;
  if (SEL && vtile < g0.tiles) {  // slot vtile of the token (as find_rows at one token)
    const int e = sel_idx[vtile];
    if (e < 0 || e >= g0.E) return;
    job.g = 0;
    job.e = e;
    job.r0 = 0;
    job.nr = 1;
    if (threadIdx.x == 0) {
      rows_sm[0] = vtile;
      toks_sm[0] = 0;
    }
    __syncthreads();
  } else if (PAIRS) {  // the expert histogram uses the dynamic LDS area
    if (!find_rows(g0, g1, mt, vtile, job, rows_sm, toks_sm, reinterpret_cast<int*>(lds),
                   sh_sm, true))
      return;
  } else {
    if (!find_job(g0, g1, mt, vtile, job)) return;
  }
  const Group G = job.g == 0 ? g0 : g1;
  const int I = G.inter;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int cg = wave & 3, kp = wave >> 2;
  const int i = lane & 15, g = lane >> 4;
  // K slice of this wavefront: slice kw * KS + kp of nsplit * KS
  const int ksl = kw * KS + kp, nsl = nsplit * KS;
  const int unit = vtile * gridDim.x + blockIdx.x;  // (NCB == 1 when SPLIT)
  // x digits of the tile rows.  Small batches (PAIRS) read their few token
  // rows straight from L2: no staging barrier before the weight loads, no LDS
  // to limit how many workgroups a CU holds.  Tiles of up to 16 rows stage them
  // in LDS (measured faster there).  A rows past the tile (i >= nr) read a real
  // row again: their products land in accumulator rows that are never stored,
  // and unconditional loads keep the compiler's count of loads in flight exact.
  // (the lambdas capture scalars by value: a reference to the selected Group
  // would keep the struct in private memory, with every pointer read from it
  // losing its address space)
  const int32_t* const row_token = G.row_token;
  const int r0 = job.r0, nr = job.nr;
  auto tile_tok = [=](int j) {
    return PAIRS ? toks_sm[j] : row_token ? gload<int>(row_token + r0 + j) : r0 + j;
  };
  const int8_t* xb0;
  if (SEL) {
    xb0 = lds;
  } else if (PAIRS) {
    xb0 = xq + (size_t)tile_tok(min(i, job.nr - 1)) * 2 * d;
  } else {
    const int ldr = 2 * d + 16;
    const int per_row = (2 * d) / 16;
    for (int q = threadIdx.x; q < job.nr * per_row; q += blockDim.x) {
      const int j = q / per_row, c = q % per_row;
      *reinterpret_cast<v4i*>(lds + j * ldr + 16 * c) =
          *reinterpret_cast<const v4i*>(xq + (size_t)tile_tok(j) * 2 * d + 16 * c);
    }
    __syncthreads();
    xb0 = lds + min(i, job.nr - 1) * ldr;
  }
  const int8_t* xb1 = xb0 + d;
  // x scale of tile rows 4g+c: loaded only after the main loop, unconditionally
  // from clamped rows, so no load in front of the loop is conditional
  auto x_scale = [=](int c) {
    const float v = SEL ? sel_xs : gload<float>(xs + tile_tok(min(4 * g + c, nr - 1)));
    return 4 * g + c < nr ? v : 0.0f;
  };

  // Operands: A = the tile's activation digits (A row = tile row lane % 16),
  // B = 16 weight rows as stored (B column = h column c0 + lane % 16).  A lane's
  // accumulator c is tile row 4 g + c of h column c0 + i, so each lane needs
  // the scale of one weight row only (one per int4 block).

#pragma unroll 1
  for (int cbi = 0; cbi < NCB; ++cbi) {
    const int cb = blockIdx.x * NCB + cbi;  // 64-column block
    if (cb * 64 >= I) break;                // uniform over the workgroup
    const int c0 = cb * 64 + cg * 16;       // this wavefront's 16 h-columns
    const size_t row0 = (size_t)job.e * 2 * I + c0;

    float gate[4], up[4];
    if (FMT == 1) {
      const int nsteps = d / kKStep;
      const int s_beg = ksl * nsteps / nsl, s_end = (ksl + 1) * nsteps / nsl;
      const int8_t* wa = i8_operand_base<LAY>(static_cast<const int8_t*>(G.wgu), row0, d, i, g,
                                              lane);
      const int8_t* wb = wa + (size_t)I * d;
      v4i a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0}, b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
      constexpr int U = 4;
      for (int s = s_beg; s < s_end; s += U) {
        v4i ra[U], rb[U], x0[U], x1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int ss = min(s + u, s_end - 1);
          ra[u] = i8_load<LAY>(wa, ss);
          rb[u] = i8_load<LAY>(wb, ss);
          x0[u] = *reinterpret_cast<const v4i*>(xb0 + ss * kKStep + 16 * g);
          x1[u] = *reinterpret_cast<const v4i*>(xb1 + ss * kKStep + 16 * g);
        }
        // steps past the slice (the last batch) multiply zero activations: no
        // branch, so the compiler keeps every load of the batch in front
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = s + u < s_end;
          const v4i z = {0, 0, 0, 0};
          const v4i xa = ok ? x0[u] : z, xb = ok ? x1[u] : z;
          a0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, ra[u], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb, ra[u], a1, 0, 0, 0);
          b0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, rb[u], b0, 0, 0, 0);
          b1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb, rb[u], b1, 0, 0, 0);
        }
      }
      // exact int32 reduction of the K slices (order-free)
      if (KS > 1) {
        int* red = reinterpret_cast<int*>(red_acc);
        if (kp > 0) {
          int* dst = red + (((kp - 1) * 4 + cg) * 64 + lane) * 16;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            dst[c] = a0[c]; dst[4 + c] = a1[c]; dst[8 + c] = b0[c]; dst[12 + c] = b1[c];
          }
        }
        __syncthreads();
        if (kp == 0) {
          for (int q = 1; q < KS; ++q) {
            const int* src = red + (((q - 1) * 4 + cg) * 64 + lane) * 16;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              a0[c] += src[c]; a1[c] += src[4 + c]; b0[c] += src[8 + c]; b1[c] += src[12 + c];
            }
          }
        }
      }
      if (SPLIT && nsplit > 1) {  // exact int32 sums across the unit's workgroups
        int v[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[c] = a0[c]; v[4 + c] = a1[c]; v[8 + c] = b0[c]; v[12 + c] = b1[c];
        }
        if (!split_join<int, 16>(sk, unit, slot0, kw, nsplit, cg, kp == 0, v, &last_sm))
          return;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          a0[c] = v[c]; a1[c] = v[4 + c]; b0[c] = v[8 + c]; b1[c] = v[12 + c];
        }
      }
      const float* se = G.sgu + (size_t)job.e * 2 * I;
      const float sgate = gload<float>(se + c0 + i), sup = gload<float>(se + I + c0 + i);
      float sx[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) sx[c] = x_scale(c);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        gate[c] = sgate * sx[c] * ((float)a0[c] + (float)a1[c] * (1.0f / 256.0f));
        up[c] = sup * sx[c] * ((float)b0[c] + (float)b1[c] * (1.0f / 256.0f));
      }
    } else {
      // int4: one 16x16x32 MFMA pair per 32 inputs on codes unpacked as
      // 16 * code.  Blocks of 32 (FMT 2): each block's two int32 digit sums
      // join as 256 p0 + p1 in int32 (below 2^28, rounded once to fp32) and are
      // scaled by max(s, 2^-14) / 16 into the fp32 accumulator.  Blocks of 128
      // (FMT 3) are the 128-input spans: the span's four MFMA pairs accumulate
      // in int32 and join once per span.  U spans (codes and their scales) are
      // loaded before any is used.
      const int nb = d / (FMT == 3 ? 128 : 32), nspan = d / 128;
      const int m_beg = ksl * nspan / nsl, m_end = (ksl + 1) * nspan / nsl;
      const uint8_t* wa = i4_operand_base<LAY>(static_cast<const uint8_t*>(G.wgu), row0, d, i,
                                               g, lane);
      const uint8_t* wb = wa + (size_t)I * (d / 2);
      const float* sa = G.sgu + ((size_t)job.e * 2 * I + c0 + i) * nb;  // this lane's rows
      const float* sb = sa + (size_t)I * nb;
      float fa[4] = {0.f, 0.f, 0.f, 0.f}, fb[4] = {0.f, 0.f, 0.f, 0.f};
      const v4i zero = {0, 0, 0, 0};
      constexpr int U = 2;
      for (int m0 = m_beg; m0 < m_end; m0 += U) {
        v4i wa4[U], wb4[U];
        v4f s1[U], s2[U];
        v2l xa[U][2], xc[U][2];  // digit 0 and 1 of the lane's 4 groups (span order)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int m = min(m0 + u, m_end - 1);
          wa4[u] = i4_load<LAY>(wa, m);
          wb4[u] = i4_load<LAY>(wb, m);
          if constexpr (FMT == 2) {
            s1[u] = gload<v4f>(sa + 4 * m);
            s2[u] = gload<v4f>(sb + 4 * m);
          } else {
            s1[u] = v4f{gload<float>(sa + m), 0.f, 0.f, 0.f};
            s2[u] = v4f{gload<float>(sb + m), 0.f, 0.f, 0.f};
          }
          const v2l* p0 = reinterpret_cast<const v2l*>(xb0 + 128 * m + 32 * g);
          const v2l* p1 = reinterpret_cast<const v2l*>(xb1 + 128 * m + 32 * g);
          xa[u][0] = p0[0];
          xa[u][1] = p0[1];
          xc[u][0] = p1[0];
          xc[u][1] = p1[1];
        }
        // spans past the slice (the last batch) multiply zero activations: no
        // branch, so the compiler keeps every load of the batch in front
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const long on = m0 + u < m_end ? -1L : 0L;
          const long x0[4] = {xa[u][0].x & on, xa[u][0].y & on, xa[u][1].x & on, xa[u][1].y & on};
          const long x1[4] = {xc[u][0].x & on, xc[u][0].y & on, xc[u][1].x & on, xc[u][1].y & on};
          if constexpr (FMT == 2) {
            const float ss1[4] = {s1[u].x, s1[u].y, s1[u].z, s1[u].w};
            const float ss2[4] = {s2[u].x, s2[u].y, s2[u].z, s2[u].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const long qa = unpack8_int4_x16((unsigned)wa4[u][q]);
              const long qb = unpack8_int4_x16((unsigned)wb4[u][q]);
              const v4i pa0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(x0[q], qa, zero, 0, 0, 0);
              const v4i pa1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(x1[q], qa, zero, 0, 0, 0);
              const v4i pb0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(x0[q], qb, zero, 0, 0, 0);
              const v4i pb1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(x1[q], qb, zero, 0, 0, 0);
              const float t1 = fmaxf(ss1[q], kScaleFloor) * kInv16;
              const float t2 = fmaxf(ss2[q], kScaleFloor) * kInv16;
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                fa[c] = fmaf(t1, (float)(pa0[c] * 256 + pa1[c]), fa[c]);
                fb[c] = fmaf(t2, (float)(pb0[c] * 256 + pb1[c]), fb[c]);
              }
            }
          } else {
            // one scale for the span: blocks in pairs through the 16x16x64 MFMA
            // (the 16x16x32 form takes as long on this chip for half the work)
            v4i pa0 = zero, pa1 = zero, pb0 = zero, pb1 = zero;
#pragma unroll
            for (int q = 0; q < 4; q += 2) {
              const long qa0 = unpack8_int4_x16((unsigned)wa4[u][q]);
              const long qa1 = unpack8_int4_x16((unsigned)wa4[u][q + 1]);
              const long qb0 = unpack8_int4_x16((unsigned)wb4[u][q]);
              const long qb1 = unpack8_int4_x16((unsigned)wb4[u][q + 1]);
              const v4i qa = {(int)qa0, (int)(qa0 >> 32), (int)qa1, (int)(qa1 >> 32)};
              const v4i qb = {(int)qb0, (int)(qb0 >> 32), (int)qb1, (int)(qb1 >> 32)};
              const v4i xa = {(int)x0[q], (int)(x0[q] >> 32), (int)x0[q + 1], (int)(x0[q + 1] >> 32)};
              const v4i xc = {(int)x1[q], (int)(x1[q] >> 32), (int)x1[q + 1], (int)(x1[q + 1] >> 32)};
              pa0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, qa, pa0, 0, 0, 0);
              pa1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xc, qa, pa1, 0, 0, 0);
              pb0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, qb, pb0, 0, 0, 0);
              pb1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xc, qb, pb1, 0, 0, 0);
            }
            const float t1 = fmaxf(s1[u].x, kScaleFloor) * kInv16;
            const float t2 = fmaxf(s2[u].x, kScaleFloor) * kInv16;
#pragma unroll
            for (int c = 0; c < 4; ++c) {  // |p0| < 2^22: each digit sum exact in fp32
              fa[c] = fmaf(t1, fmaf((float)pa0[c], 256.0f, (float)pa1[c]), fa[c]);
              fb[c] = fmaf(t2, fmaf((float)pb0[c], 256.0f, (float)pb1[c]), fb[c]);
            }
          }
        }
      }
      if (KS > 1) {  // fp32 partials added in slice order
        if (kp > 0) {
          float* dst = red_acc + (((kp - 1) * 4 + cg) * 64 + lane) * 8;
#pragma unroll
          for (int c = 0; c < 4; ++c) { dst[c] = fa[c]; dst[4 + c] = fb[c]; }
        }
        __syncthreads();
        if (kp == 0) {
          for (int q = 1; q < KS; ++q) {
            const float* src = red_acc + (((q - 1) * 4 + cg) * 64 + lane) * 8;
#pragma unroll
            for (int c = 0; c < 4; ++c) { fa[c] += src[c]; fb[c] += src[4 + c]; }
          }
        }
      }
      if (SPLIT && nsplit > 1) {  // fp32 partials added in workgroup order
        float v[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) { v[c] = fa[c]; v[4 + c] = fb[c]; }
        if (!split_join<float, 8>(sk, unit, slot0, kw, nsplit, cg, kp == 0, v, &last_sm))
          return;
#pragma unroll
        for (int c = 0; c < 4; ++c) { fa[c] = v[c]; fb[c] = v[4 + c]; }
      }
      float sx[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) sx[c] = x_scale(c);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float sig = sx[c] * (1.0f / 256.0f);
        gate[c] = fa[c] * sig;
        up[c] = fb[c] * sig;
      }
    }

    // ---- epilogue: h = act(gate) * up, encoded per (tile row, 64-column block).
    // Lane (i, g) holds tile rows 4g+c of column c0+i: the row maximum runs over
    // the 16 lanes of equal g, then over the 4 column groups through LDS.
    float h[4], mx[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      h[c] = act_f(G.act, gate[c]) * up[c];
      mx[c] = fabsf(h[c]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx[c] = fmaxf(mx[c], __shfl_xor(mx[c], o, kWave));
    }
    if (kp == 0 && i == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) red_max[cg][4 * g + c] = mx[c];
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = 4 * g + c;
        if (t >= job.nr) continue;
        const float m = fmaxf(fmaxf(red_max[0][t], red_max[1][t]),
                              fmaxf(red_max[2][t], red_max[3][t]));
        const int p = digit_exponent(m);
        int d0, d1;
        two_digits(h[c], p, d0, d1);
        const int r = PAIRS ? rows_sm[t] : job.r0 + t;
        int8_t* hrow = G.hq + (size_t)r * 2 * I;
        const int col = FMT == 1 ? c0 + i : int4_digit_pos(c0 + i);  // the down kernel's order
        hrow[col] = (int8_t)d0;
        hrow[I + col] = (int8_t)d1;
        if (cg == 0 && i == 0) G.hs[(size_t)r * (I / 64) + cb] = m > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
      }
    }
    if (NCB > 1) __syncthreads();  // red_max is reused by the next column block
  }
}

// ------------------------------------------------------------------ down
// LDS: the tile's h digit rows (mt rows of 2I bytes), their block scales
// (mt x I/64 floats), then the K-slice partials.
// NG: 16-row weight groups per wavefront (2 for int8 without K split, so each
// workgroup streams 128 output rows and its prologue is amortised over more
// bytes).  CG: 16-row column groups per workgroup (4; 2 gives a finer grid
// when the units are few).
template <int FMT, int LAY, int KS, bool PAIRS, int NG, bool SPLIT, int CG = 4>
__global__ __launch_bounds__(kWave * CG * KS) void down_kernel(Group g0, Group g1, int d, int mt,
                                                               SplitK sk) {
  extern __shared__ int8_t lds[];
  __shared__ float red_acc[KS > 1 ? (KS - 1) * CG * 64 * 4 : 1];
  __shared__ int rows_sm[kTileRows], sh_sm[3], last_sm;
  int vtile = blockIdx.y, kw = 0, nsplit = 1, slot0 = 0;  // (see SplitK)
  if constexpr (SPLIT) {
    const SplitPos sp = split_pos(sk, blockIdx.y, g0.tiles, gridDim.x, blockIdx.x);
    vtile = sp.tile;
    kw = sp.kw;
    nsplit = sp.n;
    slot0 = sp.slot0;
  }
  Job job;
  if (PAIRS) {  // the expert histogram borrows the h staging area
    if (!find_rows(g0, g1, mt, vtile, job, rows_sm, nullptr, reinterpret_cast<int*>(lds),
                   sh_sm, false))
      return;
  } else {
    if (!find_job(g0, g1, mt, vtile, job)) return;
  }
  const Group G = job.g == 0 ? g0 : g1;
  const int I = G.inter;
  const int ldr = 2 * I + 16;
  const int nhb = I / 64;
  float* lds_s = reinterpret_cast<float*>(lds + (size_t)mt * ldr);
  if (!PAIRS) {  // small batches read their few h rows straight from L2 (no LDS, more
  // workgroups resident)
    const int per_row = (2 * I) / 16;
    for (int q = threadIdx.x; q < job.nr * per_row; q += blockDim.x) {
      const int j = q / per_row, c = q % per_row;
      *reinterpret_cast<v4i*>(lds + j * ldr + 16 * c) =
          *reinterpret_cast<const v4i*>(G.hq + (size_t)(job.r0 + j) * 2 * I + 16 * c);
    }
    for (int q = threadIdx.x; q < job.nr * nhb; q += blockDim.x)
      lds_s[q] = G.hs[(size_t)(job.r0 + q / nhb) * nhb + q % nhb];
    __syncthreads();
  }

  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int cg = wave % CG, kp = wave / CG;
  // K slice of this wavefront: slice kw * KS + kp of nsplit * KS
  const int ksl = kw * KS + kp, nsl = nsplit * KS;
  const int c0 = (blockIdx.x * CG + cg) * 16 * NG;  // output rows of this wavefront
  const int i = lane & 15, g = lane >> 4;
  const bool jv = i < job.nr;
  // Small batches (PAIRS, h rows from L2): lanes of rows past the tile read
  // the tile's first row.  They only feed MFMA output column i, which those
  // lanes never store, and unconditional global loads keep the compiler's
  // count of loads in flight exact.  Tiles read h from LDS, where skipping
  // the rows past the tile is cheaper (measured).
  const bool hv = PAIRS || jv;
  const int ii = jv ? i : 0;
  const int r = PAIRS ? rows_sm[ii] : job.r0 + ii;
  const int8_t* hb0 = PAIRS ? G.hq + (size_t)r * 2 * I : lds + ii * ldr;
  const int8_t* hb1 = hb0 + I;
  // small int8 batches with two row groups per wavefront: the tile's h block
  // scales, staged in LDS (the expert histogram's area, free once the rows
  // are found), so that the K loop reads each step's scale from LDS and issues
  // only weight and digit loads (Kimi-shaped T = 8 down 52.2 -> 50.9 us; the
  // int4 down at one token and T = 2 were slower with it, so they keep
  // reading the scales from L2)
  constexpr bool kStageHs = PAIRS && FMT == 1 && NG == 2;
  if (kStageHs) {
    float* sc = reinterpret_cast<float*>(lds);
    for (int q = threadIdx.x; q < job.nr * nhb; q += blockDim.x)
      sc[q] = G.hs[(size_t)rows_sm[q / nhb] * nhb + q % nhb];
    __syncthreads();
  }
  const float* hsr = kStageHs ? reinterpret_cast<const float*>(lds) + ii * nhb
                     : PAIRS  ? G.hs + (size_t)r * nhb
                              : lds_s + ii * nhb;
  const size_t row0 = (size_t)job.e * d + c0;
  const v4i zero = {0, 0, 0, 0};
  float acc[NG][4];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[q][c] = 0.0f;

  // int8: the output-row scales, loaded before the loop (its waits cover
  // them; after it they cost a round trip at the end of every workgroup)
  float sdn[NG][4];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      sdn[q][c] = FMT == 1 ? G.sdn[(size_t)job.e * d + c0 + 16 * q + 4 * g + c] : 1.0f;
  if (FMT == 1) {
    const int nsteps = I / kKStep;
    const int s_beg = ksl * nsteps / nsl, s_end = (ksl + 1) * nsteps / nsl;
    const int8_t* wa = i8_operand_base<LAY>(static_cast<const int8_t*>(G.wdn), row0, I, i, g,
                                            lane);
    // 8 KB of weights in flight per wavefront
    constexpr int U = KS == 1 ? 8 / NG : 4;
    for (int s = s_beg; s < s_end; s += U) {
      v4i ra[NG][U], x0[U], x1[U];
      float sg[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ss = min(s + u, s_end - 1);
#pragma unroll
        for (int q = 0; q < NG; ++q) ra[q][u] = i8_load<LAY>(wa + (size_t)16 * q * I, ss);
        x0[u] = zero;
        x1[u] = zero;
        sg[u] = 0.0f;
        if (hv) {
          x0[u] = *reinterpret_cast<const v4i*>(hb0 + ss * kKStep + 16 * g);
          x1[u] = *reinterpret_cast<const v4i*>(hb1 + ss * kKStep + 16 * g);
          sg[u] = hsr[ss];
        }
      }
      // steps past the slice (the last batch) get a zero scale: their
      // (finite) products add nothing, and no branch keeps loads in front
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float su = s + u < s_end ? sg[u] : 0.0f;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const v4i p0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra[q][u], x0[u], zero, 0, 0, 0);
          const v4i p1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra[q][u], x1[u], zero, 0, 0, 0);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[q][c] = fmaf(su, fmaf((float)p1[c], 1.0f / 256.0f, (float)p0[c]), acc[q][c]);
        }
      }
    }
  } else {
    // int4 blocks of 32 (FMT 2) or 128 (FMT 3, the span: its MFMA pairs
    // accumulate in int32 per 64-column half, since h has one scale per 64)
    const int nb = I / (FMT == 3 ? 128 : 32), nspan = I / 128;
    const int m_beg = ksl * nspan / nsl, m_end = (ksl + 1) * nspan / nsl;
    const uint8_t* wa = i4_operand_base<LAY>(static_cast<const uint8_t*>(G.wdn), row0, I, i, g,
                                             lane);
    const float* sa = G.sdn + ((size_t)job.e * d + c0 + 4 * g) * nb;
    for (int m = m_beg; m < m_end; ++m) {
      const v4i w4 = i4_load<LAY>(wa, m);
      long x0[4], x1[4];
      float sg[2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x0[q] = 0;
        x1[q] = 0;
        if (hv) {
          x0[q] = *reinterpret_cast<const long*>(hb0 + 128 * m + 32 * g + 8 * q);
          x1[q] = *reinterpret_cast<const long*>(hb1 + 128 * m + 32 * g + 8 * q);
        }
      }
      sg[0] = hv ? hsr[2 * m] * (1.0f / 256.0f) : 0.0f;
      sg[1] = hv ? hsr[2 * m + 1] * (1.0f / 256.0f) : 0.0f;
      if constexpr (FMT == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int b = 4 * m + q;
          const long wq = unpack8_int4_x16((unsigned)w4[q]);
          const v4i p0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(wq, x0[q], zero, 0, 0, 0);
          const v4i p1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(wq, x1[q], zero, 0, 0, 0);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float sw = fmaxf(sa[(size_t)c * nb + b], kScaleFloor) * kInv16;
            acc[0][c] = fmaf(sw * sg[q >> 1], (float)(p0[c] * 256 + p1[c]), acc[0][c]);
          }
        }
      } else {
        // blocks 2h, 2h+1 (one h scale per 64) through one 16x16x64 MFMA per digit
        v4i p0[2], p1[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const long w0 = unpack8_int4_x16((unsigned)w4[2 * hh]);
          const long w1 = unpack8_int4_x16((unsigned)w4[2 * hh + 1]);
          const v4i wv = {(int)w0, (int)(w0 >> 32), (int)w1, (int)(w1 >> 32)};
          const v4i xa = {(int)x0[2 * hh], (int)(x0[2 * hh] >> 32), (int)x0[2 * hh + 1],
                          (int)(x0[2 * hh + 1] >> 32)};
          const v4i xc = {(int)x1[2 * hh], (int)(x1[2 * hh] >> 32), (int)x1[2 * hh + 1],
                          (int)(x1[2 * hh + 1] >> 32)};
          p0[hh] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, xa, zero, 0, 0, 0);
          p1[hh] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, xc, zero, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float sw = fmaxf(sa[(size_t)c * nb + m], kScaleFloor) * kInv16;
          const float v = fmaf(sg[0], fmaf((float)p0[0][c], 256.0f, (float)p1[0][c]),
                               sg[1] * fmaf((float)p0[1][c], 256.0f, (float)p1[1][c]));
          acc[0][c] = fmaf(sw, v, acc[0][c]);
        }
      }
    }
  }
  if (KS > 1) {  // (NG == 1 whenever KS > 1)
    if (kp > 0) {
      float* dst = red_acc + (((kp - 1) * CG + cg) * 64 + lane) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[c] = acc[0][c];
    }
    __syncthreads();
    if (!SPLIT && kp != 0) return;
    if (kp == 0) {
      for (int q = 1; q < KS; ++q) {
        const float* src = red_acc + (((q - 1) * CG + cg) * 64 + lane) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[0][c] += src[c];
      }
    }
  }
  if (SPLIT && nsplit > 1) {  // fp32 partials added in workgroup order (NG == 1 when SPLIT)
    const int unit = vtile * gridDim.x + blockIdx.x;
    if (!split_join<float, 4>(sk, unit, slot0, kw, nsplit, cg, kp == 0, acc[0], &last_sm))
      return;
  }
  if ((SPLIT && kp != 0) || !jv) return;  // (without SPLIT, kp > 0 left above)
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    float res[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) res[c] = FMT == 1 ? sdn[q][c] * acc[q][c] : acc[q][c];
    *reinterpret_cast<float4*>(G.out + (size_t)r * d + c0 + 16 * q + 4 * g) =
        make_float4(res[0], res[1], res[2], res[3]);
  }
}

// ------------------------------------------------------------------ prefill GEMM
// Many rows per expert: gate/up runs as a grouped GEMM over tiles of one
// expert's rows.  A workgroup of 8 wavefronts covers a tile and a block of
// output columns; each wavefront owns 32 columns (16 gate and 16 up rows,
// twice) and 64 tile rows, so per 64-wide K-step it runs 4 weight fragments x
// 4 row groups x 2 digits = 32 MFMAs with every operand read from LDS.  Two
// shapes (WT = wavefront rows): WT = 2 takes 128-row tiles and 128 columns
// (many rows per expert, so weights are re-read for fewer tiles); WT = 1
// takes 64-row tiles and 256 columns (few rows per expert, so fewer digit
// bytes move per weight byte).
//
// Both operands reach LDS by direct global-to-LDS loads (no registers): per
// K-step 4 weight blocks per 16-column group (each an MFMA A operand of 1 KB,
// contiguous in the tiled layout) and 2 digit blocks per row group (gathered
// by row), the same number of loads for every wavefront.  A ring of K-step
// slots (4 for WT = 2, 3 for WT = 1) keeps 3 or 2 K-steps in flight.  Every
// wavefront issues the same loads in the same order on every K-step (rows
// past the tile re-read row 0, K-steps past the end re-read the last one), so
// before the barrier of K-step s each wavefront waits until only the loads of
// the K-steps after s are still in flight: its own part of slot s has landed,
// and after the barrier every part has.  The barrier is a bare s_barrier
// between compiler fences: no wait on the loads still in flight.  The slots
// are separate LDS arrays so that the compiler can tell the loads into one
// slot from the reads of another.
constexpr int kPWaves = 8;
constexpr int kPBlk = 1024;                 // one MFMA operand

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding)
#define MOE_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | ((((n) >> 4) & 3) << 14))

__device__ inline void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global-to-LDS load: lane l's 16 bytes land at dst + 16 l.
__device__ inline void lds_load16(const void* src, int8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

__device__ inline v4i lds_frag(const int8_t* blk, int lane) {
  return *reinterpret_cast<const v4i*>(blk + 16 * lane);
}

// Source of weight block "row group rg (16 rows from row0), K-step s" for this
// lane: tiled = the block itself; rows = the lane's row and 16 bytes.
template <int LAY>
__device__ inline const int8_t* wblock_src(const int8_t* W, size_t row0, int K, int lane) {
  return LAY == kRows ? W + (row0 + (lane & 15)) * K + 16 * (lane >> 4)
                      : W + row0 * K + 16 * lane;
}
template <int LAY>
constexpr int wblock_step() {
  return LAY == kRows ? kKStep : kPBlk;
}

// Tile geometry of the gate/up GEMM for WT wavefront rows.
template <int WT>
struct GuShape {
  static constexpr int CW = kPWaves / WT;          // column wavefronts
  static constexpr int ROWS = 64 * WT;             // tile rows
  static constexpr int COLS = 32 * CW;             // output columns per workgroup
  static constexpr int NA = 4 * CW;                // weight blocks per K-step
  static constexpr int NB = 2 * ROWS / 16;         // digit blocks per K-step
  static constexpr int A_PER = NA / kPWaves;       // per wavefront
  static constexpr int B_PER = NB / kPWaves;
  static constexpr int SLOT = (NA + NB) * kPBlk;   // LDS bytes per K-step slot
  static constexpr int NS = WT == 2 ? 4 : 3;       // slots in the ring
  static constexpr int WAIT = (NS - 2) * (A_PER + B_PER);  // loads left in flight
};

#define RING_SLOT(q) ((q) == 0 ? ring0 : (q) == 1 ? ring1 : (q) == 2 ? ring2 : ring3)

// Gate activation fixed at compile time (ACT = 0 silu, 1 gelu_tanh), so that
// the epilogue's values need no branch each.  Both expert sets of a launch
// take the layer's activation.
template <int ACT>
__device__ inline float act_t(float z) {
  return ACT == 1 ? gelu_tanh_f(z) : silu_f(z);
}

template <int LAY, int WT, int ACT>
__global__ __launch_bounds__(512) void gate_up_gemm_kernel(Group g0, Group g1, int d,
                                                           const int8_t* __restrict__ xq,
                                                           const float* __restrict__ xs) {
  using S = GuShape<WT>;
  __shared__ __attribute__((aligned(16))) int8_t ring0[S::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t ring1[S::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t ring2[S::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t ring3[S::NS == 4 ? S::SLOT : 16];
  __shared__ float red_max[S::CW][S::ROWS];
  __shared__ int tok_sm[S::ROWS];
  Job job;
  if (!find_job(g0, g1, S::ROWS, blockIdx.y, job)) return;
  const Group G = job.g == 0 ? g0 : g1;
  const int I = G.inter;
  const int cb = blockIdx.x * S::COLS;
  if (cb >= I) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int wc = wave % S::CW, wt = wave / S::CW;
  const int c0 = cb + wc * 32;
  const int i = lane & 15, g = lane >> 4;
  const int ntg = min(4, max(0, (job.nr - 64 * wt + 15) / 16));
  const bool active = c0 < I && ntg > 0;  // every wavefront issues loads and meets the barriers
  for (int j = threadIdx.x; j < S::ROWS; j += blockDim.x)
    tok_sm[j] = j < job.nr ? (G.row_token ? G.row_token[job.r0 + j] : job.r0 + j) : -1;
  __syncthreads();
  // the epilogue's scales, loaded now and unconditionally (clamped indices):
  // this wavefront's gate and up row scales and the x scales of its tile
  // rows.  They are older than every load of the ring, whose waits therefore
  // cover them; loaded in the epilogue under the row conditions they cost a
  // round trip each.
  float sgate[2][4], sup[2][4], sig[4];
  {
    const float* se = G.sgu + (size_t)job.e * 2 * I;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = min(c0 + 16 * q + 4 * g + c, I - 1);
        sgate[q][c] = se[n];
        sup[q][c] = se[I + n];
      }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tj = tok_sm[64 * wt + 16 * t + i];
      sig[t] = xs[tj >= 0 ? tj : tok_sm[0]];
    }
  }

  // this wavefront's loads per K-step: weight blocks A_PER w .. (blocks
  // 0 .. 2CW-1 = gate row groups of columns cb.., then the same up rows) and
  // digit blocks B_PER w .. (block q = row group q/2, digit q%2)
  const int8_t* W = static_cast<const int8_t*>(G.wgu);
  const int8_t* asrc[S::A_PER];
  const int8_t* bsrc[S::B_PER];
#pragma unroll
  for (int u = 0; u < S::A_PER; ++u) {
    const int blk = S::A_PER * wave + u;
    const bool up = blk >= 2 * S::CW;
    const int col = cb + 16 * (up ? blk - 2 * S::CW : blk);
    const size_t row0 = (size_t)job.e * 2 * I + (col < I ? col + (up ? I : 0) : 0);
    asrc[u] = wblock_src<LAY>(W, row0, d, lane);
  }
#pragma unroll
  for (int u = 0; u < S::B_PER; ++u) {
    const int blk = S::B_PER * wave + u;
    const int j = 16 * (blk >> 1) + i;
    const int tok = tok_sm[j] >= 0 ? tok_sm[j] : tok_sm[0];
    bsrc[u] = xq + (size_t)tok * 2 * d + (blk & 1) * d + 16 * g;
  }
  const int nsteps = d / kKStep;
  const int last = nsteps - 1;
  auto issue = [&](int8_t* slot, int step) {
    const int st = min(step, last);
#pragma unroll
    for (int u = 0; u < S::A_PER; ++u)
      lds_load16(asrc[u] + (size_t)st * wblock_step<LAY>(),
                 slot + (S::A_PER * wave + u) * kPBlk);
#pragma unroll
    for (int u = 0; u < S::B_PER; ++u)
      lds_load16(bsrc[u] + st * kKStep, slot + (S::NA + S::B_PER * wave + u) * kPBlk);
  };

  v4i acc[4][4][2];  // [weight fragment][row group][digit]
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[f][t][0] = acc[f][t][1] = v4i{0, 0, 0, 0};
  // weight blocks of this wavefront's fragments: gate 2wc, 2wc+1, up 2CW+2wc, 2CW+2wc+1
  const int ablk[4] = {2 * wc, 2 * wc + 1, 2 * S::CW + 2 * wc, 2 * S::CW + 2 * wc + 1};

#pragma unroll
  for (int q = 0; q < S::NS - 1; ++q) issue(RING_SLOT(q), q);

// A wavefront with all four row groups valid (ntg == 4) reads all twelve
// fragments of the K-step at once and then runs its 32 MFMAs: with the row
// groups behind run-time conditions each group's reads wait until the
// previous group's MFMAs are issued, four LDS round trips per K-step.
#define GU_STEP(STEP, Q) { if (ntg == 4) GU_FULL(STEP, Q) else GU_PART(STEP, Q) }
#define GU_FULL(STEP, Q)                                                                      \
  {                                                                                           \
    MOE_WAIT_VM(S::WAIT);                                                                     \
    ring_barrier();                                                                           \
    if (active) {                                                                             \
      const int8_t* slot = RING_SLOT(Q);                                                      \
      v4i a[4], b[4][2];                                                                      \
      _Pragma("unroll") for (int f = 0; f < 4; ++f) a[f] = lds_frag(slot + ablk[f] * kPBlk, lane); \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                         \
        const int8_t* bb = slot + (S::NA + 2 * (4 * wt + t)) * kPBlk;                         \
        b[t][0] = lds_frag(bb, lane);                                                         \
        b[t][1] = lds_frag(bb + kPBlk, lane);                                                 \
      }                                                                                       \
      __builtin_amdgcn_sched_barrier(0);                                                      \
      _Pragma("unroll") for (int t = 0; t < 4; ++t)                                           \
        _Pragma("unroll") for (int f = 0; f < 4; ++f) {                                       \
          acc[f][t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b[t][0], acc[f][t][0], 0, 0, 0); \
          acc[f][t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b[t][1], acc[f][t][1], 0, 0, 0); \
        }                                                                                     \
    }                                                                                         \
    issue(RING_SLOT(((Q) + S::NS - 1) % S::NS), (STEP) + S::NS - 1);                          \
  }
#define GU_PART(STEP, Q)                                                                  \
  {                                                                                           \
    MOE_WAIT_VM(S::WAIT);                                                                     \
    ring_barrier();                                                                           \
    if (active) {                                                                             \
      const int8_t* slot = RING_SLOT(Q);                                                      \
      v4i a[4];                                                                               \
      _Pragma("unroll") for (int f = 0; f < 4; ++f) a[f] = lds_frag(slot + ablk[f] * kPBlk, lane); \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                         \
        if (t < ntg) {                                                                        \
          const int8_t* bb = slot + (S::NA + 2 * (4 * wt + t)) * kPBlk;                       \
          const v4i b0 = lds_frag(bb, lane);                                                  \
          const v4i b1 = lds_frag(bb + kPBlk, lane);                                          \
          _Pragma("unroll") for (int f = 0; f < 4; ++f) {                                     \
            acc[f][t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b0, acc[f][t][0], 0, 0, 0); \
            acc[f][t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b1, acc[f][t][1], 0, 0, 0); \
          }                                                                                   \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
    issue(RING_SLOT(((Q) + S::NS - 1) % S::NS), (STEP) + S::NS - 1);                          \
  }
  int s0 = 0;
  if constexpr (S::NS == 4) {
    for (; s0 + 4 <= nsteps; s0 += 4) {
      GU_STEP(s0, 0)
      GU_STEP(s0 + 1, 1)
      GU_STEP(s0 + 2, 2)
      GU_STEP(s0 + 3, 3)
    }
    if (s0 < nsteps) GU_STEP(s0, 0)
    if (s0 + 1 < nsteps) GU_STEP(s0 + 1, 1)
    if (s0 + 2 < nsteps) GU_STEP(s0 + 2, 2)
  } else {
    for (; s0 + 3 <= nsteps; s0 += 3) {
      GU_STEP(s0, 0)
      GU_STEP(s0 + 1, 1)
      GU_STEP(s0 + 2, 2)
    }
    if (s0 < nsteps) GU_STEP(s0, 0)
    if (s0 + 1 < nsteps) GU_STEP(s0 + 1, 1)
  }
#undef GU_STEP
#undef GU_FULL
#undef GU_PART
  MOE_WAIT_VM(0);

  // epilogue: h per row, one scale per row and 128-column block (4 wavefronts)
  float h[2][4][4];  // [column half][row group][c]
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = 64 * wt + 16 * t + i;
    const bool rv = active && t < ntg && j < job.nr;
    float mx = 0.0f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float gt = sgate[q][c] * sig[t] *
                         ((float)acc[q][t][0][c] + (float)acc[q][t][1][c] * (1.0f / 256.0f));
        const float upv = sup[q][c] * sig[t] *
                          ((float)acc[2 + q][t][0][c] + (float)acc[2 + q][t][1][c] * (1.0f / 256.0f));
        const float hv = act_t<ACT>(gt) * upv;
        h[q][t][c] = rv ? hv : 0.0f;
        mx = fmaxf(mx, fabsf(h[q][t][c]));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    if (g == 0) red_max[wc][j] = mx;
  }
  __syncthreads();
  if (!active) return;
  const int grp = wc >> 2;  // 128-column scale block of this wavefront
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = 64 * wt + 16 * t + i;
    if (t >= ntg || j >= job.nr) continue;
    const float mx = fmaxf(fmaxf(red_max[4 * grp][j], red_max[4 * grp + 1][j]),
                           fmaxf(red_max[4 * grp + 2][j], red_max[4 * grp + 3][j]));
    const int p = digit_exponent(mx);
    const int r = job.r0 + j;
    int8_t* hrow = G.hq + (size_t)r * 2 * I;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int d0[4], d1[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) two_digits(h[q][t][c], p, d0[c], d1[c]);
      const int col = c0 + 16 * q + 4 * g;
      *reinterpret_cast<unsigned*>(hrow + col) = pack4(d0[0], d0[1], d0[2], d0[3]);
      *reinterpret_cast<unsigned*>(hrow + I + col) = pack4(d1[0], d1[1], d1[2], d1[3]);
    }
    if ((wc & 3) == 0 && g == 0)
      G.hs[(size_t)r * ((I + 127) / 128) + (cb >> 7) + grp] = mx > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
  }
}
#undef RING_SLOT

// Down projection as a grouped GEMM on the gate/up kernel's scheme: tiles of
// 64 WT rows of one expert, 8 wavefronts of 64 rows x 16 NF output columns (NF
// weight fragments of 16 output rows), every operand a 1 KB MFMA block moved
// straight into an LDS ring slot (weight blocks of the tiled layout, and h
// digit blocks gathered by row), 3 K-steps in flight, one bare barrier per
// K-step.  h carries one scale per row and 128 inputs: each 128-input block's
// two K-steps accumulate in int32 on the matrix cores, then fold into fp32 as
// (256 d0 + d1) times the block scale / 256.  The tile's block scales are
// staged in LDS once, before the ring starts, so that the loads in the K loop
// follow the ring's fixed pattern.
constexpr int kDnMaxBlocks = 32;  // 128-input scale blocks staged per row (I <= 4096)
constexpr int kDnFrags = 4;       // weight fragments (16 output columns each) per wavefront
template <int WT, int NF>
struct DnShape {
  static constexpr int CW = kPWaves / WT;          // column wavefronts
  static constexpr int ROWS = 64 * WT;             // tile rows
  static constexpr int COLS = 16 * NF * CW;        // output columns per workgroup
  static constexpr int NA = COLS / 16;             // weight blocks per K-step
  static constexpr int NB = 2 * ROWS / 16;         // digit blocks per K-step
  static constexpr int A_PER = NA / kPWaves;       // per wavefront
  static constexpr int B_PER = NB / kPWaves;
  static constexpr int SLOT = (NA + NB) * kPBlk;   // LDS bytes per K-step slot
  // slots in the ring: 4 where they fit beside the staged scales
  static constexpr int NS = 4 * SLOT + ROWS * kDnMaxBlocks * 4 <= 160 * 1024 - 1024 ? 4 : 3;
  static constexpr int WAIT = (NS - 2) * (A_PER + B_PER);  // loads left in flight
};

#define RING_SLOT(q) ((q) == 0 ? ring0 : (q) == 1 ? ring1 : (q) == 2 ? ring2 : ring3)

template <int LAY, int WT, int NF>
__global__ __launch_bounds__(512) void down_gemm_kernel(Group g0, Group g1, int d) {
  using S = DnShape<WT, NF>;
  __shared__ __attribute__((aligned(16))) int8_t ring0[S::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t ring1[S::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t ring2[S::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t ring3[S::NS == 4 ? S::SLOT : 16];
  __shared__ float sc_sm[S::ROWS][kDnMaxBlocks];
  Job job;
  if (!find_job(g0, g1, S::ROWS, blockIdx.y, job)) return;
  const Group G = job.g == 0 ? g0 : g1;
  const int I = G.inter;
  const int cb = blockIdx.x * S::COLS;
  if (cb >= d) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int wc = wave % S::CW, wt = wave / S::CW;
  const int c0 = cb + wc * 16 * NF;  // this wavefront's 16 NF output columns
  const int i = lane & 15, g = lane >> 4;
  const int r0 = job.r0, nr = job.nr;
  const int ntg = min(4, max(0, (nr - 64 * wt + 15) / 16));
  const bool active = c0 < d && ntg > 0;  // every wavefront issues loads and meets the barriers
  const int nhb = I / 128 + (I % 128 != 0);  // h scale blocks per row
  for (int q = threadIdx.x; q < S::ROWS * nhb; q += blockDim.x) {
    const int j = q / nhb, b = q % nhb;
    sc_sm[j][b] = j < nr ? G.hs[(size_t)(r0 + j) * nhb + b] * (1.0f / 256.0f) : 0.0f;
  }
  __syncthreads();

  // this wavefront's loads per K-step: weight blocks A_PER w .. (block q =
  // output rows cb + 16 q) and digit blocks B_PER w .. (block q = row group
  // q / 2, digit q % 2; rows past the tile re-read the tile's first row)
  const int8_t* W = static_cast<const int8_t*>(G.wdn);
  const int8_t* asrc[S::A_PER];
  const int8_t* bsrc[S::B_PER];
#pragma unroll
  for (int u = 0; u < S::A_PER; ++u) {
    const int col = cb + 16 * (S::A_PER * wave + u);
    const size_t row0 = (size_t)job.e * d + (col < d ? col : 0);
    asrc[u] = wblock_src<LAY>(W, row0, I, lane);
  }
#pragma unroll
  for (int u = 0; u < S::B_PER; ++u) {
    const int blk = S::B_PER * wave + u;
    const int j = 16 * (blk >> 1) + i;
    bsrc[u] = G.hq + (size_t)(r0 + (j < nr ? j : 0)) * 2 * I + (blk & 1) * I + 16 * g;
  }
  const int nsteps = I / kKStep;
  const int last = nsteps - 1;
  auto issue = [=](int8_t* slot, int step) {
    const int st = min(step, last);
#pragma unroll
    for (int u = 0; u < S::A_PER; ++u)
      lds_load16(asrc[u] + (size_t)st * wblock_step<LAY>(),
                 slot + (S::A_PER * wave + u) * kPBlk);
#pragma unroll
    for (int u = 0; u < S::B_PER; ++u)
      lds_load16(bsrc[u] + st * kKStep, slot + (S::NA + S::B_PER * wave + u) * kPBlk);
  };

  v4i p[NF][4][2];      // [weight fragment][row group][digit]: int32 sums of a 128-input block
  float acc[NF][4][4];  // fp32 sums over the blocks
  const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      p[f][t][0] = p[f][t][1] = zero4;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[f][t][c] = 0.0f;
    }

#pragma unroll
  for (int q = 0; q < S::NS - 1; ++q) issue(RING_SLOT(q), q);

  // PAR = the K-step's parity when the unrolling fixes it (4 slots): an even
  // step (0) opens a 128-input block, its MFMAs starting from zero so that the
  // int32 sums need no clearing, and an odd step (1) closes it and folds it
  // into fp32.  PAR = 2: parity known at run time only (3 slots; unrolling
  // those by 6 spills), the sums cleared after each fold.
// As in the gate/up GEMM, a wavefront with all four row groups valid runs a
// copy of the step without the per-row-group conditions (DN_FULL), so that
// its fragment reads need not wait for the previous group's MFMAs.
#define DN_STEP(STEP, Q, PAR) { if (ntg == 4) DN_STEP1(STEP, Q, PAR, true) else DN_STEP1(STEP, Q, PAR, false) }
#define DN_STEP1(STEP, Q, PAR, full)                                                          \
  {                                                                                           \
    MOE_WAIT_VM(S::WAIT);                                                                     \
    ring_barrier();                                                                           \
    if (active) {                                                                             \
      const int8_t* slot = RING_SLOT(Q);                                                      \
      v4i a[NF];                                                                              \
      _Pragma("unroll") for (int f = 0; f < NF; ++f)                                          \
        a[f] = lds_frag(slot + (NF * wc + f) * kPBlk, lane);                                  \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                         \
        if (full || t < ntg) {                                                                \
          const int8_t* bb = slot + (S::NA + 2 * (4 * wt + t)) * kPBlk;                       \
          const v4i b0 = lds_frag(bb, lane);                                                  \
          const v4i b1 = lds_frag(bb + kPBlk, lane);                                          \
          _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                    \
            p[f][t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b0,                      \
                                                               PAR ? p[f][t][0] : zero4, 0, 0, 0); \
            p[f][t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f], b1,                      \
                                                               PAR ? p[f][t][1] : zero4, 0, 0, 0); \
          }                                                                                   \
        }                                                                                     \
      }                                                                                       \
      if ((PAR == 1) || (PAR == 2 && ((STEP) & 1)) || (STEP) == last) { /* block end */       \
        const int blk = (STEP) >> 1;                                                          \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                       \
          if (full || t < ntg) {                                                              \
            const float sg = sc_sm[64 * wt + 16 * t + i][blk];                                \
            _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                  \
              _Pragma("unroll") for (int c = 0; c < 4; ++c)                                   \
                acc[f][t][c] = fmaf(sg, (float)(p[f][t][0][c] * 256 + p[f][t][1][c]),         \
                                    acc[f][t][c]);                                            \
              if (PAR == 2) p[f][t][0] = p[f][t][1] = zero4;                                  \
            }                                                                                 \
          }                                                                                   \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
    issue(RING_SLOT(((Q) + S::NS - 1) % S::NS), (STEP) + S::NS - 1);                          \
  }
  int s0 = 0;
  if constexpr (S::NS == 4) {
    for (; s0 + 4 <= nsteps; s0 += 4) {
      DN_STEP(s0, 0, 0)
      DN_STEP(s0 + 1, 1, 1)
      DN_STEP(s0 + 2, 2, 0)
      DN_STEP(s0 + 3, 3, 1)
    }
    if (s0 < nsteps) DN_STEP(s0, 0, 0)
    if (s0 + 1 < nsteps) DN_STEP(s0 + 1, 1, 1)
    if (s0 + 2 < nsteps) DN_STEP(s0 + 2, 2, 0)
  } else {
    for (; s0 + 3 <= nsteps; s0 += 3) {
      DN_STEP(s0, 0, 2)
      DN_STEP(s0 + 1, 1, 2)
      DN_STEP(s0 + 2, 2, 2)
    }
    if (s0 < nsteps) DN_STEP(s0, 0, 2)
    if (s0 + 1 < nsteps) DN_STEP(s0 + 1, 1, 2)
  }
#undef DN_STEP
#undef DN_STEP1
  MOE_WAIT_VM(0);
  if (!active) return;
  // lane (i, g) holds output columns c0 + 16 f + 4 g + c of tile row 64 wt + 16 t + i;
  // the output-row scales are loaded together and unconditionally (clamped
  // columns): conditional loads would each cost a round trip
  float sdv[NF][4];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int col = min(c0 + 16 * f, d - 16) + 4 * g;  // (d is a multiple of 16)
    const float4 v = *reinterpret_cast<const float4*>(G.sdn + (size_t)job.e * d + col);
    sdv[f][0] = v.x; sdv[f][1] = v.y; sdv[f][2] = v.z; sdv[f][3] = v.w;
  }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (c0 + 16 * f >= d) break;
    const float s0v = sdv[f][0], s1v = sdv[f][1], s2v = sdv[f][2], s3v = sdv[f][3];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = 64 * wt + 16 * t + i;
      if (t >= ntg || j >= nr) continue;
      *reinterpret_cast<float4*>(G.out + (size_t)(r0 + j) * d + c0 + 16 * f + 4 * g) =
          make_float4(s0v * acc[f][t][0], s1v * acc[f][t][1], s2v * acc[f][t][2],
                      s3v * acc[f][t][3]);
    }
  }
}
#undef RING_SLOT

// The down projection uses smaller tiles: up to 64 rows, a workgroup of 8
// wavefronts owning 128 output columns (16 per wavefront).  Its h scales
// change every 128 inputs (the gate/up GEMM writes one per row and 128-column
// block), so its K loop accumulates two K-steps of each digit in int32 on the
// matrix cores, joins the digits as 256 d0 + d1 (exact in int32) and folds
// that into fp32 with one multiply-add per output, holding 16 fp32 sums per
// lane; the smaller tile keeps registers low enough for two workgroups per CU.  The tile's h digits are staged in LDS 256
// inputs at a time (double-buffered); weight fragments and digits of chunk
// c+1 are loaded into registers while chunk c is computed.  All loads are
// unconditional (clamped addresses, masked values) so the compiler waits only
// for the loads a chunk consumes.
constexpr int kDRows = 64, kDChunk = 256;
constexpr int kDLdr = 2 * kDChunk + 16;           // LDS bytes per staged row
constexpr int kDStage = kDRows * 32 / (kPWaves * kWave);  // 16-byte pieces per thread

// Piece q = tid + 512 u of a chunk: row q / 32, digit (q % 32) / 16, bytes
// 16 (q % 16) of the chunk.  Source offsets are fixed per thread; rows past
// the tile and bytes past the end of the row are masked to zero.
struct DSrc {
  const int8_t* p[kDStage];
  int row_ok[kDStage];
  int col[kDStage];  // byte offset inside the chunk
};

__device__ inline DSrc dsrc_init(const int8_t* __restrict__ base, int rowbytes, int plane,
                                 int r0, int nr) {
  DSrc src;
#pragma unroll
  for (int u = 0; u < kDStage; ++u) {
    const int q = threadIdx.x + u * kPWaves * kWave;
    const int j = q >> 5, c = q & 31;
    src.row_ok[u] = j < nr;
    src.col[u] = 16 * (c & 15);
    src.p[u] = base + (size_t)(r0 + (j < nr ? j : 0)) * rowbytes + (c < 16 ? 0 : plane) + 16 * (c & 15);
  }
  return src;
}

struct DStage {
  v4i v[kDStage];
};

// chunk starting at input k0 with `valid` bytes (a multiple of 64) per digit row
__device__ inline void dstage_load(DStage& st, const DSrc& src, int k0, int valid) {
#pragma unroll
  for (int u = 0; u < kDStage; ++u) {
    const int off = src.col[u] < valid ? k0 : k0 - src.col[u];  // stay inside the row
    st.v[u] = *reinterpret_cast<const v4i*>(src.p[u] + off);
  }
}

__device__ inline void dstage_store(const DStage& st, const DSrc& src, int valid, int8_t* buf) {
#pragma unroll
  for (int u = 0; u < kDStage; ++u) {
    const int q = threadIdx.x + u * kPWaves * kWave;
    const int j = q >> 5, c = q & 31;
    const int m = (src.row_ok[u] && src.col[u] < valid) ? -1 : 0;
    *reinterpret_cast<v4i*>(buf + j * kDLdr + (c < 16 ? 0 : kDChunk) + 16 * (c & 15)) =
        st.v[u] & m;
  }
}

template <int LAY>
__global__ __launch_bounds__(512) void down_gemm64_kernel(Group g0, Group g1, int d) {
  __shared__ __attribute__((aligned(16))) int8_t bsm[2][kDRows * kDLdr];
  __shared__ float ssm[2][kDRows][kDChunk / 128];
  Job job;
  if (!find_job(g0, g1, kDRows, blockIdx.y, job)) return;
  const Group G = job.g == 0 ? g0 : g1;
  const int I = G.inter;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int c0 = blockIdx.x * 128 + wave * 16;
  const bool active = c0 < d;
  const int i = lane & 15, g = lane >> 4;
  const int r0 = job.r0, nr = job.nr;
  const int ntg = (nr + 15) / 16;
  const int nhb = (I + 127) / 128;  // h scale blocks per row
  const size_t row0 = (size_t)job.e * d + (active ? c0 : 0);
  const int8_t* wa = i8_operand_base<LAY>(static_cast<const int8_t*>(G.wdn), row0, I, i, g, lane);
  const DSrc src = dsrc_init(G.hq, 2 * I, I, r0, nr);
  // h scales: thread tid < 128 reads row tid / 2, block tid % 2 of a chunk
  // (divided by 256, exactly, for the joined digits)
  const int sj = (threadIdx.x >> 1) & (kDRows - 1), sb = threadIdx.x & 1;
  const bool s_ok = sj < nr;
  const float* sp = G.hs + (size_t)(r0 + (s_ok ? sj : 0)) * nhb;
  float acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[t][c] = 0.0f;
  const v4i zero = {0, 0, 0, 0};
  const int nchunk = (I + kDChunk - 1) / kDChunk;
  const int lastc = nchunk - 1;
  auto valid_of = [&](int c) { return min(kDChunk, I - c * kDChunk); };
  auto scale_of = [&](int c) {  // clamp the block index inside the row
    const int b = c * (kDChunk / 128) + sb;
    return sp[b < nhb ? b : nhb - 1] * (1.0f / 256.0f);
  };

  v4i ra[4];
  {
    const int nst = valid_of(0) / kKStep;
#pragma unroll
    for (int u = 0; u < 4; ++u) ra[u] = i8_load_cached<LAY>(wa, min(u, nst - 1));
    DStage st;
    dstage_load(st, src, 0, valid_of(0));
    const float sv = scale_of(0);
    dstage_store(st, src, valid_of(0), bsm[0]);
    if (threadIdx.x < kDRows * 2)
      ssm[0][sj][sb] = (s_ok && 2 * sb < nst) ? sv : 0.0f;
  }
  __syncthreads();

  for (int c = 0; c < nchunk; ++c) {
    const int nst = valid_of(c) / kKStep;
    const int c1 = min(c + 1, lastc);
    const int val1 = valid_of(c1), nst1 = val1 / kKStep;
    v4i na[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) na[u] = i8_load_cached<LAY>(wa, c1 * (kDChunk / kKStep) + min(u, nst1 - 1));
    DStage st;
    dstage_load(st, src, c1 * kDChunk, val1);
    const float sv = scale_of(c1);
    const int8_t* buf = bsm[c & 1];
    if (active) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {  // the chunk's two 128-input scale blocks
        const int u0 = 2 * pr;
        if (u0 < nst) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (t < ntg) {
              const int8_t* brow = buf + (16 * t + i) * kDLdr;
              v4i p0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                  ra[u0], *reinterpret_cast<const v4i*>(brow + 64 * u0 + 16 * g), zero, 0, 0, 0);
              v4i p1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                  ra[u0], *reinterpret_cast<const v4i*>(brow + kDChunk + 64 * u0 + 16 * g), zero,
                  0, 0, 0);
              if (u0 + 1 < nst) {
                p0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    ra[u0 + 1], *reinterpret_cast<const v4i*>(brow + 64 * (u0 + 1) + 16 * g), p0,
                    0, 0, 0);
                p1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    ra[u0 + 1],
                    *reinterpret_cast<const v4i*>(brow + kDChunk + 64 * (u0 + 1) + 16 * g), p1,
                    0, 0, 0);
              }
              const float sg = ssm[c & 1][16 * t + i][pr];
#pragma unroll
              for (int q = 0; q < 4; ++q)
                acc[t][q] = fmaf(sg, (float)(p0[q] * 256 + p1[q]), acc[t][q]);
            }
          }
        }
      }
    }
    if (c + 1 < nchunk) {
      dstage_store(st, src, val1, bsm[(c + 1) & 1]);
      if (threadIdx.x < kDRows * 2)
        ssm[(c + 1) & 1][sj][sb] = (s_ok && 2 * sb < nst1) ? sv : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) ra[u] = na[u];
    __syncthreads();
  }
  if (!active) return;
  const float* sd = G.sdn + (size_t)job.e * d + c0 + 4 * g;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = 16 * t + i;
    if (t >= ntg || j >= nr) continue;
    *reinterpret_cast<float4*>(G.out + (size_t)(r0 + j) * d + c0 + 4 * g) =
        make_float4(sd[0] * acc[t][0], sd[1] * acc[t][1], sd[2] * acc[t][2], sd[3] * acc[t][3]);
  }
}

// ------------------------------------------------------------------ layout conversion
// Row-major codes -> tiled codes (a byte permutation; see the layout note).
// One thread per 16-byte lane chunk of the tiled output.
template <int FMT>
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint8_t* __restrict__ src,
                                                           uint8_t* __restrict__ dst,
                                                           long long nrows, int K) {
  const long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // chunk id
  const int bytes_per_row = FMT == 1 ? K : K / 2;
  const long long nchunks = nrows * bytes_per_row / 16;
  if (q >= nchunks) return;
  const int lane = (int)(q % 64);
  const long long blk = q / 64;  // 1 KB block: (row group, step/span)
  const int per_group = FMT == 1 ? K / 64 : K / 128;
  const long long rg = blk / per_group;
  const int st = (int)(blk % per_group);
  const int i = lane & 15, g = lane >> 4;
  const uint8_t* row = src + (rg * 16 + i) * bytes_per_row;
  v4i v;
  if (FMT == 1) {
    v = *reinterpret_cast<const v4i*>(row + 64 * st + 16 * g);
  } else {
    const unsigned* p = reinterpret_cast<const unsigned*>(row + 64 * st + 4 * g);
    v = v4i{(int)p[0], (int)p[4], (int)p[8], (int)p[12]};
  }
  *reinterpret_cast<v4i*>(dst + 16 * q) = v;
}

// ------------------------------------------------------------------ fp32
// Plain fp32 weights: one wavefront per output column, lanes split the
// reduction, a fixed butterfly adds the lanes.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ W,
                                                      const float* __restrict__ act,
                                                      const int32_t* __restrict__ row_token,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int K, int N_out, int R, int actf,
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
    if (lane == 0) out[(size_t)r * N_out + n] = MODE == 0 ? act_f(actf, sa) * sb : sa;
  }
}

int g_cu_count = 256;

template <int FMT, int LAY, bool PAIRS>
hipError_t launch_pair(const Group& a, const Group& b, int d, int mt, const int8_t* xq,
                       const float* xs, const FfnWs& ws, hipStream_t s, const SelIn* sel) {
  const int tiles = a.tiles + b.tiles;
  const int imax = a.inter > b.inter ? a.inter : b.inter;
  // K split inside and across workgroups (plan.h); the C ABI ran the same plan
  // before anything was enqueued and refused one beyond the join area, so this
  // check cannot fail on a call that passed it
  FfnPlan plan{};
  plan_launches(FMT == 1 ? 1 : 2, a.tiles, b.tiles, imax, d, g_cu_count, PAIRS, plan);
  if (!plan.ok) return hipErrorInvalidValue;
  const int ks = plan.gu.ks;
  SplitK sk{plan.gu.n0, plan.gu.n1, ws.cnt, ws.part};
  const bool gsplit = sk.n0 > 1 || sk.n1 > 1;
  const size_t emax = (size_t)(a.E > b.E ? a.E : b.E) * sizeof(int);  // histogram
  // PAIRS: the expert histogram only (x digits come from L2); tiles: x rows
  const size_t lds_gu = PAIRS ? emax : (size_t)mt * (2 * d + 16);
  // SEL: the token's x digits (2d bytes) in the dynamic area
  const size_t lds_sel = lds_gu > (size_t)(2 * d) ? lds_gu : (size_t)(2 * d);
#define MOE_GU(KSV, SPL)                                                                   \
  do {                                                                                     \
    if (PAIRS && sel)                                                                      \
      moe_launch((gate_up_kernel<FMT, LAY, KSV, PAIRS, 1, SPL, PAIRS>), grid,              \
                 dim3(256 * KSV), lds_sel, s, a, b, d, mt, xq, xs, sk, *sel);              \
    else                                                                                   \
      moe_launch((gate_up_kernel<FMT, LAY, KSV, PAIRS, 1, SPL>), grid, dim3(256 * KSV),    \
                 lds_gu, s, a, b, d, mt, xq, xs, sk, SelIn{});                             \
  } while (0)
  {
    TimedLaunch tl(FMT == 1 ? K_FFN_I8_GATE_UP : K_FFN_I4_GATE_UP, s);
    dim3 grid(imax / 64, gsplit ? a.tiles * sk.n0 + b.tiles * sk.n1 : tiles);
    if (gsplit) {
      if (ks == 1) MOE_GU(1, PAIRS);
      else if (ks == 2) MOE_GU(2, PAIRS);
      else MOE_GU(4, PAIRS);
    } else {
      if (ks == 1) MOE_GU(1, false);
      else if (ks == 2) MOE_GU(2, false);
      else MOE_GU(4, false);
    }
  }
#undef MOE_GU
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int dks = plan.dn.ks;
  const bool ng2 = plan.dn.ng2;
  SplitK dsk{plan.dn.n0, plan.dn.n1, ws.cnt, ws.part};
  const bool dsplit = dsk.n0 > 1 || dsk.n1 > 1;
  const int dgy = dsplit ? a.tiles * dsk.n0 + b.tiles * dsk.n1 : tiles;
  // PAIRS: the expert histogram, then (int8, two row groups per wavefront)
  // the tile's h block scales
  const size_t lds_hs = (size_t)mt * (imax / 64) * sizeof(float);
  const size_t lds_dn = PAIRS ? (emax > lds_hs ? emax : lds_hs)
                              : (size_t)mt * (2 * imax + 16) + (size_t)mt * (imax / 64) * 4;
#define MOE_DN(KSV, NGV, SPL)                                                               \
  moe_launch((down_kernel<FMT, LAY, KSV, PAIRS, NGV, SPL>),                         \
                     dim3(d / (64 * NGV), dgy), dim3(256 * KSV), lds_dn, s, a, b, d, mt, dsk)
  TimedLaunch tl(FMT == 1 ? K_FFN_I8_DOWN : K_FFN_I4_DOWN, s);
  if (plan.dn.cg == 2)  // 32-column workgroups, 2 K slices, no split (plan.h)
    moe_launch((down_kernel<FMT, LAY, 2, PAIRS, 1, false, 2>), dim3(d / 32, tiles), dim3(256),
               lds_dn, s, a, b, d, mt, dsk);
  else if (ng2) MOE_DN(1, 2, false);
  else if (dsplit) {
    if (dks == 1) MOE_DN(1, 1, PAIRS);
    else if (dks == 2) MOE_DN(2, 1, PAIRS);
    else MOE_DN(4, 1, PAIRS);
  } else {
    if (dks == 1) MOE_DN(1, 1, false);
    else if (dks == 2) MOE_DN(2, 1, false);
    else MOE_DN(4, 1, false);
  }
#undef MOE_DN
  return hipGetLastError();
}


// ------------------------------------------------------------------ int4 grouped GEMM
// Prefill for int4 experts (blocks of 32 or 128 along the input), gate/up
// (DOWN = false) and down (DOWN = true) in one kernel shape: tiles of 64 rows
// of one expert x 512 weight rows (gate/up: 256 h columns as their gate and up
// rows; down: 512 output columns), 8 wavefronts of 64 rows x 64 weight rows
// (4 fragments of 16).  Per 128-input span a double-buffered LDS ring slot
// takes, straight from global memory (global_load_lds): the 32 weight blocks
// of the tiled layout (1 KB: 16 rows x 128 inputs), the tile's activation
// digits (x for gate/up, h for down; 2 KB per 16 rows and digit, in the int4
// digit order, laid out [half][lane][16 B] so that each lane reads its own
// 32 bytes without bank conflicts) and the weight rows' block scales.  The
// digits are the MFMA A operand (a lane's accumulators are 4 tile rows of one
// weight row, so it needs one weight scale per block); each block of 32
// inputs takes one 16x16x32 MFMA per digit on codes unpacked as 16 * code;
// the two int32 digit sums join as 256 p0 + p1 (exact) and fold into fp32
// with the block's scale raised to 2^-14 (block 128: the span's four blocks
// accumulate in int32 and fold once).  down also applies the h scale of the
// row and span (one per 128 h columns, written by the gate/up epilogue).
constexpr int k4Rows = 64;                        // tile rows
constexpr int k4Frags = 4;                        // weight fragments per wavefront
constexpr int k4NA = kPWaves * k4Frags;           // weight blocks per span (32)
constexpr int k4Cols = 16 * k4NA;                 // weight rows per workgroup (512)
constexpr int k4Dig = (k4Rows / 16) * 2 * 2048;   // digit bytes per span (16 KB)
constexpr int k4MaxSpans = 64;                    // h scales staged per row (I <= 8192)

template <int FMT>
struct G4Shape {
  static constexpr int SCB = FMT == 2 ? 16 : 4;   // scale bytes per weight row and span
  static constexpr int SC_OFF = k4NA * kPBlk + k4Dig;
  static constexpr int SLOT = SC_OFF + k4Cols * SCB;  // 56 KB (block 32), 50 KB (block 128)
};

// Direct global-to-LDS load of 4 bytes per lane: lane l's word lands at dst + 4 l.
__device__ inline void lds_load4(const void* src, int8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

template <int FMT, bool DOWN>
__global__ __launch_bounds__(512) void gemm4_kernel(Group g0, Group g1, int d,
                                                    const int8_t* __restrict__ xq,
                                                    const float* __restrict__ xs) {
  using S = G4Shape<FMT>;
  __shared__ __attribute__((aligned(16))) int8_t ring0[S::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t ring1[S::SLOT];
  __shared__ float red_max[kPWaves][k4Rows];
  __shared__ float hsc_sm[DOWN ? k4Rows : 1][DOWN ? k4MaxSpans : 1];
  __shared__ int tok_sm[k4Rows];
  Job job;
  if (!find_job(g0, g1, k4Rows, blockIdx.y, job)) return;
  // (the tile is uniform over the workgroup: scalar registers, scalar branches)
  job.g = __builtin_amdgcn_readfirstlane(job.g);
  job.e = __builtin_amdgcn_readfirstlane(job.e);
  job.r0 = __builtin_amdgcn_readfirstlane(job.r0);
  job.nr = __builtin_amdgcn_readfirstlane(job.nr);
  const Group G = job.g == 0 ? g0 : g1;
  const int I = G.inter;
  const int K = DOWN ? I : d;                      // inputs of the product
  const int N = DOWN ? d : I;                      // output columns (gate/up: h columns)
  const int cb = blockIdx.x * (DOWN ? k4Cols : k4Cols / 2);
  if (cb >= N) return;
  // (wave-uniform values go to scalar registers: the load addresses below
  // are a scalar base plus the lane's offset)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, g = lane >> 4;
  const int r0 = job.r0, nr = job.nr;
  const int ntg = min(4, (nr + 15) / 16);           // row groups holding tile rows
  const int nsp = K / 128;                          // spans
  const int nb = FMT == 2 ? K / 32 : K / 128;       // scale blocks per weight row
  for (int j = threadIdx.x; j < k4Rows; j += blockDim.x)
    tok_sm[j] = j < nr ? (DOWN ? r0 + j : (G.row_token ? G.row_token[r0 + j] : r0 + j)) : -1;
  if (DOWN) {  // h scale of each tile row and span, with the 1/256 of the digit join
    for (int q = threadIdx.x; q < k4Rows * nsp; q += blockDim.x) {
      const int j = q / nsp, m = q % nsp;
      hsc_sm[j][m] = j < nr ? G.hs[(size_t)(r0 + j) * nsp + m] * (1.0f / 256.0f) : 0.0f;
    }
  }
  __syncthreads();

  // weight row of local column jc (gate/up: jc < 256 gate rows cb + jc, then the
  // up rows I + cb + jc - 256; down: output rows cb + jc), clamped into the matrix
  auto wrow = [=](int jc) {
    if (DOWN) return min(cb + jc, N - 1);
    const int h = min(cb + (jc & 255), N - 1);
    return jc < 256 ? h : I + h;
  };
  const uint8_t* W = static_cast<const uint8_t*>(DOWN ? G.wdn : G.wgu);
  const float* SC = DOWN ? G.sdn : G.sgu;
  const size_t wrows = DOWN ? (size_t)d : (size_t)2 * I;   // weight rows per expert
  // this wavefront's loads per span: weight blocks 4w..4w+3, digit chunks 2w, 2w+1
  // (chunk c: row group c/4, digit (c/2)%2, half c%2), scale chunk w (64 rows)
  const uint8_t* asrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int blk = 4 * wave + u;  // 16 weight rows from local column 16 blk
    // (N and I are multiples of 128: a clamped block start stays 16-row aligned)
    asrc[u] = W + ((size_t)job.e * wrows + (wrow(16 * blk) & ~15)) * (K / 2) + 16 * lane;
  }
  const int8_t* bsrc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = 2 * wave + u;
    const int j = 16 * (c >> 2) + i;
    const int row = tok_sm[j] >= 0 ? tok_sm[j] : tok_sm[0];
    const int8_t* base = DOWN ? G.hq + (size_t)row * 2 * I : xq + (size_t)row * 2 * d;
    bsrc[u] = base + ((c >> 1) & 1) * K + 32 * g + 16 * (c & 1);
  }
  const float* ssrc = SC + ((size_t)job.e * wrows + wrow(64 * wave + lane)) * nb;
  // part 0, 1: two weight blocks each; 2: the digit chunks; 3: the scales.  The
  // parts of the next span are issued between the current span's fragments:
  // a wavefront that issues all seven loads at once stalls until the CU's
  // memory pipeline takes them, and the span's arithmetic waits with it
  auto issue = [&](int8_t* slot, int m, int part) {
    const int ms = min(m, nsp - 1);
    if (part < 2) {
#pragma unroll
      for (int u = 2 * part; u < 2 * part + 2; ++u)
        lds_load16(asrc[u] + (size_t)ms * 1024, slot + (4 * wave + u) * kPBlk);
    } else if (part == 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        lds_load16(bsrc[u] + 128 * ms, slot + k4NA * kPBlk + (2 * wave + u) * kPBlk);
    } else {
      if constexpr (FMT == 2) lds_load16(ssrc + 4 * ms, slot + S::SC_OFF + wave * 1024);
      else lds_load4(ssrc + ms, slot + S::SC_OFF + wave * 256);
    }
  };

  // this wavefront's fragments: gate/up: gate blocks 2w, 2w+1 and the up blocks
  // 16 + 2w, 17 + 2w (the same h columns); down: blocks 4w..4w+3
  int fblk[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) fblk[f] = DOWN ? 4 * wave + f : (f < 2 ? 2 * wave + f : 14 + 2 * wave + f);
  const int c0 = DOWN ? cb + 64 * wave : cb + 32 * wave;  // first output column of the wavefront
  const bool active = c0 < N;
  float acc[4][4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[f][t][c] = 0.0f;
  const v4i zero = {0, 0, 0, 0};

  // the span loop unrolled by two, so that each slot is a known LDS array
#define G4_SPAN(CUR, NXT, M) \
  { \
    MOE_WAIT_VM(0); /* this span's loads, issued during the last span */ \
    ring_barrier(); \
    { \
  /* the span's digits of every row group in registers (rows past the tile */ \
  /* are real rows again; their results are never stored), then one weight */ \
  /* fragment at a time: unpack, then its MFMAs and folds for each row group */ \
  /* (block 32: every (fragment, row group) reads its digits from LDS again, */ \
  /* which keeps its registers below the 256 of two wavefronts per SIMD) */ \
      constexpr int XT = FMT == 2 ? 1 : 4;  /* row groups whose digits stay in registers */ \
      long x0[XT][4], x1[XT][4];  /* [row group][block], digit 0 and 1 */ \
      float hs4[4][4];  /* down: h scale (with 1/256) of tile row 16 t + 4 g + c */ \
      auto load_digits = [&](int t, long* d0, long* d1) { \
        const int8_t* db = (CUR) + k4NA * kPBlk + 4 * t * kPBlk;  /* chunks (t, digit, half) */ \
        const v2l a0 = *reinterpret_cast<const v2l*>(db + 16 * lane); \
        const v2l a1 = *reinterpret_cast<const v2l*>(db + kPBlk + 16 * lane); \
        const v2l b0 = *reinterpret_cast<const v2l*>(db + 2 * kPBlk + 16 * lane); \
        const v2l b1 = *reinterpret_cast<const v2l*>(db + 3 * kPBlk + 16 * lane); \
        d0[0] = a0.x; d0[1] = a0.y; d0[2] = a1.x; d0[3] = a1.y; \
        d1[0] = b0.x; d1[1] = b0.y; d1[2] = b1.x; d1[3] = b1.y; \
      }; \
_Pragma("unroll") \
      for (int t = 0; t < 4; ++t) { \
        if (XT == 4) load_digits(t, x0[t % XT], x1[t % XT]); \
_Pragma("unroll") \
        for (int c = 0; c < 4; ++c) hs4[t][c] = DOWN ? hsc_sm[16 * t + 4 * g + c][(M)] : 1.0f; \
      } \
_Pragma("unroll") \
      for (int f = 0; f < 4; ++f) { \
       if (active) { \
        long wq[4];  /* unpacked weight codes of the fragment's 4 blocks */ \
        float sc[4];  /* their scales, raised to 2^-14, with the 1/16 of the unpacking */ \
        { \
          const v4i w = lds_frag((CUR) + fblk[f] * kPBlk, lane); \
_Pragma("unroll") \
          for (int q = 0; q < 4; ++q) wq[q] = unpack8_int4_x16((unsigned)w[q]); \
          if constexpr (FMT == 2) { \
            const v4f sv = *reinterpret_cast<const v4f*>((CUR) + S::SC_OFF + (16 * fblk[f] + i) * 16); \
_Pragma("unroll") \
            for (int q = 0; q < 4; ++q) sc[q] = fmaxf(sv[q], kScaleFloor) * kInv16; \
          } else { \
            sc[0] = fmaxf(*reinterpret_cast<const float*>((CUR) + S::SC_OFF + (16 * fblk[f] + i) * 4), \
                          kScaleFloor) * kInv16; \
          } \
        } \
_Pragma("unroll") \
        for (int t = 0; t < 4; ++t) { \
          if (t >= ntg) break; \
          if constexpr (FMT == 2) { \
            load_digits(t, x0[0], x1[0]); \
  /* the span's four blocks summed with their scales, then (down) times */ \
  /* the rows' h scales: sum_m hs[row][m] sum_q s[col][q] p_q */ \
            float sp[4] = {0.0f, 0.0f, 0.0f, 0.0f}; \
_Pragma("unroll") \
            for (int q = 0; q < 4; ++q) { \
              const v4i p0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(x0[0][q], wq[q], zero, 0, 0, 0); \
              const v4i p1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(x1[0][q], wq[q], zero, 0, 0, 0); \
_Pragma("unroll") \
              for (int c = 0; c < 4; ++c) sp[c] = fmaf(sc[q], (float)(p0[c] * 256 + p1[c]), sp[c]); \
            } \
_Pragma("unroll") \
            for (int c = 0; c < 4; ++c) \
              acc[f][t][c] = DOWN ? fmaf(hs4[t][c], sp[c], acc[f][t][c]) : acc[f][t][c] + sp[c]; \
 \
          } else { \
            /* one scale for the span: blocks 0, 1 and 2, 3 go through the 16x16x64 */ \
            /* MFMA in pairs (a lane's K values of two blocks side by side in A and */ \
            /* B; the 16x16x32 form takes as long on this chip for half the work) */ \
            v4i p0 = zero, p1 = zero; \
_Pragma("unroll") \
            for (int q = 0; q < 4; q += 2) { \
              const v4i wv = {(int)wq[q], (int)(wq[q] >> 32), (int)wq[q + 1], (int)(wq[q + 1] >> 32)}; \
              const long* xa = x0[t % XT]; \
              const long* xb = x1[t % XT]; \
              const v4i av = {(int)xa[q], (int)(xa[q] >> 32), (int)xa[q + 1], (int)(xa[q + 1] >> 32)}; \
              const v4i bv = {(int)xb[q], (int)(xb[q] >> 32), (int)xb[q + 1], (int)(xb[q + 1] >> 32)}; \
              p0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, wv, p0, 0, 0, 0); \
              p1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, wv, p1, 0, 0, 0); \
            } \
_Pragma("unroll") \
            for (int c = 0; c < 4; ++c) {  /* |p0| < 2^22: each digit sum exact in fp32 */ \
              const float v = fmaf((float)p0[c], 256.0f, (float)p1[c]); \
              acc[f][t][c] = fmaf(DOWN ? sc[0] * hs4[t][c] : sc[0], v, acc[f][t][c]); \
            } \
          } \
        } \
       } /* active */ \
        issue(NXT, (M) + 1, f); /* (the last span re-reads a span) */ \
      } \
    } \
    ring_barrier();  /* every wavefront is done with CUR before it is refilled */ \
 \
  }
#pragma unroll
  for (int part = 0; part < 4; ++part) issue(ring0, 0, part);
  int m = 0;
  for (; m + 2 <= nsp; m += 2) {
    G4_SPAN(ring0, ring1, m)
    G4_SPAN(ring1, ring0, m + 1)
  }
  if (m < nsp) G4_SPAN(ring0, ring1, m)
#undef G4_SPAN
  MOE_WAIT_VM(0);

  if constexpr (DOWN) {
    if (!active) return;
    // lane (i, g) holds tile rows 16 t + 4 g + c of output column c0 + 16 f + i
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int col = c0 + 16 * f + i;
      if (col >= N) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 16 * t + 4 * g + c;
          if (j < nr) G.out[(size_t)(r0 + j) * d + col] = acc[f][t][c];
        }
    }
  } else {
    // h = act(gate) * up for tile rows 16 t + 4 g + c, h column c0 + 16 fq + i
    // (fq = 0, 1; gate in fragments 0, 1, up in 2, 3), encoded as two digits per
    // row and 128-column span (the span's four wavefronts meet in red_max); the
    // digits go through LDS (the ring, free now) so that rows are stored in
    // 16-byte pieces, in the int4 digit order the down kernel reads
    float h[2][4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float sig[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int tj = tok_sm[16 * t + 4 * g + c];
        sig[c] = xs[tj >= 0 ? tj : tok_sm[0]] * (1.0f / 256.0f);
      }
      float mx[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mx[c] = 0.0f;
#pragma unroll
        for (int fq = 0; fq < 2; ++fq) {
          const bool ok = active && c0 + 16 * fq + i < N;
          const float gt = acc[fq][t][c] * sig[c], up = acc[2 + fq][t][c] * sig[c];
          h[fq][t][c] = ok ? act_f(G.act, gt) * up : 0.0f;
          mx[c] = fmaxf(mx[c], fabsf(h[fq][t][c]));
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx[c] = fmaxf(mx[c], __shfl_xor(mx[c], o, kWave));
      }
      if (i == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) red_max[wave][16 * t + 4 * g + c] = mx[c];
      }
    }
    __syncthreads();
    // staging [row][digit][256 bytes] in ring0 (32 KB of its 56 / 50 KB)
    int8_t* stg = ring0;
    const int sp = wave >> 2;  // this wavefront's 128-column span within the 256
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 16 * t + 4 * g + c;
        const float m = fmaxf(fmaxf(red_max[4 * sp][j], red_max[4 * sp + 1][j]),
                              fmaxf(red_max[4 * sp + 2][j], red_max[4 * sp + 3][j]));
        const int p = digit_exponent(m);
#pragma unroll
        for (int fq = 0; fq < 2; ++fq) {
          int d0, d1;
          two_digits(h[fq][t][c], p, d0, d1);
          const int lc = 32 * wave + 16 * fq + i;  // column within the 256
          const int pos = 128 * (lc >> 7) + int4_digit_pos(lc & 127);
          stg[j * 512 + pos] = (int8_t)d0;
          stg[j * 512 + 256 + pos] = (int8_t)d1;
        }
        if ((wave & 3) == 0 && i == 0 && j < nr && cb + 128 * sp < N)
          G.hs[(size_t)(r0 + j) * (I / 128) + (cb >> 7) + sp] = m > 0.0f ? ldexpf(1.0f, -p) : 0.0f;
      }
    __syncthreads();
    const int valid = min(256, N - cb);  // bytes per digit row inside the matrix
    for (int q = threadIdx.x; q < k4Rows * 2 * 16; q += blockDim.x) {
      const int j = q >> 5, dg = (q >> 4) & 1, ch = q & 15;
      if (j >= nr || 16 * ch >= valid) continue;
      *reinterpret_cast<v4i*>(G.hq + (size_t)(r0 + j) * 2 * I + dg * I + cb + 16 * ch) =
          *reinterpret_cast<const v4i*>(stg + j * 512 + dg * 256 + 16 * ch);
    }
  }
}

}  // namespace

void set_device_info(int cu_count) { g_cu_count = cu_count > 0 ? cu_count : 256; }
int device_cu_count() { return g_cu_count; }

hipError_t launch_encode_rows(const float* v, int n, int K, int8_t* q, float* sig, bool perm,
                              int* split_cnt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimedLaunch tl(K_ENCODE_ROWS, s);
  moe_launch(encode_rows_kernel, dim3((n + 3) / 4), dim3(256), 0, s, v, n, K, q, sig,
                     perm, split_cnt);
  return hipGetLastError();
}

hipError_t launch_tile_weights(int fmt, const void* src, void* dst, long long nrows, int K,
                               hipStream_t s) {
  const long long chunks = nrows * (fmt == 1 ? K : K / 2) / 16;
  if (chunks <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((chunks + 255) / 256);
  if (fmt == 1)
    moe_launch(tile_weights_kernel<1>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), nrows, K);
  else
    moe_launch(tile_weights_kernel<2>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), nrows, K);
  return hipGetLastError();
}

template <int LAY>
hipError_t launch_gemm_pair(Group a, Group b, int d, const int8_t* xq, const float* xs,
                            hipStream_t s) {
  auto tiles_of = [](const Group& G, int mt) {
    if (G.R <= 0) return 0;
    return G.offsets ? max_tiles(G.R, G.E, mt) : (G.R + mt - 1) / mt;
  };
  const int imax = a.inter > b.inter ? a.inter : b.inter;
  // gate/up: 64-row tiles x 256 columns below 96 rows per expert on average,
  // else 128-row tiles x 128 columns
  const bool tall = a.R >= 96LL * a.E;
  const int act = a.act;  // the layer's activation, the same for both sets
  {
    TimedLaunch tl(K_FFN_I8_GATE_UP_GEMM, s);
    if (tall) {
      using S = GuShape<2>;
      a.tiles = tiles_of(a, S::ROWS);
      b.tiles = tiles_of(b, S::ROWS);
      if (act == 1)
        moe_launch((gate_up_gemm_kernel<LAY, 2, 1>), dim3((imax + S::COLS - 1) / S::COLS,
                           a.tiles + b.tiles), dim3(kPWaves * kWave), 0, s, a, b, d, xq, xs);
      else
        moe_launch((gate_up_gemm_kernel<LAY, 2, 0>), dim3((imax + S::COLS - 1) / S::COLS,
                           a.tiles + b.tiles), dim3(kPWaves * kWave), 0, s, a, b, d, xq, xs);
    } else {
      using S = GuShape<1>;
      a.tiles = tiles_of(a, S::ROWS);
      b.tiles = tiles_of(b, S::ROWS);
      if (act == 1)
        moe_launch((gate_up_gemm_kernel<LAY, 1, 1>), dim3((imax + S::COLS - 1) / S::COLS,
                           a.tiles + b.tiles), dim3(kPWaves * kWave), 0, s, a, b, d, xq, xs);
      else
        moe_launch((gate_up_gemm_kernel<LAY, 1, 0>), dim3((imax + S::COLS - 1) / S::COLS,
                           a.tiles + b.tiles), dim3(kPWaves * kWave), 0, s, a, b, d, xq, xs);
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  TimedLaunch tl(K_FFN_I8_DOWN_GEMM, s);
  if (imax <= 128 * kDnMaxBlocks) {  // block scales staged in LDS: I <= 4096
    if (tall) {
      using S = DnShape<2, kDnFrags>;
      a.tiles = tiles_of(a, S::ROWS);
      b.tiles = tiles_of(b, S::ROWS);
      moe_launch((down_gemm_kernel<LAY, 2, kDnFrags>), dim3((d + S::COLS - 1) / S::COLS,
                         a.tiles + b.tiles), dim3(kPWaves * kWave), 0, s, a, b, d);
    } else {
      using S = DnShape<1, kDnFrags>;
      a.tiles = tiles_of(a, S::ROWS);
      b.tiles = tiles_of(b, S::ROWS);
      moe_launch((down_gemm_kernel<LAY, 1, kDnFrags>), dim3((d + S::COLS - 1) / S::COLS,
                         a.tiles + b.tiles), dim3(kPWaves * kWave), 0, s, a, b, d);
    }
    return hipGetLastError();
  }
  a.tiles = tiles_of(a, kDRows);
  b.tiles = tiles_of(b, kDRows);
  moe_launch(down_gemm64_kernel<LAY>, dim3((d + 127) / 128, a.tiles + b.tiles),
                     dim3(kPWaves * kWave), 0, s, a, b, d);
  return hipGetLastError();
}

// int4 grouped GEMM pair (gemm4_kernel): gate/up, then down.
template <int FMT>
hipError_t launch_gemm4_pair(Group a, Group b, int d, const int8_t* xq, const float* xs,
                             hipStream_t s) {
  auto tiles_of = [](const Group& G) {
    if (G.R <= 0) return 0;
    return G.offsets ? max_tiles(G.R, G.E, k4Rows) : (G.R + k4Rows - 1) / k4Rows;
  };
  a.tiles = tiles_of(a);
  b.tiles = tiles_of(b);
  const int imax = a.inter > b.inter ? a.inter : b.inter;
  const int tiles = a.tiles + b.tiles;
  {
    TimedLaunch tl(K_FFN_I4_GATE_UP_GEMM, s);
    moe_launch((gemm4_kernel<FMT, false>), dim3((imax + k4Cols / 2 - 1) / (k4Cols / 2),
                       tiles), dim3(kPWaves * kWave), 0, s, a, b, d, xq, xs);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  TimedLaunch tl(K_FFN_I4_DOWN_GEMM, s);
  moe_launch((gemm4_kernel<FMT, true>), dim3((d + k4Cols - 1) / k4Cols, tiles),
                     dim3(kPWaves * kWave), 0, s, a, b, d, xq, xs);
  return hipGetLastError();
}

hipError_t launch_ffn_quant(const FfnSet* sets, int nsets, int d, const float* x, int T,
                            const FfnWs& ws, bool x_encoded, hipStream_t s, const SelIn* sel) {
  hipError_t err = hipSuccess;
  if (!x_encoded) {
    // int4 kernels read the digits in their permuted order (encode8)
    err = launch_encode_rows(x, T, d, ws.xq, ws.xs, sets[0].fmt != 1, ws.cnt, s);
    if (err != hipSuccess) return err;
  }
  // int4 (tiled codes) with many rows per expert: the int4 grouped GEMM
  const int imax4 = nsets > 1 && sets[1].inter > sets[0].inter ? sets[1].inter : sets[0].inter;
  if (sets[0].fmt != 1 && sets[0].layout == 1 && sets[0].pairs_idx == nullptr &&
      sets[0].R >= 16LL * sets[0].E && imax4 <= 128 * k4MaxSpans) {
    Group grp[2] = {};
    for (int q = 0; q < nsets; ++q) {
      const FfnSet& f = sets[q];
      Group& G = grp[q];
      G.E = f.E; G.inter = f.inter; G.R = f.R;
      G.wgu = f.wgu; G.sgu = f.sgu; G.wdn = f.wdn; G.sdn = f.sdn;
      G.row_token = f.row_token; G.offsets = f.offsets;
      G.hq = f.hq; G.hs = f.hs; G.out = f.out; G.act = f.act;
    }
    if (nsets < 2) grp[1].inter = grp[0].inter;
    return sets[0].fmt == 2 ? launch_gemm4_pair<2>(grp[0], grp[1], d, ws.xq, ws.xs, s)
                            : launch_gemm4_pair<3>(grp[0], grp[1], d, ws.xq, ws.xs, s);
  }
  // int8 with many rows per expert: grouped GEMM
  if (sets[0].fmt == 1 && sets[0].pairs_idx == nullptr && sets[0].R >= 16LL * sets[0].E) {
    Group grp[2] = {};
    for (int q = 0; q < nsets; ++q) {
      const FfnSet& f = sets[q];
      Group& G = grp[q];
      G.E = f.E; G.inter = f.inter; G.R = f.R;
      G.wgu = f.wgu; G.sgu = f.sgu; G.wdn = f.wdn; G.sdn = f.sdn;
      G.row_token = f.row_token; G.offsets = f.offsets;
      G.hq = f.hq; G.hs = f.hs; G.out = f.out; G.act = f.act;
    }
    if (nsets < 2) grp[1].inter = grp[0].inter;
    return sets[0].layout == 1 ? launch_gemm_pair<kTiled>(grp[0], grp[1], d, ws.xq, ws.xs, s)
                               : launch_gemm_pair<kRows>(grp[0], grp[1], d, ws.xq, ws.xs, s);
  }
  // rows per tile (plan.h): at most 16, fewer for small batches and wide rows
  int inters[2] = {sets[0].inter, nsets > 1 ? sets[1].inter : 0};
  const int mt = ffn_tile_rows(T, d, nsets, inters);
  if (mt < 1) return hipErrorInvalidValue;
  Group grp[2] = {};
  for (int q = 0; q < nsets; ++q) {
    const FfnSet& f = sets[q];
    Group& G = grp[q];
    G.E = f.E;
    G.inter = f.inter;
    G.R = f.R;
    G.tiles = f.offsets ? max_tiles(f.R, f.E, mt) : (f.R + mt - 1) / mt;
    G.wgu = f.wgu;
    G.sgu = f.sgu;
    G.wdn = f.wdn;
    G.sdn = f.sdn;
    G.row_token = f.row_token;
    G.offsets = f.offsets;
    G.hq = f.hq;
    G.hs = f.hs;
    G.out = f.out;
    G.pairs_idx = f.pairs_idx;
    G.k = f.k;
    G.act = f.act;
  }
  if (nsets < 2) grp[1].inter = grp[0].inter;
  const bool tiled = sets[0].layout == 1;
  const bool pairs = sets[0].pairs_idx != nullptr || (nsets > 1 && sets[1].pairs_idx != nullptr);
#define MOE_PAIR(F, L)                                                               \
  (pairs ? launch_pair<F, L, true>(grp[0], grp[1], d, mt, ws.xq, ws.xs, ws, s, sel)  \
         : launch_pair<F, L, false>(grp[0], grp[1], d, mt, ws.xq, ws.xs, ws, s, nullptr))
  if (sets[0].fmt == 1) return tiled ? MOE_PAIR(1, kTiled) : MOE_PAIR(1, kRows);
  if (sets[0].fmt == 3) return tiled ? MOE_PAIR(3, kTiled) : MOE_PAIR(3, kRows);
  return tiled ? MOE_PAIR(2, kTiled) : MOE_PAIR(2, kRows);
#undef MOE_PAIR
}

hipError_t launch_ffn_f32(const float* wgu, const float* wdn, int E, int d, int inter,
                          const float* x, int T, const int32_t* row_token,
                          const int32_t* offsets, int R, float* rows_out, float* h, int act,
                          hipStream_t s) {
  (void)T;
  const int tiles = offsets ? max_tiles(R, E, kTileRows) : (R + kTileRows - 1) / kTileRows;
  {
    TimedLaunch tl(K_FFN_F32_GATE_UP, s);
    moe_launch(ffn_f32_kernel<0>, dim3((inter + 3) / 4, tiles), dim3(256), 0, s, wgu,
                       x, row_token, offsets, E, d, inter, R, act, h);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  TimedLaunch tl(K_FFN_F32_DOWN, s);
  moe_launch(ffn_f32_kernel<1>, dim3((d + 3) / 4, tiles), dim3(256), 0, s, wdn, h,
                     row_token, offsets, E, inter, d, R, 0, rows_out);
  return hipGetLastError();
}

}  // namespace moe
