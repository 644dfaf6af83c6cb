// Launch planning of the small-batch FFN kernels: tile height, K split inside
// a workgroup, and K split across workgroups with its join area.  Plain host
// C++ (no HIP types), so that the argument checks of the C ABI can run the
// same plan before anything is enqueued, and so that a CPU test can sweep it.
#pragma once

#include <stddef.h>

namespace moe {

constexpr int kPlanKStep = 64;        // K of one int8 MFMA (16x16x64)
constexpr int kPlanTileRows = 16;     // routed rows per decode FFN tile (MFMA N)
constexpr size_t kPlanLdsBytes = 160 * 1024;

// Decode launches with fewer work units than the chip has CUs (or a few more)
// split K across workgroups: unit u's n workgroups write partial sums into
// slots u*n .. u*n+n-1 and the last to arrive adds them in slot order.
constexpr int kSplitSlots = 1024;
constexpr size_t kSplitSlotBytes = 16384;

// One token whose gate/up launch selects and encodes for itself: each of at
// least 256 threads holds at most two groups of 8 inputs of the x row.
inline bool sel_fits(int d) { return d % 8 == 0 && d <= 2 * 256 * 8; }

// Upper bound on the number of FFN tiles (mt rows of one expert each) for R
// rows spread over E experts: sum_e ceil(c_e/mt) <= n + (R - n)/mt with
// n = min(E, R) non-empty experts at most.
inline int max_tiles(int R, int E, int mt) {
  int n = R < E ? R : E;
  return n + (R - n + mt - 1) / mt;
}

// Rows per decode tile: at most 16 (the MFMA N side); small batches use
// fewer; wide rows use fewer so that a tile's staged rows (x digits for
// gate/up, h digits and block scales for down) fit the LDS beside the
// kernels' largest static arrays (the K-slice partials, under 50 KB).
// Returns 0 if not even one row fits (not reachable for widths <= 16384).
inline int ffn_tile_rows(int T, int d, int nsets, const int* inter) {
  int mt = T < kPlanTileRows ? (T > 0 ? T : 1) : kPlanTileRows;
  size_t per_row = (size_t)2 * d + 16;
  for (int q = 0; q < nsets; ++q) {
    const size_t dn = (size_t)2 * inter[q] + 16 + (size_t)(inter[q] / 64) * 4;
    if (dn > per_row) per_row = dn;
  }
  const size_t cap = (kPlanLdsBytes - 50 * 1024) / per_row;
  if (cap < 1) return 0;
  if ((size_t)mt > cap) mt = (int)cap;
  return mt;
}

// Workgroups per work unit (K split) for a launch of `units` units on `cus`
// CUs: the time of a launch follows its busiest CU, ceil(units n / CUs)
// workgroups of 1/n unit each plus a fixed cost per workgroup (tile lookup,
// the first loads' latency, the join through device-coherent memory; about
// half a unit's streaming at decode sizes, measured), so n = 1 unless CUs
// would sit idle.  Each wavefront keeps at least min_steps K-steps, and the
// slots never exceed the join area.
inline int split_ways(long long units, int ksteps_per_wave_at_1, int min_steps, long long cus) {
  int best = 1;
  double best_cost = 1e30;
  for (int n = 1; n <= 8; ++n) {
    if (n > 1 && (units * n > kSplitSlots || ksteps_per_wave_at_1 / n < min_steps)) break;
    const double waves = (double)((units * n + cus - 1) / cus);
    const double cost = waves * (1.0 / n + 0.5);
    if (cost < best_cost * 0.97) {
      best_cost = cost;
      best = n;
    }
  }
  return best;
}

// Whether a split plan fits the join area: kSplitSlots arrival counts (one
// per unit of the launch) and kSplitSlots partial-sum slots (n per unit of
// each group that splits).
inline bool split_fits(long long u0, int n0, long long u1, int n1) {
  if (n0 < 1 || n1 < 1 || u0 < 0 || u1 < 0) return false;
  if (n0 == 1 && n1 == 1) return true;
  const long long slots = (n0 > 1 ? u0 * n0 : 0) + (n1 > 1 ? u1 * n1 : 0);
  return slots <= kSplitSlots && u0 + u1 <= kSplitSlots;
}

// Split plan for a launch of t0 + t1 tiles (groups 0 and 1) x gx column
// units: every unit alike (n0 = n1 from split_ways) when CUs would otherwise
// sit idle; else, when group 0's units fit the chip and group 1's spill over
// it (e.g. 256 routed units and the shared expert's 32 at one token), group 1
// alone splits into small workgroups, enough for every other CU to take one
// beside its group-0 unit (Kimi-shaped gate/up at one token, 32 shared units:
// 4 ways 21.7 us, 8 ways 23.4 us, 2 ways 23.9 us, event-timed).  kpw: K-steps
// per wavefront unsplit.  Returns false when the join area cannot hold the
// plan's slots and counts.
inline bool plan_split(long long t0, long long t1, int gx, int kpw, int min_steps, long long cus,
                       int& n0, int& n1) {
  const long long u0 = t0 * gx, u1 = t1 * gx;
  n0 = n1 = split_ways(u0 + u1, kpw, min_steps, cus);
  if (n0 == 1 && u1 > 0 && u0 <= cus && u0 + u1 > cus) {
    int n = (int)((cus + 2 * u1 - 1) / (2 * u1));
    n = n < 8 ? n : 8;
    while (n > 1 && (kpw / n < min_steps || u1 * n > kSplitSlots)) --n;
    n1 = n < 1 ? 1 : n;
  }
  return split_fits(u0, n0, u1, n1);
}

// The two launches (gate/up, then down) of the decode FFN kernels.
//   ks: wavefronts per 16 columns, each taking a K slice (1, 2 or 4)
//   n0, n1: workgroups per work unit of group 0 / group 1 (K split across
//           workgroups; only small batches, whose pairs the kernels group
//           themselves, split)
//   ng2 (down only): two 64-column blocks per workgroup
//   cg (down only): 16-column groups per workgroup (4, or 2 for a finer grid)
struct LaunchSplit {
  int ks, n0, n1;
  bool ng2;
  int cg;
};
struct FfnPlan {
  int mt;  // rows per tile
  long long tiles0, tiles1;
  LaunchSplit gu, dn;
  bool ok;  // false: the plan does not fit the join area (nothing may be launched)
};

// fmt: 1 int8, 2 int4 block 32, 3 int4 block 128.  imax: the larger
// intermediate width of the two groups.
inline void plan_launches(int fmt, long long tiles0, long long tiles1, int imax, int d,
                          long long cus, bool pairs, FfnPlan& p) {
  p.tiles0 = tiles0;
  p.tiles1 = tiles1;
  const long long tiles = tiles0 + tiles1;
  // split K across more wavefronts when the tiles alone cannot fill the chip:
  // 4 ways (1024-thread workgroups, one per CU) while the units fit one per
  // CU for int4, whose waves stream half the bytes per K-step (measured:
  // Qwen-shaped T = 2 gate/up 20.6 -> 17.4 us; past one round it lost);
  // int8 takes 4 ways only below half the CUs (4 ways at 288 units lost)
  const auto kway = [&](long long units) {
    if (units >= 2LL * cus) return 1;
    const long long four_below = fmt == 1 ? cus / 2 : cus + 1;
    return units < four_below ? 4 : 2;
  };
  p.ok = true;
  p.gu.ks = kway(tiles * (imax / 64));
  p.gu.n0 = p.gu.n1 = 1;
  p.gu.ng2 = false;
  p.gu.cg = 4;
  const int ksteps = fmt == 1 ? d / kPlanKStep : d / 128;  // K-steps (int4: spans) per unit
  if (pairs && !plan_split(tiles0, tiles1, imax / 64, ksteps / p.gu.ks, 2, cus, p.gu.n0, p.gu.n1))
    p.ok = false;
  // int8 down: with enough units for one K slice per workgroup, two 64-column
  // blocks per 256-thread workgroup (fewer, longer streams); with fewer (2-way
  // K slices), 32-column workgroups of 2 x 2 wavefronts instead, so that the
  // busiest CU streams fewer bytes: at one Kimi-shaped token (324 units of
  // 64 columns) 648 of them take 11.1 us, against 12.7 us for 162 two-block
  // workgroups and 15.3 us for 324 of 512 threads (2 K slices, 4 groups)
  p.dn.ks = kway(tiles * (d / 64));
  p.dn.n0 = p.dn.n1 = 1;
  p.dn.cg = 4;
  const int dsteps = fmt == 1 ? imax / kPlanKStep : imax / 128;
  p.dn.ng2 = fmt == 1 && p.dn.ks == 1 && d % 128 == 0;
  if (fmt == 1 && p.dn.ks == 2 && d % 32 == 0) p.dn.cg = 2;
  if (pairs && !p.dn.ng2 && p.dn.cg == 4 &&
      !plan_split(tiles0, tiles1, d / 64, dsteps / p.dn.ks, 2, cus, p.dn.n0, p.dn.n1))
    p.ok = false;
}

// The plan of the decode FFN launches of a quantised layer in one call, from
// the call's arguments: group 0 is the routed experts (R0 = T*k rows over E0
// experts, tiles bounded by max_tiles; or one expert over R0 rows when
// grouped0 is false), group 1 an optional second set over T identity rows
// (inter1 = 0: none).  pairs: the pairs are grouped in-kernel (small batches).
inline FfnPlan plan_ffn(int fmt, int T, int R0, int E0, bool grouped0, int d, int inter0,
                        int inter1, long long cus, bool pairs) {
  FfnPlan p{};
  const int inters[2] = {inter0, inter1};
  p.mt = ffn_tile_rows(T, d, inter1 > 0 ? 2 : 1, inters);
  if (p.mt < 1) {
    p.ok = false;
    return p;
  }
  const long long t0 = grouped0 ? max_tiles(R0, E0, p.mt) : (R0 + p.mt - 1) / p.mt;
  const long long t1 = inter1 > 0 ? (T + p.mt - 1) / p.mt : 0;
  const int imax = inter1 > inter0 ? inter1 : inter0;
  plan_launches(fmt, t0, t1, imax, d, cus, pairs, p);
  return p;
}

}  // namespace moe
