// Host check of the small-batch FFN launch plan (sparse_moe_expert_sigmoid_amd/
// csrc/plan.h), the plan the C ABI runs before it enqueues a layer and the
// launcher runs again to size its grids.
//
//  1. Every plan over a sweep of layer shapes fits the split-K join area:
//     the arrival counts (one per work unit of a launch that splits) and the
//     partial-sum slots, laid out as the kernels lay them out (group 0's
//     units first, n0 slots each, then group 1's, n1 each), stay below
//     kSplitSlots, and each split keeps at least two K-steps per wavefront.
//  2. The shapes the benchmark and the GPU tests run plan as stated in the
//     design notes (no split at the Kimi-shaped T = 8, the shared expert alone
//     8 ways at the Kimi-shaped T = 1, 2 ways at the Qwen-shaped T = 1).
//  3. split_fits refuses plans past either limit.
// Prints one line per check with its failure count; exit status 0 iff all are 0.
#include <stdio.h>

#include "../../sparse_moe_expert_sigmoid_amd/csrc/plan.h"

using namespace moe;

static long long g_fail = 0;

static bool within(const FfnPlan& p, const LaunchSplit& s, int gx, int ksteps) {
  const long long u0 = p.tiles0 * gx, u1 = p.tiles1 * gx;
  if (s.n0 == 1 && s.n1 == 1) return true;
  // last slot index written: group 0 units take u0 * n0 slots when they
  // split, then group 1 units u1 * n1
  const long long slots = (s.n0 > 1 ? u0 * s.n0 : 0) + (s.n1 > 1 ? u1 * s.n1 : 0);
  if (slots > kSplitSlots) return false;
  if (u0 + u1 > kSplitSlots) return false;  // one arrival count per unit
  const int ways = s.n0 > s.n1 ? s.n0 : s.n1;
  return ksteps / s.ks / ways >= 2;
}

int main() {
  long long plans = 0, bad_fit = 0, not_ok = 0;
  const int Es[] = {1, 2, 3, 8, 16, 32, 40, 64, 128, 256, 300, 512, 1024};
  const int ks_[] = {1, 2, 4, 6, 8, 16};
  const int widths[] = {128, 256, 384, 512, 768, 1024, 2048, 2304, 4096, 4224, 8192, 16384};
  const long long cus_list[] = {256, 80, 304};
  for (long long cus : cus_list)
    for (int fmt = 1; fmt <= 3; ++fmt)
      for (int T = 1; T <= 16; ++T)
        for (int E : Es)
          for (int k : ks_) {
            if (k > E) continue;
            for (int d : widths)
              for (int I : widths)
                for (int Is = 0; Is <= 1; ++Is) {
                  const int I1 = Is ? I : 0;
                  const FfnPlan p = plan_ffn(fmt, T, T * k, E, true, d, I, I1, cus, true);
                  ++plans;
                  if (!p.ok) { ++not_ok; continue; }
                  const int imax = I1 > I ? I1 : I;
                  const int gsteps = fmt == 1 ? d / 64 : d / 128;
                  const int dsteps = fmt == 1 ? imax / 64 : imax / 128;
                  if (!within(p, p.gu, imax / 64, gsteps)) ++bad_fit;
                  if (!p.dn.ng2 && !within(p, p.dn, d / 64, dsteps)) ++bad_fit;
                }
          }
  printf("plans within the join area: %lld failures of %lld plans (%lld refused)\n", bad_fit,
         plans, not_ok);
  g_fail += bad_fit + not_ok;

  // shapes with known plans (256 CUs)
  long long bad_known = 0;
  {
    // Kimi-shaped decode T = 8 (int8, E = 256, k = 8, d = 2304, I = 2048, shared): no split
    FfnPlan p = plan_ffn(1, 8, 64, 256, true, 2304, 2048, 2048, 256, true);
    if (!p.ok || p.gu.n0 != 1 || p.gu.n1 != 1) ++bad_known;
    // Kimi-shaped T = 1: 256 routed units beside the shared expert's 32, split 4
    // ways; down: 32-column workgroups with 2 K slices, no split across workgroups
    p = plan_ffn(1, 1, 8, 256, true, 2304, 2048, 2048, 256, true);
    if (!p.ok || p.gu.n0 != 1 || p.gu.n1 != 4 || p.tiles0 != 8 || p.tiles1 != 1) ++bad_known;
    if (p.dn.ng2 || p.dn.cg != 2 || p.dn.ks != 2 || p.dn.n0 != 1 || p.dn.n1 != 1) ++bad_known;
    // Kimi-shaped T = 8: down two column blocks per workgroup
    p = plan_ffn(1, 8, 64, 256, true, 2304, 2048, 2048, 256, true);
    if (!p.dn.ng2 || p.dn.cg != 4 || p.dn.ks != 1) ++bad_known;
    // Qwen-shaped T = 1 (int4 b32, E = 128, d = 2048, I = 768, no shared): gate/up 2 ways
    p = plan_ffn(2, 1, 8, 128, true, 2048, 768, 0, 256, true);
    if (!p.ok || p.gu.n0 != 2 || p.gu.n1 != 2) ++bad_known;
    // the split tests' int8 gate/up at T = 1 (d 2304, E 64, I 512, shared 512): 3 ways
    p = plan_ffn(1, 1, 8, 64, true, 2304, 512, 512, 256, true);
    if (!p.ok || p.gu.n0 != 3 || p.gu.n1 != 3) ++bad_known;
  }
  printf("known plans: %lld mismatches\n", bad_known);
  g_fail += bad_known;

  // refusals
  long long bad_refuse = 0;
  if (split_fits(kSplitSlots / 2 + 1, 2, 0, 1)) ++bad_refuse;          // slots past the area
  if (split_fits(100, 1, kSplitSlots, 2)) ++bad_refuse;                // counts past the area
  if (split_fits(kSplitSlots, 1, 1, 2)) ++bad_refuse;                  // counts: u0 + u1
  if (!split_fits(kSplitSlots / 2, 2, 0, 1)) ++bad_refuse;             // exactly full
  if (!split_fits(5000, 1, 0, 1)) ++bad_refuse;                        // no split, no slots
  if (split_fits(10, 0, 0, 1)) ++bad_refuse;                           // malformed
  printf("refusals: %lld mismatches\n", bad_refuse);
  g_fail += bad_refuse;

  // one-token self-selection: the x row in at most two groups of 8 per thread
  // of a 256-thread workgroup
  long long bad_sel = 0;
  if (!sel_fits(2304) || !sel_fits(2048) || !sel_fits(4096) || !sel_fits(64)) ++bad_sel;
  if (sel_fits(4104) || sel_fits(4160) || sel_fits(2308)) ++bad_sel;
  printf("self-selection sizes: %lld mismatches\n", bad_sel);
  g_fail += bad_sel;
  return g_fail == 0 ? 0 : 1;
}
