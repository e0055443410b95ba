// pass_plan.h -- host-only planning of Jacobi passes for the ping-pong entry
// point: how many sweeps each pass over HBM fuses.  No HIP dependency, so a
// plain C++ compiler can test it.
#pragma once

#include <stdint.h>

namespace st {

constexpr int kMaxFusedSweeps = 8;
constexpr int kPlanExact = 256;  // sweeps planned exactly by the dynamic program

// `sweeps` Jacobi sweeps as passes of 1..maxns sweeps each.  Every pass
// moves the field to the other buffer, so the number of passes must have the
// parity of `sweeps` (the result then lands where one sweep per pass would
// leave it).  Up to kPlanExact sweeps the split is the cheapest one under
// the relative pass costs cost[1..maxns] (dynamic programming over the
// count and the parity); longer runs start with passes of the size that is
// cheapest per sweep and leave the last kPlanExact/2 or more sweeps to the
// dynamic program.  (The cheapest size per sweep alone is not always best:
// at costs 1, 1.42, 1.525, 1.842 for 1..4 sweeps, 21 sweeps are cheapest
// as seven passes of three.)
struct PassPlan {
    int bulk_ns;                        // size of the bulk passes
    int64_t bulk;                       // bulk passes, run first
    int ntail;                          // then tail[0..ntail-1]
    int tail[kPlanExact + kMaxFusedSweeps];
};

inline PassPlan plan_passes(int sweeps, int maxns, const double *cost) {
    constexpr int kTail = kPlanExact + kMaxFusedSweeps;
    PassPlan p;
    if (maxns < 1) maxns = 1;
    if (maxns > kMaxFusedSweeps) maxns = kMaxFusedSweeps;
    if (sweeps < 0) sweeps = 0;
    p.bulk_ns = 1;
    for (int ns = 2; ns <= maxns; ++ns)
        if (cost[ns] * p.bulk_ns < cost[p.bulk_ns] * ns) p.bulk_ns = ns;
    const int keep = kPlanExact / 2;  // sweeps left to the dynamic program, at least
    p.bulk = sweeps > kPlanExact ? (sweeps - keep) / p.bulk_ns : 0;
    const int r = sweeps - (int)(p.bulk * p.bulk_ns);  // <= kPlanExact < kTail
    const int want = (int)((sweeps - p.bulk) & 1);     // parity of the tail's pass count
    double best[kTail + 1][2];
    int last[kTail + 1][2];
    for (int i = 0; i <= r; ++i) {
        best[i][0] = best[i][1] = -1.0;
        last[i][0] = last[i][1] = 1;
    }
    best[0][0] = 0.0;
    for (int i = 1; i <= r; ++i)
        for (int par = 0; par < 2; ++par)
            for (int ns = 1; ns <= maxns && ns <= i; ++ns) {
                const double prev = best[i - ns][par ^ 1];
                if (prev < 0.0) continue;
                const double c = prev + cost[ns];
                if (best[i][par] < 0.0 || c < best[i][par]) {
                    best[i][par] = c;
                    last[i][par] = ns;
                }
            }
    // (r, want) is reachable: with bulk passes r >= kPlanExact/2 >= 2, and
    // two passes of one sweep or one of two fix either parity; without, r
    // passes of one sweep have parity r = sweeps.
    int rev[kTail];
    p.ntail = 0;
    for (int i = r, par = want; i > 0; par ^= 1) {
        const int ns = last[i][par];
        rev[p.ntail++] = ns;
        i -= ns;
    }
    for (int k = 0; k < p.ntail; ++k) p.tail[k] = rev[p.ntail - 1 - k];
    return p;
}

}  // namespace st
