// Checks st::plan_passes: every plan covers the sweeps exactly, uses passes
// of 1..maxns sweeps, has the parity of the sweep count, and (for small
// counts) costs no more than the best split found by exhaustive search.
#include <cmath>
#include <cstdio>
#include <vector>

#include "pass_plan.h"

// cheapest split of n sweeps into passes whose count has parity par, by
// exhaustive search over the last pass (memoised: n <= kMaxN)
constexpr int kMaxN = 64;
static double brute(int n, int par, int maxns, const double *cost, double (*memo)[2]) {
    if (n == 0) return par == 0 ? 0.0 : -1.0;
    if (memo[n][par] > -1.5) return memo[n][par];
    double best = -1.0;
    for (int ns = 1; ns <= maxns && ns <= n; ++ns) {
        const double rest = brute(n - ns, par ^ 1, maxns, cost, memo);
        if (rest < 0.0) continue;
        if (best < 0.0 || rest + cost[ns] < best) best = rest + cost[ns];
    }
    return memo[n][par] = best;
}

int main() {
    const double f32[] = {0.0, 1.0, 1.42, 1.525, 1.842, 2.176, 2.696};
    const double flat[] = {0.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0};
    struct Case { int maxns; const double *cost; } cases[] = {{1, f32}, {2, f32}, {4, f32}, {6, f32}, {8, flat}};
    int bad = 0, checked = 0;
    for (const Case &c : cases) {
        double memo[kMaxN + 1][2];
        for (auto &m : memo) m[0] = m[1] = -2.0;
        for (int s = 0; s <= 200; ++s) {
            const st::PassPlan p = st::plan_passes(s, c.maxns, c.cost);
            long total = (long)p.bulk * p.bulk_ns, passes = p.bulk;
            double cost = (double)p.bulk * c.cost[p.bulk_ns];
            bool ok = p.bulk_ns >= 1 && p.bulk_ns <= c.maxns;
            for (int k = 0; k < p.ntail; ++k) {
                ok = ok && p.tail[k] >= 1 && p.tail[k] <= c.maxns;
                total += p.tail[k];
                cost += c.cost[p.tail[k]];
                ++passes;
            }
            ok = ok && total == s && (passes & 1) == (s & 1);
            if (ok && s <= kMaxN) {
                const double b = brute(s, s & 1, c.maxns, c.cost, memo);
                ok = std::fabs(cost - b) < 1e-9;
            }
            ++checked;
            if (!ok) {
                ++bad;
                std::printf("FAIL maxns=%d sweeps=%d bulk=%ld tail=%d\n", c.maxns, s, (long)p.bulk, p.ntail);
            }
        }
    }
    // long runs (bulk passes first): valid splits of the right parity
    for (const Case &c : cases)
        for (int s : {257, 300, 1001, 123457}) {
            const st::PassPlan p = st::plan_passes(s, c.maxns, c.cost);
            long total = (long)p.bulk * p.bulk_ns, passes = p.bulk;
            bool ok = p.bulk > 0 && p.bulk_ns >= 1 && p.bulk_ns <= c.maxns;
            for (int k = 0; k < p.ntail; ++k) {
                ok = ok && p.tail[k] >= 1 && p.tail[k] <= c.maxns;
                total += p.tail[k];
                ++passes;
            }
            ok = ok && total == s && (passes & 1) == (s & 1);
            ++checked;
            if (!ok) {
                ++bad;
                std::printf("FAIL long maxns=%d sweeps=%d\n", c.maxns, s);
            }
        }
    const st::PassPlan ten = st::plan_passes(10, 6, f32);
    std::printf("10 sweeps, up to 6 fused:");
    for (long k = 0; k < ten.bulk; ++k) std::printf(" %d", ten.bulk_ns);
    for (int k = 0; k < ten.ntail; ++k) std::printf(" %d", ten.tail[k]);
    std::printf("\nchecked %d plans, %d bad\n", checked, bad);
    return bad != 0;
}
