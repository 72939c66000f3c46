// Host side of the quality-aware runtime planner (PagedWeight pages:
// legiblepapers "Summary & Methodology Analysis" and FAQ Q8; arxivlens summary
// paragraph): given the bytes to free, greedily take the quantisation actions
// with the least damage per released byte, the damage combining offline
// sensitivity, online routing mass and prompt residuals. With a negative
// target (bytes that may be spent) it takes the upgrades with the most
// benefit per added byte instead. No GPU work: the plan it writes is passed to
// pw_moe_plan_set by the caller.
//
// Readings (the pages give no formula):
//   - an action moves one block (expert, linear) by one bit;
//   - a block at bitwidth b holds R*K*b/8 bytes of planes plus R*2^b*2 bytes of
//     LUT, so b -> b-1 releases R*K/8 + R*2^(b-1)*2 bytes;
//   - damage of b -> b-1 = (sensitivity + residual) * mass * (4^-(b-1) - 4^-b):
//     the quantisation noise power of a b-bit quantiser scales as 4^-b;
//   - mass of a routed expert = its routed assignments / T (how often it is
//     used), 1 for the shared expert (every token uses it).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <queue>
#include <vector>

#include "pw.h"
#include "pw_internal.h"

namespace pw {

double block_bytes(int64_t R, int64_t K, int b) {
    return (double)R * (double)K * b / 8.0 + (double)R * (double)(1 << b) * 2.0;
}

namespace {

struct Cand {
    double ratio;   // damage per released byte (downgrade) or -benefit per added byte (upgrade)
    int block;
    int from;       // bitwidth the action starts from
    bool operator<(const Cand& o) const {   // priority_queue pops the largest: invert
        if (ratio != o.ratio) return ratio > o.ratio;
        return block > o.block;            // ties: lower block index first
    }
};

}  // namespace

// Greedy over a max-heap of per-block next actions. Returns the number of actions.
int plan_greedy(const PlanProblem& P, double bytes_to_free, uint8_t* bits, double* moved, double* damage) {
    const int n = P.n_blocks;
    auto weight = [&](int i) { return ((double)P.sens[i] + (P.resid ? (double)P.resid[i] : 0.0)) * P.mass[i]; };
    auto noise = [](int b) { return std::ldexp(1.0, -2 * b); };
    std::priority_queue<Cand> heap;
    const bool down = bytes_to_free > 0;
    auto push = [&](int i) {
        const int b = bits[i];
        const double R = P.rows[i], K = P.cols[i];
        if (down) {
            if (b <= P.min_bits[i]) return;
            const double dB = block_bytes((int64_t)R, (int64_t)K, b) - block_bytes((int64_t)R, (int64_t)K, b - 1);
            const double dmg = weight(i) * (noise(b - 1) - noise(b));
            heap.push(Cand{dmg / dB, i, b});
        } else {
            if (b >= P.max_bits[i]) return;
            const double dB = block_bytes((int64_t)R, (int64_t)K, b + 1) - block_bytes((int64_t)R, (int64_t)K, b);
            const double gain = weight(i) * (noise(b) - noise(b + 1));
            heap.push(Cand{-gain / dB, i, b});
        }
    };
    for (int i = 0; i < n; ++i) push(i);
    double done = 0.0, dmg_total = 0.0;
    int actions = 0;
    const double target = std::fabs(bytes_to_free);
    while (!heap.empty() && (down ? done < target : true)) {
        const Cand c = heap.top();
        heap.pop();
        const int i = c.block, b = bits[i];
        const double R = P.rows[i], K = P.cols[i];
        if (down) {
            done += block_bytes((int64_t)R, (int64_t)K, b) - block_bytes((int64_t)R, (int64_t)K, b - 1);
            dmg_total += weight(i) * (noise(b - 1) - noise(b));
            bits[i] = (uint8_t)(b - 1);
        } else {
            const double add = block_bytes((int64_t)R, (int64_t)K, b + 1) - block_bytes((int64_t)R, (int64_t)K, b);
            if (done + add > target) continue;   // does not fit: this block stays (its later steps cost more)
            done += add;
            dmg_total -= weight(i) * (noise(b) - noise(b + 1));
            bits[i] = (uint8_t)(b + 1);
        }
        ++actions;
        push(i);
    }
    *moved = down ? done : -done;
    *damage = dmg_total;
    return actions;
}

}  // namespace pw
