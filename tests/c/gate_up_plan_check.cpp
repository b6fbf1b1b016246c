// Host check of the gate/up work split (gate_up_groups in expert_kernel.h) and of
// the share arithmetic k_expert uses with it: for every plan over a range of tile
// counts, K step counts and upper bounds, every (tile, K step) is covered by
// exactly one work group; for every tile, the contributors the kernel computes
// (first .. last) are exactly the work groups whose shares meet the tile, in K
// order and consecutive, at most kMaxContrib of them, so the finaliser (the last)
// holds the highest id; cut tiles' counter indices stay below kMaxSplitTiles; and
// the arithmetic stays below 2^31; the same for the remainder cut (RcPlan).  Prints
// "ok <plans checked> <remainder-cut plans checked>" or the first failure.
#include <cstdio>
#include <vector>
#include "../../expert_ffn_amd/csrc/expert_kernel.h"

using namespace moe_k;

static int fail(int tiles, int S1, int upper, const char* what) {
    std::printf("FAIL tiles=%d S1=%d upper=%d: %s\n", tiles, S1, upper, what);
    return 1;
}

int main() {
    long plans = 0;
    const int uppers[] = {2 * kCUs, kDedupSplitUpper};
    for (int upper : uppers)
        for (int S1 : {1, 2, 3, 5, 24, 64, 128, 448, 512})
            for (int tiles = 1; tiles <= 3 * kCUs + 40; ++tiles) {
                for (int ok = 0; ok < 2; ++ok) {
                    const int g1 = gate_up_groups(tiles, S1, ok != 0, upper);
                    const bool split = g1 != tiles;  // as the kernel: some tile is cut
                    if (!ok && split) return fail(tiles, S1, upper, "cut without room");
                    const long ltot = (long)tiles * S1;
                    if (split && (ltot + S1) * (long)(g1 + 1) >= (1l << 31)) return fail(tiles, S1, upper, "overflow");
                    // owner of each step, from the work groups' ranges as the kernel forms them
                    std::vector<int> owner((size_t)ltot, -1);
                    for (int wi = 0; wi < g1; ++wi) {
                        const long lbeg = split ? (long)wi * ltot / g1 : (long)wi * S1;
                        const long lend = split ? (long)(wi + 1) * ltot / g1 : (long)(wi + 1) * S1;
                        for (long L = lbeg; L < lend; ++L) {
                            if (owner[L] != -1) return fail(tiles, S1, upper, "step covered twice");
                            owner[L] = wi;
                        }
                    }
                    for (size_t L = 0; L < owner.size(); ++L)
                        if (owner[L] < 0) return fail(tiles, S1, upper, "step not covered");
                    for (int tile = 0; tile < tiles; ++tile) {
                        const int first = split ? (int)((((long)tile * S1 + 1) * g1 - 1) / ltot) : tile;
                        const int last = split ? (int)((((long)tile * S1 + S1) * g1 - 1) / ltot) : tile;
                        // the work groups meeting the tile, in K order
                        std::vector<int> meet;
                        for (int k = 0; k < S1; ++k) {
                            const int w = owner[(size_t)tile * S1 + k];
                            if (meet.empty() || meet.back() != w) meet.push_back(w);
                        }
                        if (meet.front() != first || meet.back() != last || (int)meet.size() != last - first + 1)
                            return fail(tiles, S1, upper, "contributors");
                        for (size_t i = 1; i < meet.size(); ++i)
                            if (meet[i] != meet[i - 1] + 1) return fail(tiles, S1, upper, "contributors not consecutive");
                        if ((int)meet.size() > kMaxContrib) return fail(tiles, S1, upper, "too many contributors");
                        if (meet.size() > 1 && tile >= kMaxSplitTiles)
                            return fail(tiles, S1, upper, "cut-tile counter out of range");
                    }
                    ++plans;
                }
            }
    // the remainder cut (kernels built with RC): whole tiles one work group each, the
    // remainder's K steps in equal shares; same properties, cut-tile counters indexed
    // by tile - W
    long rc_plans = 0;
    std::vector<int> sizes;
    for (int t = 2 * kCUs - 8; t <= 4 * kCUs + 40; ++t) sizes.push_back(t);
    for (int t : {896, 1792, 2688, 3584, 4480, 5376, 6272, 7168, 8192 + 77, 131072 - 5}) sizes.push_back(t);
    for (int upper : uppers)
        for (int S1 : {2, 3, 5, 44, 64, 128, 129, 448, 512})
            for (int tiles : sizes) {
                if (tiles < upper) continue;
                const int g1 = gate_up_groups_rc(tiles, S1, true, upper);
                if (g1 == tiles) {
                    if (tiles % kCUs != 0) return fail(tiles, S1, upper, "rc: remainder left whole");
                    continue;
                }
                const RcPlan rp(tiles, S1, g1);
                if ((long)rp.Lr * rp.G2 >= (1l << 31) || (long)tiles * S1 >= (1l << 31))
                    return fail(tiles, S1, upper, "rc: overflow");
                if (rp.G2 < 1 || rp.G2 > kCUs) return fail(tiles, S1, upper, "rc: remainder shares");
                const long ltot = (long)tiles * S1;
                std::vector<int> owner((size_t)ltot, -1);
                for (int wi = 0; wi < g1; ++wi)
                    for (long L = rp.lbeg(wi); L < rp.lend(wi); ++L) {
                        if (L < 0 || L >= ltot || owner[L] != -1) return fail(tiles, S1, upper, "rc: step covered twice");
                        owner[L] = wi;
                    }
                for (size_t L = 0; L < owner.size(); ++L)
                    if (owner[L] < 0) return fail(tiles, S1, upper, "rc: step not covered");
                for (int tile = 0; tile < tiles; ++tile) {
                    std::vector<int> meet;
                    for (int k = 0; k < S1; ++k) {
                        const int w = owner[(size_t)tile * S1 + k];
                        if (meet.empty() || meet.back() != w) meet.push_back(w);
                    }
                    if (meet.front() != rp.first(tile) || meet.back() != rp.last(tile) ||
                        (int)meet.size() != rp.last(tile) - rp.first(tile) + 1)
                        return fail(tiles, S1, upper, "rc: contributors");
                    for (size_t i = 1; i < meet.size(); ++i)
                        if (meet[i] != meet[i - 1] + 1) return fail(tiles, S1, upper, "rc: contributors not consecutive");
                    if ((int)meet.size() > kMaxContrib) return fail(tiles, S1, upper, "rc: too many contributors");
                    if (meet.size() > 1 && (tile < rp.W || tile - rp.W >= kMaxSplitTiles))
                        return fail(tiles, S1, upper, "rc: cut-tile counter out of range");
                }
                ++rc_plans;
            }
    std::printf("ok %ld %ld\n", plans, rc_plans);
    return 0;
}
