// Expert placement for load balancing across EP ranks (host code).
//
// Moreh report ("21K output tokens/s DeepSeek inference on AMD Instinct
// MI300X GPUs with Expert Parallelism"), section on load balancing between
// GPUs: group the experts into equal-size sets whose activation totals are
// as equal as possible (a balanced number partitioning variant), renumber
// them so every set is a contiguous id range, and let the router emit the
// new ids.  The report does not give its algorithm; this one: greedy in
// decreasing load into the least-loaded group with room, then swaps between
// the most and the least loaded group while one narrows their gap, then
// ascending logical ids inside each group.  Ties always go to the lower id
// or group index, so the result is a pure function of the loads.
#include <algorithm>
#include <cstdlib>
#include <numeric>
#include <vector>

#include "launch.hpp"

namespace moeep {

bool place_experts(const int64_t* load, int E, int G, int32_t* phys_of_logical) {
    const int S = E / G;
    std::vector<int> order(E);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return load[a] > load[b]; });
    std::vector<std::vector<int>> groups(G);
    std::vector<long long> gl(G, 0);
    for (int e : order) {
        int pick = -1;
        for (int g = 0; g < G; ++g)
            if ((int)groups[g].size() < S && (pick < 0 || gl[g] < gl[pick])) pick = g;
        groups[pick].push_back(e);
        gl[pick] += load[e];
    }
    // every swap lowers the sum of squared group loads, so this ends; the cap
    // only guards against a logic error
    for (long long iter = 0; iter < 100000000LL; ++iter) {
        int gmax = 0, gmin = 0;
        for (int g = 1; g < G; ++g) {
            if (gl[g] > gl[gmax]) gmax = g;
            if (gl[g] < gl[gmin]) gmin = g;
        }
        const long long diff = gl[gmax] - gl[gmin];
        if (diff <= 0) break;
        std::vector<int> A = groups[gmax], B = groups[gmin];
        std::sort(A.begin(), A.end());
        std::sort(B.begin(), B.end());
        long long best_score = -1, best_d = 0;
        int best_a = -1, best_b = -1;
        for (int a : A)
            for (int b : B) {
                const long long d = load[a] - load[b];
                if (d <= 0 || d >= diff) continue;
                const long long score = std::llabs((diff - d) - d);   // |diff - 2d| without overflow
                if (best_score < 0 || score < best_score) {
                    best_score = score;
                    best_a = a;
                    best_b = b;
                    best_d = d;
                }
            }
        if (best_a < 0) break;
        *std::find(groups[gmax].begin(), groups[gmax].end(), best_a) = best_b;
        *std::find(groups[gmin].begin(), groups[gmin].end(), best_b) = best_a;
        gl[gmax] -= best_d;
        gl[gmin] += best_d;
    }
    for (int g = 0; g < G; ++g) {
        std::vector<int> v = groups[g];
        std::sort(v.begin(), v.end());
        for (int i = 0; i < S; ++i) phys_of_logical[v[i]] = g * S + i;
    }
    return true;
}

}  // namespace moeep
