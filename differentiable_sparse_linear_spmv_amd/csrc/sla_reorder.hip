// sla_reorder.hip -- host code: a bandwidth-reducing row order for the grouped batch
// kernels.
//
// Reverse Cuthill-McKee (Cuthill and McKee, "Reducing the bandwidth of sparse symmetric
// matrices", 1969; the reversal after George, 1971): breadth-first search from a
// pseudo-peripheral node of each connected component, visiting the neighbours of each
// node in order of increasing degree, then the whole order reversed.  On a mesh whose
// vertex ids are scattered, this brings every row's columns within about one front of
// the row, so the SpMV's gathers hit the cache lines their neighbours just brought in.
// Any order gives the same solution; only the order of the sums inside a row changes.
#include <algorithm>
#include <numeric>
#include <vector>

#include "sla_internal.h"

namespace sla {
namespace {

// Breadth-first levels from s over the neighbours of the pattern; returns the node of
// least degree in the last level and the number of levels.  mark/stamp: scratch.
int32_t last_level_node(const int32_t* rp, const int32_t* col, const std::vector<int32_t>& deg, int32_t s,
                        std::vector<int32_t>& mark, int32_t stamp, int& levels)
{
    std::vector<int32_t> cur{s}, nxt;
    mark[s] = stamp;
    levels = 0;
    int32_t best = s;
    while (!cur.empty()) {
        ++levels;
        best = cur[0];
        for (int32_t u : cur)
            if (deg[u] < deg[best] || (deg[u] == deg[best] && u < best)) best = u;
        nxt.clear();
        for (int32_t u : cur)
            for (int32_t k = rp[u]; k < rp[u + 1]; ++k) {
                const int32_t v = col[k];
                if (mark[v] != stamp) {
                    mark[v] = stamp;
                    nxt.push_back(v);
                }
            }
        cur.swap(nxt);
    }
    return best;
}

}  // namespace

void rcm_order(const int32_t* rp, const int32_t* col, int64_t n, int32_t* perm)
{
    std::vector<int32_t> deg(n);
    for (int64_t i = 0; i < n; ++i) deg[i] = rp[i + 1] - rp[i];
    std::vector<int32_t> by_deg(n);
    std::iota(by_deg.begin(), by_deg.end(), 0);
    std::stable_sort(by_deg.begin(), by_deg.end(), [&](int32_t a, int32_t b) { return deg[a] < deg[b]; });
    std::vector<char> seen(n, 0);
    std::vector<int32_t> mark(n, -1), order, nb;
    order.reserve(n);
    int32_t stamp = 0;
    size_t scan = 0;
    while (static_cast<int64_t>(order.size()) < n) {
        while (seen[by_deg[scan]]) ++scan;
        // pseudo-peripheral start: move to the far end of the component while the
        // number of levels grows (a few sweeps)
        int32_t start = by_deg[scan];
        int levels = 0, best_levels = -1;
        for (int sweep = 0; sweep < 4; ++sweep) {
            const int32_t far = last_level_node(rp, col, deg, start, mark, stamp++, levels);
            if (levels <= best_levels) break;
            best_levels = levels;
            start = far;
        }
        size_t head = order.size();
        order.push_back(start);
        seen[start] = 1;
        while (head < order.size()) {
            const int32_t u = order[head++];
            nb.clear();
            for (int32_t k = rp[u]; k < rp[u + 1]; ++k) {
                const int32_t v = col[k];
                if (!seen[v]) {
                    seen[v] = 1;
                    nb.push_back(v);
                }
            }
            std::sort(nb.begin(), nb.end(),
                      [&](int32_t a, int32_t b) { return deg[a] < deg[b] || (deg[a] == deg[b] && a < b); });
            order.insert(order.end(), nb.begin(), nb.end());
        }
    }
    for (int64_t i = 0; i < n; ++i) perm[i] = order[n - 1 - i];
}

}  // namespace sla
