// Work items, their cost and the min-heap greedy (longest processing time first)
// assignment of items to the persistent workgroups of the forward kernel.
//
// Follows the MagiAttention v1.1.0 news ("system-level co-optimisation": a
// Dispatch Solver built on a min-heap greedy keeps every unit's load balanced
// under any mask so that no straggler sets the pace) and the UltraAttn blog, 4.1
// (block weights: full 1, causal about half a full block, empty 0, adjustable from
// profiling; imbalance bound ceil(avg)/avg - 1).  Here the units are workgroup
// slots on the GPU's compute units instead of devices, and the weights are
// calibrated to this forward kernel, which runs a partial tile at the cost of a
// full one plus its per-element mask.
//
// Item = (query head h, query tile qt); id = h * n_qt + qt.  Items of one key/value
// head share K/V tiles, so they are kept on one accelerator die (XCD) when that
// costs little balance: MI355X hands workgroups to its 8 XCDs round-robin, so bin
// b runs on XCD b % 8, and each XCD has its own L2.
#include <algorithm>
#include <functional>
#include <cmath>
#include <queue>
#include <utility>

#include "bsfa_internal.h"

namespace bsfa {

// LPT of items already in decreasing-cost order onto the given bins: each item to
// the least-loaded bin (ties by bin id).  Appends (bin, item) in assignment order.
// The bins sit in a binary min-heap keyed on (load, bin id); the root takes the item,
// its load grows and one sift-down restores the heap (keys are unique, so the choice
// is the same as any other exact min-heap's).
void lpt_sorted(const std::vector<int32_t> &order, const std::vector<float> &cost,
                const std::vector<int32_t> &bins, std::vector<std::pair<int32_t, int32_t>> &assign,
                std::vector<double> &load)
{
    const size_t n = bins.size();
    if (n == 0) return;
    std::vector<double> hl(n);
    std::vector<int32_t> hb(n);
    auto less = [&](size_t i, size_t j) { return hl[i] < hl[j] || (hl[i] == hl[j] && hb[i] < hb[j]); };
    auto sift_down = [&](size_t i) {
        for (;;) {
            size_t c = 2 * i + 1;
            if (c >= n) break;
            if (c + 1 < n && less(c + 1, c)) ++c;
            if (!less(c, i)) break;
            std::swap(hl[i], hl[c]);
            std::swap(hb[i], hb[c]);
            i = c;
        }
    };
    for (size_t i = 0; i < n; ++i) {
        hl[i] = load[(size_t)bins[i]];
        hb[i] = bins[i];
    }
    for (size_t i = n / 2; i-- > 0;) sift_down(i);
    for (int32_t it : order) {
        assign.push_back({hb[0], it});
        hl[0] += cost[(size_t)it];
        load[(size_t)hb[0]] = hl[0];
        sift_down(0);
    }
}

// LPT onto the given bins: heaviest item first (ties by id).
void lpt(const std::vector<int32_t> &items, const std::vector<float> &cost,
         const std::vector<int32_t> &bins, std::vector<std::pair<int32_t, int32_t>> &assign,
         std::vector<double> &load)
{
    std::vector<int32_t> order(items);
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        if (cost[a] != cost[b]) return cost[a] > cost[b];
        return a < b;
    });
    lpt_sorted(order, cost, bins, assign, load);
}

// 64-key steps of an entry of key tile col.
int64_t entry_steps(const bsfa_plan &p, int32_t col)
{
    const int64_t c0 = (int64_t)col * p.bk;
    const int64_t keys = std::min<int64_t>(c0 + p.bk, p.sk) - c0;
    return (keys + kKernelBk - 1) / kKernelBk;
}

void row_steps_host(const bsfa_plan &p, RowSteps &rs)
{
    rs.full.assign((size_t)p.n_qt, 0);
    rs.partial.assign((size_t)p.n_qt, 0);
    for (int32_t qt = 0; qt < p.n_qt; ++qt)
        for (int32_t e = p.row_ptr[qt]; e < p.row_ptr[(size_t)qt + 1]; ++e)
            (p.tag[e] == BSFA_TILE_FULL ? rs.full : rs.partial)[qt] += entry_steps(p, p.col[e]);
}

void entry_costs_host(const bsfa_plan &p, int32_t e0, int32_t e1, std::vector<double> &out)
{
    out.resize((size_t)(e1 - e0));
    for (int32_t e = e0; e < e1; ++e)
        out[(size_t)(e - e0)] = (double)entry_steps(p, p.col[e]) * bsfa_tile_cost(p.tag[e], kCostPartial);
}

void build_schedule(bsfa_plan &p, int n_bins_max, const RowSteps &rs, const EntryCosts &entry_costs)
{
    const int32_t n_items = p.hq * p.n_qt;
    // cost of a row: the per-item constant plus its 64-key steps weighted by tag (the
    // same for every head); entries' own costs are needed only to cut split rows
    std::vector<double> row_cost((size_t)p.n_qt, 0.0);
    for (int32_t qt = 0; qt < p.n_qt; ++qt)
        row_cost[qt] = kCostItem + (double)rs.full[qt] + (double)rs.partial[qt] * kCostPartial;
    p.item_cost.assign((size_t)n_items, 0.f);
    double total = 0.0;
    for (int32_t h = 0; h < p.hq; ++h)
        for (int32_t qt = 0; qt < p.n_qt; ++qt) {
            p.item_cost[(size_t)h * p.n_qt + qt] = (float)row_cost[qt];
            total += row_cost[qt];
        }
    p.total_cost = total;

    // Rows costlier than the per-bin target are split (UltraAttn 3.2: a row's key range
    // may be cut anywhere, the parts' summaries merge exactly): parts of contiguous
    // entries with about equal cost, each of at least kMinPartCost.
    const double target = std::max(total / std::max(1, n_bins_max), kMinPartCost);
    std::vector<int32_t> parts((size_t)p.n_qt, 1);
    std::vector<int32_t> cut_ptr((size_t)p.n_qt + 1, 0);   // into cuts
    std::vector<int32_t> cuts;                               // entry boundaries per row
    std::vector<double> ec;                                  // entry costs of one split row
    std::vector<std::pair<int32_t, std::vector<double>>> split_costs;   // (row, its entry costs)
    for (int32_t qt = 0; qt < p.n_qt; ++qt) {
        const int32_t e0 = p.row_ptr[qt], e1 = p.row_ptr[(size_t)qt + 1];
        int32_t np = 1;
        if (row_cost[qt] > target && e1 - e0 >= 2)
            np = (int32_t)std::min<double>({(double)kMaxParts, (double)(e1 - e0), std::ceil(row_cost[qt] / target)});
        parts[qt] = np;
        cut_ptr[(size_t)qt + 1] = cut_ptr[qt] + np;
        cuts.push_back(e0);
        if (np > 1) {
            entry_costs(e0, e1, ec);
            const double work = row_cost[qt] - kCostItem;
            double acc = 0.0;
            int32_t e = e0;
            for (int32_t k = 1; k < np; ++k) {
                // end of part k-1: first entry where the running cost reaches k/np of the
                // row, leaving at least one entry for each later part
                const double goal = work * k / np;
                while (e < e1 - (np - k) && acc + ec[(size_t)(e - e0)] * 0.5 < goal) acc += ec[(size_t)(e++ - e0)];
                if (e == cuts.back()) acc += ec[(size_t)(e++ - e0)];
                cuts.push_back(e);
            }
            split_costs.emplace_back(qt, ec);
        }
        cuts.push_back(e1);
    }
    // cuts holds, per row, np + 1 boundaries: rebase cut_ptr onto that layout
    {
        int32_t at = 0;
        for (int32_t qt = 0; qt < p.n_qt; ++qt) {
            cut_ptr[qt] = at;
            at += parts[qt] + 1;
        }
        cut_ptr[(size_t)p.n_qt] = at;
    }

    // units: id = h * units_per_head + row_base[qt] + k; partial slots likewise over the
    // split rows only
    std::vector<int32_t> row_base((size_t)p.n_qt + 1, 0), slot_base((size_t)p.n_qt + 1, 0);
    for (int32_t qt = 0; qt < p.n_qt; ++qt) {
        row_base[(size_t)qt + 1] = row_base[qt] + parts[qt];
        slot_base[(size_t)qt + 1] = slot_base[qt] + (parts[qt] > 1 ? parts[qt] : 0);
    }
    const int32_t upr = row_base[(size_t)p.n_qt], spr = slot_base[(size_t)p.n_qt];
    const int32_t n_units = p.hq * upr;
    p.n_slots = p.hq * spr;
    p.units.assign((size_t)n_units, Unit{0, 0, 0, -1});
    p.unit_cost.assign((size_t)n_units, 0.f);
    p.splits.clear();
    std::vector<float> rk_cost((size_t)upr);   // cost of (row, part) = of its unit in any head
    {
        size_t si = 0;
        for (int32_t qt = 0; qt < p.n_qt; ++qt) {
            if (parts[qt] == 1) {
                rk_cost[(size_t)row_base[qt]] = (float)row_cost[qt];
                continue;
            }
            const std::vector<double> &rc = split_costs[si++].second;
            const int32_t e0 = p.row_ptr[qt];
            for (int32_t k = 0; k < parts[qt]; ++k) {
                const int32_t eb = cuts[(size_t)cut_ptr[qt] + k], ee = cuts[(size_t)cut_ptr[qt] + k + 1];
                double c = kCostItem;
                for (int32_t e = eb; e < ee; ++e) c += rc[(size_t)(e - e0)];
                rk_cost[(size_t)row_base[qt] + k] = (float)c;
            }
        }
    }
    for (int32_t h = 0; h < p.hq; ++h)
        for (int32_t qt = 0; qt < p.n_qt; ++qt) {
            const int32_t item = h * p.n_qt + qt;
            const int32_t first = parts[qt] > 1 ? h * spr + slot_base[qt] : -1;
            if (parts[qt] > 1) p.splits.push_back(Split{item, first, parts[qt], 0});
            for (int32_t k = 0; k < parts[qt]; ++k) {
                const int32_t u = h * upr + row_base[qt] + k;
                p.units[(size_t)u] = Unit{item, cuts[(size_t)cut_ptr[qt] + k], cuts[(size_t)cut_ptr[qt] + k + 1],
                                          first < 0 ? -1 : first + k};
                p.unit_cost[(size_t)u] = rk_cost[(size_t)row_base[qt] + k];
            }
        }

    const int32_t n_bins = std::max(1, std::min(n_units, n_bins_max));
    std::vector<std::pair<int32_t, int32_t>> assign;   // (bin, unit) in assignment order
    assign.reserve((size_t)n_units);
    std::vector<double> load((size_t)n_bins, 0.0);

    bool placed = false;
    const int32_t group = p.hq / p.hkv;  // query heads per key/value head
    if (n_bins % kNumXcd == 0 && p.hkv >= kNumXcd) {
        // level 1: key/value heads onto XCDs (LPT on head totals)
        std::vector<double> head_cost((size_t)p.hkv, (double)group * (total / std::max(1, p.hq)));
        std::vector<int32_t> gorder((size_t)p.hkv);
        for (int32_t g = 0; g < p.hkv; ++g) gorder[g] = g;
        std::vector<double> xload(kNumXcd, 0.0);
        std::vector<std::vector<int32_t>> xheads(kNumXcd);
        for (int32_t g : gorder) {
            int32_t best = 0;
            for (int32_t x = 1; x < kNumXcd; ++x)
                if (xload[x] < xload[best]) best = x;
            xheads[best].push_back(g);
            xload[best] += head_cost[g];
        }
        const double xmax = *std::max_element(xload.begin(), xload.end());
        const double xavg = total / kNumXcd;
        if (xavg > 0 && xmax / xavg - 1.0 <= 0.03) {
            // level 2: within each XCD, LPT over the bins that XCD runs.  Every head has
            // the same (row, part) costs, so those are sorted once: units go in order of
            // decreasing cost, ties by row and part, then head.
            std::vector<int32_t> order((size_t)upr);
            for (int32_t i = 0; i < upr; ++i) order[i] = i;
            std::stable_sort(order.begin(), order.end(),
                             [&](int32_t x, int32_t y) { return rk_cost[x] > rk_cost[y]; });
            std::vector<int32_t> items, bins;
            for (int32_t x = 0; x < kNumXcd; ++x) {
                items.clear();
                bins.clear();
                std::vector<int32_t> heads;
                for (int32_t g : xheads[x])
                    for (int32_t h = g * group; h < (g + 1) * group; ++h) heads.push_back(h);
                std::sort(heads.begin(), heads.end());
                for (int32_t r : order)
                    for (int32_t h : heads) items.push_back(h * upr + r);
                for (int32_t b = x; b < n_bins; b += kNumXcd) bins.push_back(b);
                lpt_sorted(items, p.unit_cost, bins, assign, load);
            }
            placed = true;
        }
    }
    if (!placed) {
        std::vector<int32_t> items((size_t)n_units), bins((size_t)n_bins);
        for (int32_t i = 0; i < n_units; ++i) items[i] = i;
        for (int32_t b = 0; b < n_bins; ++b) bins[b] = b;
        lpt(items, p.unit_cost, bins, assign, load);
    }

    // per-bin lists in assignment order (counting sort by bin)
    p.bin_ptr.assign((size_t)n_bins + 1, 0);
    for (const auto &ba : assign) ++p.bin_ptr[(size_t)ba.first + 1];
    for (int32_t b = 0; b < n_bins; ++b) p.bin_ptr[(size_t)b + 1] += p.bin_ptr[b];
    p.bin_items.assign((size_t)n_units, 0);
    {
        std::vector<int32_t> fill(p.bin_ptr.begin(), p.bin_ptr.end() - 1);
        for (const auto &ba : assign) p.bin_items[(size_t)fill[ba.first]++] = ba.second;
    }
    p.makespan = 0.0;
    for (int32_t b = 0; b < n_bins; ++b) p.makespan = std::max(p.makespan, load[b]);
    // the cost of split rows includes one per-item constant per part
    p.total_cost = 0.0;
    for (float c : p.unit_cost) p.total_cost += c;
}

}  // namespace bsfa

extern "C" double bsfa_tile_cost(int32_t tag, double w_partial)
{
    if (tag == BSFA_TILE_FULL) return 1.0;
    if (tag == BSFA_TILE_PARTIAL) return w_partial;
    return 0.0;
}

extern "C" double bsfa_lpt_assign(const float *cost, int32_t n_items, int32_t n_bins,
                                  int32_t *bin_of, double *bin_load)
{
    if (n_items < 0 || n_bins < 1 || (n_items > 0 && (!cost || !bin_of))) return -1.0;
    for (int32_t i = 0; i < n_items; ++i)
        if (!(cost[i] >= 0.f) || !std::isfinite(cost[i])) return -1.0;
    try {
        std::vector<float> c(cost, cost + n_items);
        std::vector<int32_t> items((size_t)n_items), bins((size_t)n_bins);
        for (int32_t i = 0; i < n_items; ++i) items[i] = i;
        for (int32_t b = 0; b < n_bins; ++b) bins[b] = b;
        std::vector<std::pair<int32_t, int32_t>> assign;
        std::vector<double> load((size_t)n_bins, 0.0);
        bsfa::lpt(items, c, bins, assign, load);
        double mk = 0.0;
        for (const auto &ba : assign) bin_of[ba.second] = ba.first;
        for (int32_t b = 0; b < n_bins; ++b) {
            if (bin_load) bin_load[b] = load[b];
            mk = std::max(mk, load[b]);
        }
        return mk;
    } catch (...) {
        return -1.0;
    }
}

extern "C" double bsfa_imbalance_bound(double total_cost, int32_t n_bins)
{
    if (n_bins <= 0 || total_cost <= 0.0) return 0.0;
    const double avg = total_cost / n_bins;
    return std::ceil(avg) / avg - 1.0;
}
