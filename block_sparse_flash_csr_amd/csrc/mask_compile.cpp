// Mask compiler: a list of slices -> the CSR of non-empty (bq x bk) tiles per
// query tile, each tagged full or partial, with the clipped slice pieces of every
// partial tile.
//
// Follows the MagiAttention v1.1.0 news ("Blackwell adaptation" list: generate the
// block-sparse structure without instantiating a dense mask, keep mask metadata
// CSR-compressed) and the UltraAttn blog, 3 (a block is Full when every position
// is valid, Causal when some are, Empty when none are) and 3.3 (Empty blocks are
// skipped).  The work is geometric: each slice visits only the tiles its
// rectangle and diagonal reach, so the cost is O(sum of tiles touched), never
// O(Sq * Sk).  A tile no single slice covers is still full when the union of its
// pieces covers it; that case is settled by counting the union row by row over
// the tile's pieces.
#include <algorithm>
#include <cstring>
#include <new>

#include "bsfa_internal.h"

namespace bsfa {
namespace {

struct Touch {
    int32_t qt, kt, slice;
    int32_t covers;  // 1 when this slice alone admits every in-range pair of the tile
};

// Largest admitted key + 1 for row i of a piece/slice with the given bounds.
inline int64_t row_hi(int64_t i, int64_t k_hi, int64_t diag)
{
    const int64_t lim = i + diag + 1;
    return lim < k_hi ? lim : k_hi;
}

// Admitted pairs of one piece inside rows [r0, r1) x keys [c0, c1), in closed form:
// row i admits [lo, min(hi, i + diag + 1)) with lo = max(k_lo, c0), hi = min(k_hi, c1).
int64_t piece_count(const Piece &p, int64_t r0, int64_t r1, int64_t c0, int64_t c1)
{
    const int64_t a = std::max<int64_t>(p.q_lo, r0), b = std::min<int64_t>(p.q_hi, r1);
    const int64_t lo = std::max<int64_t>(p.k_lo, c0), hi = std::min<int64_t>(p.k_hi, c1);
    if (a >= b || lo >= hi) return 0;
    // width(i) = clamp(i + diag + 1 - lo, 0, hi - lo): zero below i0, full from i1 on
    const int64_t i0 = lo - p.diag;            // first row with width >= 1
    const int64_t i1 = hi - p.diag - 1;        // first row with full width
    int64_t total = 0;
    const int64_t ra = std::max(a, i0), rb = std::min(b, i1);   // rows on the ramp
    if (ra < rb) {
        const int64_t w0 = ra + p.diag + 1 - lo, w1 = rb - 1 + p.diag + 1 - lo;
        total += (w0 + w1) * (rb - ra) / 2;
    }
    const int64_t fa = std::max(a, std::max(i1, i0));           // rows at full width
    if (fa < b) total += (b - fa) * (hi - lo);
    return total;
}

// Admitted pairs of the union of pieces inside rows [r0, r1) x keys [c0, c1).
int64_t union_count(const std::vector<Piece> &pc, int64_t r0, int64_t r1, int64_t c0, int64_t c1,
                    std::vector<std::pair<int64_t, int64_t>> &ivs)
{
    int64_t total = 0;
    for (int64_t i = r0; i < r1; ++i) {
        ivs.clear();
        for (const Piece &p : pc) {
            if (i < p.q_lo || i >= p.q_hi) continue;
            int64_t lo = std::max<int64_t>(p.k_lo, c0);
            int64_t hi = std::min<int64_t>(row_hi(i, p.k_hi, p.diag), c1);
            if (lo < hi) ivs.emplace_back(lo, hi);
        }
        std::sort(ivs.begin(), ivs.end());
        int64_t cur_lo = -1, cur_hi = -1;
        for (auto &iv : ivs) {
            if (iv.first > cur_hi) {
                total += cur_hi - cur_lo;
                cur_lo = iv.first;
                cur_hi = iv.second;
            } else if (iv.second > cur_hi) {
                cur_hi = iv.second;
            }
        }
        total += cur_hi - cur_lo;
    }
    return total;
}

}  // namespace

bsfa_status compile_mask(const bsfa_slice *slices, int32_t n_slices, bsfa_plan &p)
{
    const int64_t bq = p.bq, bk = p.bk, sq = p.sq, sk = p.sk;
    p.n_qt = (int32_t)((sq + bq - 1) / bq);
    p.n_kt = (int32_t)((sk + bk - 1) / bk);
    auto live = [&](const bsfa_slice &sl) { return sl.q0 < sl.q1 && sl.k0 < sl.k1; };
    // Key tiles [kt0, kt1) that slice sl reaches in query tile qt (empty when no row of
    // the tile admits a key of the slice).
    auto kt_range = [&](const bsfa_slice &sl, int64_t qt, int64_t &kt0, int64_t &kt1) {
        const int64_t r1 = std::min((qt + 1) * bq, sq);
        const int64_t b = std::min<int64_t>(sl.q1, r1);
        const int64_t diag = sl.type == BSFA_CAUSAL ? (int64_t)sl.k1 - sl.q1 : kDiagFull;
        const int64_t j_lo = sl.k0, j_hi = row_hi(b - 1, sl.k1, diag);
        kt0 = j_lo / bk;
        kt1 = j_lo < j_hi ? (j_hi + bk - 1) / bk : kt0;
    };
    try {
        // 1. the slices that reach each query tile, in slice order (CSR over query tiles;
        //    O(n_slices + sum of query tiles per slice))
        std::vector<int64_t> sptr((size_t)p.n_qt + 1, 0);
        {
            std::vector<int64_t> diff((size_t)p.n_qt + 1, 0);
            for (int32_t s = 0; s < n_slices; ++s) {
                if (!live(slices[s])) continue;
                ++diff[(size_t)(slices[s].q0 / bq)];
                --diff[(size_t)((slices[s].q1 - 1) / bq) + 1];
            }
            int64_t run = 0;
            for (int32_t qt = 0; qt < p.n_qt; ++qt) {
                run += diff[qt];
                sptr[(size_t)qt + 1] = sptr[qt] + run;
            }
        }
        std::vector<int32_t> slist((size_t)sptr[p.n_qt]);
        int64_t bound = 0;   // tiles touched, counted with multiplicity: >= nnz
        {
            std::vector<int64_t> fill(sptr.begin(), sptr.end() - 1);
            for (int32_t s = 0; s < n_slices; ++s) {
                const bsfa_slice &sl = slices[s];
                if (!live(sl)) continue;
                for (int64_t qt = sl.q0 / bq; qt * bq < sl.q1; ++qt) {
                    slist[(size_t)fill[qt]++] = s;
                    int64_t kt0, kt1;
                    kt_range(sl, qt, kt0, kt1);
                    bound += kt1 - kt0;
                }
            }
        }

        p.row_ptr.assign((size_t)p.n_qt + 1, 0);
        p.col.clear();
        p.tag.clear();
        p.piece_ptr.assign(1, 0);
        p.pieces.clear();
        const size_t cap = (size_t)std::min<int64_t>(bound, (int64_t)kMaxEntries);
        p.col.reserve(cap);
        p.tag.reserve(cap);
        p.piece_ptr.reserve(cap + 1);
        p.n_full = p.n_partial = p.pairs = 0;

        // 2. per query tile: its (tile, slice) incidences with at least one admitted pair,
        //    ordered by key tile and then slice, grouped into tiles and classified
        auto by_col = [](const Touch &x, const Touch &y) {
            if (x.kt != y.kt) return x.kt < y.kt;
            return x.slice < y.slice;
        };
        std::vector<Touch> row;
        std::vector<Piece> cand;
        std::vector<std::pair<int64_t, int64_t>> ivs;
        for (int32_t qt = 0; qt < p.n_qt; ++qt) {
            const int64_t r0 = (int64_t)qt * bq, r1 = std::min(r0 + bq, sq);
            row.clear();
            for (int64_t x = sptr[qt]; x < sptr[(size_t)qt + 1]; ++x) {
                const int32_t s = slist[(size_t)x];
                const bsfa_slice &sl = slices[s];
                const int64_t diag = sl.type == BSFA_CAUSAL ? (int64_t)sl.k1 - sl.q1 : kDiagFull;
                const int64_t a = std::max<int64_t>(sl.q0, r0), b = std::min<int64_t>(sl.q1, r1);
                const bool rows_all = a == r0 && b == r1;
                int64_t kt0, kt1;
                kt_range(sl, qt, kt0, kt1);
                for (int64_t kt = kt0; kt < kt1; ++kt) {
                    const int64_t c0 = kt * bk, c1 = std::min(c0 + bk, sk);
                    const bool covers = rows_all && sl.k0 <= c0 && sl.k1 >= c1 && (c1 - 1) <= r0 + diag;
                    row.push_back(Touch{qt, (int32_t)kt, s, covers ? 1 : 0});
                }
            }
            if (!std::is_sorted(row.begin(), row.end(), by_col)) std::sort(row.begin(), row.end(), by_col);

            size_t t = 0;
            while (t < row.size()) {
                size_t u = t;
                bool covered = false;
                while (u < row.size() && row[u].kt == row[t].kt) {
                    covered |= row[u].covers != 0;
                    ++u;
                }
                const int64_t kt = row[t].kt;
                const int64_t c0 = kt * bk, c1 = std::min(c0 + bk, sk);
                const int64_t area = (r1 - r0) * (c1 - c0);
                bool full = covered;
                int64_t count = area;
                if (!covered) {
                    // clipped pieces of the tile, in slice order
                    cand.clear();
                    for (size_t x = t; x < u; ++x) {
                        const bsfa_slice &sl = slices[row[x].slice];
                        Piece pc;
                        pc.q_lo = std::max<int32_t>(sl.q0, (int32_t)r0);
                        pc.q_hi = std::min<int32_t>(sl.q1, (int32_t)r1);
                        pc.k_lo = std::max<int32_t>(sl.k0, (int32_t)c0);
                        pc.k_hi = std::min<int32_t>(sl.k1, (int32_t)c1);
                        pc.diag = sl.type == BSFA_CAUSAL ? sl.k1 - sl.q1 : kDiagFull;
                        pc.pad0 = pc.pad1 = pc.pad2 = 0;
                        cand.push_back(pc);
                    }
                    // one piece that does not cover the tile leaves it partial; several
                    // pieces may still cover it together, which the union count settles
                    count = cand.size() == 1 ? piece_count(cand[0], r0, r1, c0, c1)
                                             : union_count(cand, r0, r1, c0, c1, ivs);
                    full = count == area;
                }
                p.col.push_back((int32_t)kt);
                if (full) {
                    p.tag.push_back(BSFA_TILE_FULL);
                    ++p.n_full;
                } else {
                    p.tag.push_back(BSFA_TILE_PARTIAL);
                    ++p.n_partial;
                    p.pieces.insert(p.pieces.end(), cand.begin(), cand.end());
                }
                p.piece_ptr.push_back((int32_t)p.pieces.size());
                p.pairs += count;
                t = u;
            }
            p.row_ptr[(size_t)qt + 1] = (int32_t)p.col.size();
            // past the kernels' addressing limits: stop here instead of compiling the rest
            if (p.col.size() >= kMaxEntries || p.pieces.size() >= kMaxPieces) return BSFA_ERR_UNSUPPORTED;
        }
    } catch (const std::bad_alloc &) {
        return BSFA_ERR_OOM;
    }
    return BSFA_OK;
}

void build_transpose(bsfa_plan &p)
{
    // counting sort of the entries by column; rows are visited in order, so every
    // column's list comes out by ascending query tile
    p.t_ptr.assign((size_t)p.n_kt + 1, 0);
    for (int32_t c : p.col) ++p.t_ptr[(size_t)c + 1];
    for (int32_t kt = 0; kt < p.n_kt; ++kt) p.t_ptr[(size_t)kt + 1] += p.t_ptr[kt];
    p.t_list.assign(2 * p.col.size(), 0);
    std::vector<int32_t> fill(p.t_ptr.begin(), p.t_ptr.end() - 1);
    for (int32_t qt = 0; qt < p.n_qt; ++qt)
        for (int32_t e = p.row_ptr[qt]; e < p.row_ptr[(size_t)qt + 1]; ++e) {
            const int32_t at = fill[p.col[e]]++;
            p.t_list[2 * (size_t)at] = qt;
            p.t_list[2 * (size_t)at + 1] = e;
        }
    build_orders(p);
}

void build_orders(bsfa_plan &p)
{
    // Launch orders of the gradient kernels.  A workgroup's work is about its number of
    // CSR entries (times the query heads of a key/value head for dK/dV), so items run
    // longest first ([MA] Dispatch Solver: greedy, heaviest first).  The hardware hands
    // workgroup i to XCD i mod 8; when the heads split evenly over the 8 XCDs, XCD x gets
    // a contiguous block of heads (their rows share its L2) and item j of its own
    // longest-first list runs as workgroup 8 j + x.
    // The cost is the same for every head, so the tiles are sorted once (counting sort
    // by cost, descending, ties by tile) and expanded: among equal costs, items go in
    // ascending id (head-major), which is the same order as sorting the items by
    // (cost descending, id ascending).
    auto order = [&](int32_t n_heads, int32_t n_t, const std::vector<int32_t> &ptr, std::vector<int32_t> &out) {
        int32_t cmax = 0;
        for (int32_t t = 0; t < n_t; ++t) cmax = std::max(cmax, ptr[(size_t)t + 1] - ptr[t]);
        std::vector<int32_t> start((size_t)cmax + 2, 0), tiles((size_t)n_t);
        for (int32_t t = 0; t < n_t; ++t) ++start[(size_t)(cmax - (ptr[(size_t)t + 1] - ptr[t])) + 1];
        for (int32_t c = 0; c <= cmax; ++c) start[(size_t)c + 1] += start[c];
        {
            std::vector<int32_t> fill(start.begin(), start.end() - 1);
            for (int32_t t = 0; t < n_t; ++t) tiles[(size_t)fill[(size_t)(cmax - (ptr[(size_t)t + 1] - ptr[t]))]++] = t;
        }
        // items of heads [h0, h1) in (cost desc, id asc) order, written at out[o0 + j * stride]
        auto expand = [&](int32_t h0, int32_t h1, size_t o0, size_t stride) {
            size_t j = 0;
            for (int32_t c = 0; c <= cmax; ++c)
                for (int32_t h = h0; h < h1; ++h)
                    for (int32_t k = start[c]; k < start[(size_t)c + 1]; ++k)
                        out[o0 + (j++) * stride] = h * n_t + tiles[(size_t)k];
        };
        out.resize((size_t)n_heads * n_t);
        if (n_heads % kNumXcd == 0) {
            const int32_t per = n_heads / kNumXcd;
            for (int32_t x = 0; x < kNumXcd; ++x) expand(x * per, (x + 1) * per, (size_t)x, kNumXcd);
        } else {
            expand(0, n_heads, 0, 1);
        }
    };
    order(p.hq, p.n_qt, p.row_ptr, p.dq_order);
    order(p.hkv, p.n_kt, p.t_ptr, p.dkv_order);
}

}  // namespace bsfa
