// Host-side consistency check of plan metadata before upload: plans are built with the
// C ABI, one field at a time is corrupted through the library's internal plan layout,
// and bsfa_plan_upload must refuse each corrupted plan with BSFA_ERR_PLAN before any
// device work (the kernels trust the metadata completely).  An intact plan must pass the
// check (its upload then succeeds on a GPU, or fails with BSFA_ERR_HIP where none is).
// Exit status 0 when every case behaves; one line per case on stdout.
#include <cstdio>
#include <functional>
#include <vector>

#include "../../block_sparse_flash_csr_amd/csrc/bsfa_internal.h"

namespace {

bsfa_plan *make_plan(bool split)
{
    // causal 1000 tokens, 2 query heads on 1 key/value head, plus a full slice, so that
    // the plan has full and partial tiles, pieces and (optionally) split rows
    std::vector<bsfa_slice> sl = {{0, 1000, 0, 1000, BSFA_CAUSAL}, {300, 420, 10, 900, BSFA_FULL}};
    bsfa_plan *p = nullptr;
    if (split) {
        // few long rows: 128 queries x 32 heads against 65536 keys are split into parts
        sl = {{0, 128, 0, 65536, BSFA_CAUSAL}};
        if (bsfa_plan_create(sl.data(), 1, 128, 65536, 32, 8, 128, 128, 128, &p) != BSFA_OK) return nullptr;
        return p;
    }
    if (bsfa_plan_create(sl.data(), (int32_t)sl.size(), 1000, 1000, 2, 1, 128, 128, 128, &p) != BSFA_OK)
        return nullptr;
    return p;
}

}  // namespace

int main()
{
    int bad = 0;
    struct Case {
        const char *name;
        bool split;
        std::function<void(bsfa_plan &)> corrupt;
    };
    const std::vector<Case> cases = {
        {"key tile past the last column", false, [](bsfa_plan &p) { p.col[1] = p.n_kt; }},
        {"negative key tile", false, [](bsfa_plan &p) { p.col[0] = -1; }},
        {"row offsets not monotone", false, [](bsfa_plan &p) { p.row_ptr[2] = p.row_ptr[1] - 1; }},
        {"last row offset != nnz", false, [](bsfa_plan &p) { p.row_ptr.back() += 1; }},
        {"unknown tile tag", false, [](bsfa_plan &p) { p.tag[0] = 3; }},
        {"full tile with pieces", false,
         [](bsfa_plan &p) {
             for (size_t e = 0; e < p.tag.size(); ++e)
                 if (p.tag[e] == BSFA_TILE_PARTIAL) {
                     p.tag[e] = BSFA_TILE_FULL;
                     return;
                 }
         }},
        {"piece past the query extent", false, [](bsfa_plan &p) { p.pieces[0].q_hi = p.sq + 1; }},
        {"piece offsets past the pieces", false, [](bsfa_plan &p) { p.piece_ptr.back() += 1; }},
        {"unit past its CSR row", false, [](bsfa_plan &p) { p.units[0].ee = p.row_ptr[(size_t)p.n_qt] + 1; }},
        {"unit with an unknown item", false, [](bsfa_plan &p) { p.units[0].item = p.hq * p.n_qt; }},
        {"unit scheduled twice", false, [](bsfa_plan &p) { p.bin_items[1] = p.bin_items[0]; }},
        {"bin offsets past the units", false, [](bsfa_plan &p) { p.bin_ptr.back() += 1; }},
        {"unit slot past the workspace", true, [](bsfa_plan &p) { p.units[0].slot = p.n_slots; }},
        {"split past the workspace", true, [](bsfa_plan &p) { p.splits[0].parts = p.n_slots + 1; }},
        {"column view entry out of range", false, [](bsfa_plan &p) { p.t_list[1] = (int32_t)p.col.size(); }},
        {"gradient launch order out of range", false, [](bsfa_plan &p) { p.dkv_order[0] = p.hkv * p.n_kt; }},
    };
    for (bool split : {false, true}) {
        bsfa_plan *p = make_plan(split);
        if (!p) {
            std::printf("FAIL plan creation (split=%d)\n", (int)split);
            return 1;
        }
        if (split && p->splits.empty()) {
            std::printf("FAIL the split plan has no split row\n");
            return 1;
        }
        const bsfa_status st = bsfa_plan_upload(p, nullptr);
        const bool ok = st == BSFA_OK || st == BSFA_ERR_HIP;
        std::printf("%s intact plan (split=%d): status %d\n", ok ? "ok  " : "FAIL", (int)split, (int)st);
        bad += !ok;
        bsfa_plan_destroy(p);
    }
    for (const Case &c : cases) {
        bsfa_plan *p = make_plan(c.split);
        if (!p) {
            std::printf("FAIL plan creation for %s\n", c.name);
            return 1;
        }
        c.corrupt(*p);
        const bsfa_status st = bsfa_plan_upload(p, nullptr);
        const bool ok = st == BSFA_ERR_PLAN;
        std::printf("%s %s: status %d\n", ok ? "ok  " : "FAIL", c.name, (int)st);
        bad += !ok;
        bsfa_plan_destroy(p);
    }
    return bad == 0 ? 0 : 1;
}
