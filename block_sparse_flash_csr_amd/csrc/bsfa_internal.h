// Internal declarations of libbsfa: the plan (compiled mask + schedule), the
// device-side metadata layout and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <functional>
#include <mutex>
#include <vector>

#include "../../include/bsfa.h"

namespace bsfa {

// A slice clipped to one tile.  Pair (i, j) is admitted by the piece iff
// q_lo <= i < q_hi, k_lo <= j < k_hi and j <= i + diag.  A causal slice
// (q0, q1, k0, k1) keeps diag = k1 - q1 after clipping, so its diagonal does not
// move; a full slice uses kDiagFull (no constraint for any i >= 0).
struct Piece {
    int32_t q_lo, q_hi, k_lo, k_hi, diag, pad0, pad1, pad2;
};
static_assert(sizeof(Piece) == 32, "Piece is two 16-byte words");

// Device form of one CSR entry: key-tile column, first piece, piece count
// (0 for a full tile) and the tag.
struct Entry {
    int32_t col, piece_begin, piece_count, tag;
};
static_assert(sizeof(Entry) == 16, "Entry is one 16-byte word");

// One unit of forward work: item = h * n_qt + qt over the entry range [eb, ee) of the
// query tile's CSR row.  slot < 0: the unit covers the whole row and writes O / LSE;
// otherwise it writes partial results into workspace slot `slot` (the row was split).
struct Unit {
    int32_t item, eb, ee, slot;
};
static_assert(sizeof(Unit) == 16, "Unit is one 16-byte word");

// A split row of one query head: its parts occupy slots first .. first + parts - 1.
struct Split {
    int32_t item, first, parts, pad;
};
static_assert(sizeof(Split) == 16, "Split is one 16-byte word");

constexpr int32_t kDiagFull = 1 << 30;
constexpr int kKernelBq = 128;   // query rows per work item (4 waves x 32)
constexpr int kKernelBk = 64;    // keys per inner step of the forward kernel
// The kernels address the entries (16 B each) and the pieces (32 B each) of a plan
// through 32-bit buffer offsets: a plan whose entry or piece array reaches 2^31 bytes
// is refused (BSFA_ERR_UNSUPPORTED).
constexpr size_t kMaxEntries = (size_t)1 << 27, kMaxPieces = (size_t)1 << 26;
constexpr int kNumXcd = 8;       // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kNumCu = 256;

// Scheduler cost model, in units of one full 64-key inner step of one item.
// A partial tile runs the same matrix work plus the per-element mask; the
// per-item constant covers the Q load and the O/LSE epilogue.
constexpr double kCostPartial = 1.15;
// Rows costlier than the per-bin target (total / bins) are split into parts of about
// the target, at most kMaxParts; a part is never below kMinPartCost.
constexpr double kMinPartCost = 16.0;
constexpr int32_t kMaxParts = 16;
constexpr double kCostItem = 1.0;

struct DeviceMeta {
    const int32_t *row_ptr = nullptr;
    const Entry *entries = nullptr;
    const Piece *pieces = nullptr;
    const int32_t *bin_ptr = nullptr;
    const int32_t *bin_items = nullptr;   // unit ids in execution order per bin
    const Unit *units = nullptr;
    const Split *splits = nullptr;
    const int32_t *t_ptr = nullptr;       // transposed CSR: per key tile [n_kt + 1]
    const int32_t *t_list = nullptr;      // (query tile, entry) pairs, ascending query tile
    const int32_t *dq_order = nullptr;    // gradient launch orders: workgroup -> item
    const int32_t *dkv_order = nullptr;   // (h * n_qt + qt, resp. g * n_kt + kt)
};

}  // namespace bsfa

struct bsfa_plan {
    int32_t sq = 0, sk = 0, hq = 0, hkv = 0, d = 0, bq = 0, bk = 0;
    int32_t n_qt = 0, n_kt = 0;
    // A plan built over a device-compiled CSR keeps its CSR arrays (col, tag, piece_ptr,
    // pieces, t_list) only in its device image, assembled on the device; the host holds
    // row_ptr, t_ptr, the schedule and the launch orders.
    bool device_built = false;
    int64_t dev_nnz = 0, dev_npieces = 0;
    size_t off_entries = 0, off_pieces = 0;   // byte offsets of those sections in dbuf
    size_t nnz() const { return device_built ? (size_t)dev_nnz : col.size(); }
    size_t npieces() const { return device_built ? (size_t)dev_npieces : pieces.size(); }
    // tile CSR
    std::vector<int32_t> row_ptr;
    std::vector<int32_t> col;
    std::vector<uint8_t> tag;
    std::vector<int32_t> piece_ptr;    // [nnz + 1]; empty range for full tiles
    std::vector<bsfa::Piece> pieces;
    int64_t n_full = 0, n_partial = 0, pairs = 0;
    // the same CSR by key-tile column: t_ptr [n_kt + 1], t_list [2 * nnz] = (qt, entry)
    std::vector<int32_t> t_ptr;
    std::vector<int32_t> t_list;
    // launch orders of the gradient kernels (workgroup index -> item), longest first per XCD
    std::vector<int32_t> dq_order;     // items h * n_qt + qt
    std::vector<int32_t> dkv_order;    // items g * n_kt + kt
    // schedule
    std::vector<float> item_cost;      // by item id = h * n_qt + qt
    std::vector<bsfa::Unit> units;     // by unit id; unit id == item id when no row is split
    std::vector<float> unit_cost;      // by unit id
    std::vector<bsfa::Split> splits;   // split (head, row) pairs
    int32_t n_slots = 0;               // partial-result slots of the split rows
    std::vector<int32_t> bin_ptr;      // [n_bins + 1]
    std::vector<int32_t> bin_items;    // unit ids in execution order per bin
    double makespan = 0.0, total_cost = 0.0;
    // device copy: a pooled buffer, handed back when the plan is destroyed and reused
    // only once the work enqueued on every stream that used it has run
    int device = -1;
    void *dbuf = nullptr;
    void *slot = nullptr;                   // the pool slot that owns dbuf
    hipStream_t ustream = nullptr;          // upload stream
    mutable std::mutex streams_mu;
    mutable std::vector<hipStream_t> used_streams;  // launch streams other than ustream
    bsfa::DeviceMeta dev;
};

// A tile CSR compiled on the device (see bsfa_dcsr_build).
struct bsfa_dcsr {
    int device = -1;
    int32_t n_qt = 0, n_kt = 0;
    int64_t n_touch = 0;
    void *buf = nullptr;
    hipEvent_t done = nullptr;
    const int32_t *row_ptr = nullptr, *col = nullptr, *piece_ptr = nullptr, *pieces = nullptr;
    const uint8_t *tag = nullptr;
    unsigned long long *totals_dev = nullptr;
    unsigned long long totals[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    bool have_totals = false;
};

namespace bsfa {

// Mask compiler: validated slices -> tile CSR with pieces and the pair count.
bsfa_status compile_mask(const bsfa_slice *slices, int32_t n_slices, bsfa_plan &p);
// Column view of the tile CSR (for the key/value gradients) and the launch orders of the
// gradient kernels.
void build_transpose(bsfa_plan &p);
// Launch orders of the gradient kernels from row_ptr and t_ptr.
void build_orders(bsfa_plan &p);
// Scheduler: items, costs and the per-bin lists.  A row's cost is the per-item constant
// plus its full and partial 64-key steps (RowSteps, per query tile); the entries' own
// costs (EntryCosts: entries [e0, e1) of one row) are asked for only for rows that are
// split into parts.
struct RowSteps {
    std::vector<int64_t> full, partial;
};
using EntryCosts = std::function<void(int32_t e0, int32_t e1, std::vector<double> &out)>;
int64_t entry_steps(const bsfa_plan &p, int32_t col);
void row_steps_host(const bsfa_plan &p, RowSteps &rs);
void entry_costs_host(const bsfa_plan &p, int32_t e0, int32_t e1, std::vector<double> &out);
void build_schedule(bsfa_plan &p, int n_bins_max, const RowSteps &rs, const EntryCosts &entry_costs);
// Min-heap greedy (LPT) of the given items onto the given bins; appends (bin, item)
// pairs in assignment order and updates the loads.
void lpt(const std::vector<int32_t> &items, const std::vector<float> &cost,
         const std::vector<int32_t> &bins, std::vector<std::pair<int32_t, int32_t>> &assign,
         std::vector<double> &load);

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    // element strides; validated to fit 32 bits (token strides at most 2^24)
    int32_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh, lse_sh;
    int32_t sq, sk, hq, hkv, n_qt, bk_plan;
    float c;  // scale * log2(e)
    float tau, rsum;               // rescale threshold (log2 units) and 2^tau
    DeviceMeta meta;
    float *ws;                     // partial results of split rows (caller's workspace): per
                                   // slot O [128][d] then LSE [128], fp32
    int32_t n_bins;
    int32_t n_entries, n_pieces;   // sizes of meta.entries / meta.pieces (bounds of vector loads)
    int32_t o_f32;                 // O is fp32 (else bf16)
};
hipError_t launch_attn_fwd(const FwdArgs &a, int d, hipStream_t stream);

// Size of the static device workspace of bsfa_attn_fwd_noalloc, and its address on the
// current device (looked up once per device).
constexpr size_t kStaticWorkspaceBytes = (size_t)32 << 20;
hipError_t static_workspace(float **ptr);

// Merge of split rows: partial results in the workspace -> O (bf16 or fp32) and LSE.
struct SplitMergeArgs {
    const float *ws;
    const Split *splits;
    int32_t n_splits, n_qt, sq;
    void *o;
    float *lse;
    int32_t o_st, o_sh, lse_sh;
    int32_t o_f32;                 // O is fp32 (else bf16)
};
hipError_t launch_split_merge(const SplitMergeArgs &a, int d, hipStream_t stream);

// Backward: delta_i = sum_j P_ij dP_ij per query row (a first pass over the CSR row);
// dQ per query tile over its CSR row; dK, dV per key tile over its CSR column and the
// query heads of its key/value head.
struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *lse;
    float *delta;
    float *dq, *dk, *dv;                 // fp32, contiguous [tokens, heads, d]
    int32_t q_st, q_sh, k_st, k_sh, v_st, v_sh, do_st, do_sh, lse_sh;
    int32_t sq, sk, hq, hkv, n_qt, n_kt, bk_plan;
    float scale, c;                      // c = scale * log2(e)
    DeviceMeta meta;
    int32_t n_entries, n_pieces;
    const float *o;                      // the forward's fp32 O (D_i = dO_i . O_i), or null
    int32_t o_st, o_sh;
};
hipError_t launch_attn_bwd(const BwdArgs &a, int d, hipStream_t stream);

// Device mask compiler (same CSR as compile_mask, built on the GPU).  Keys are
// (tile << sbits) | slice with tile = qt * n_kt + kt; the work arrays hold n_touch
// elements (every (tile, slice) incidence), an upper bound of nnz and of n_pieces.
struct DcsrArgs {
    int32_t sq, sk, bq, bk, n_qt, n_kt, sbits, end_bit;
    int64_t n_touch, n_pairs;
    const bsfa_slice *slices;      // [n_slices]
    const int32_t *pair_info;      // [n_pairs][4]: slice, qt, kt_lo, kt_hi
    const int64_t *pair_off;       // [n_pairs]: first key of the pair
    uint64_t *keys_in, *keys;      // [n_touch] unsorted / sorted
    int32_t *flag, *seg, *e_first, *e_n, *e_pieces, *p_off;   // [n_touch]
    uint8_t *e_full;               // [n_touch]
    void *temp;                    // sort / scan scratch
    size_t temp_bytes;
    int32_t *row_ptr;              // [n_qt + 1]
    int32_t *col;                  // [n_touch]
    uint8_t *tag;                  // [n_touch]
    int32_t *piece_ptr;            // [n_touch + 1]
    Piece *pieces;                 // [n_touch]
    unsigned long long *totals;    // [8]: nnz, n_full, n_partial, n_pieces, pairs
};
size_t dcsr_sort_temp_bytes(int64_t n, int32_t end_bit);
hipError_t launch_dcsr(const DcsrArgs &a, hipStream_t stream);

// Device part of a plan over a device-compiled CSR (plan_dev.hip): per-row full and
// partial 64-key steps and per-key-tile entry counts (launch_plan_counts), then the
// entry records and the column view (launch_plan_image: a stable radix sort of the
// entries' key tiles; end_bit covers n_kt).
struct DevPlanArgs {
    const int32_t *row_ptr, *col, *piece_ptr;   // the compiled CSR
    const uint8_t *tag;
    int32_t n_qt, n_kt, bk, sk, end_bit;
    int64_t nnz;
    int64_t *row_full, *row_partial;           // [n_qt]
    int32_t *col_count;                        // [n_kt]
    Entry *entries;                            // [nnz], in the plan's device image
    int32_t *t_list;                           // [2 nnz], in the plan's device image
    int32_t *iota, *keys_out, *sorted_e, *row_of;   // [nnz] scratch
    void *temp;
    size_t temp_bytes;
};
hipError_t launch_plan_counts(const DevPlanArgs &a, hipStream_t stream);
size_t plan_sort_temp_bytes(int64_t nnz, int32_t end_bit);
hipError_t launch_plan_image(const DevPlanArgs &a, hipStream_t stream);

struct MergeArgs {
    const void *o_parts[BSFA_MERGE_MAX_PARTS];
    const float *lse_parts[BSFA_MERGE_MAX_PARTS];
    int32_t n;
    int64_t p_st, p_sh, lse_sh;
    int32_t n_tok, n_head;
    void *o;
    float *lse;
    int64_t o_st, o_sh;
    int32_t parts_f32, o_f32;      // partials / result are fp32 (else bf16)
};
hipError_t launch_attn_merge(const MergeArgs &a, int d, hipStream_t stream);

}  // namespace bsfa
