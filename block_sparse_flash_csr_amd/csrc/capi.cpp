// C ABI of libbsfa: argument checks, plan lifecycle and kernel dispatch.
// The declarations and their contracts are in include/bsfa.h.
#include <climits>
#include <cmath>
#include <algorithm>
#include <cstring>
#include <atomic>
#include <mutex>
#include <thread>
#include <new>
#include <vector>

#include "bsfa_internal.h"
#include "dcsr_blocks.h"

using namespace bsfa;

namespace {

constexpr int kBinsPerCu = 2;  // forward workgroups resident per CU (LDS and VGPR budget)

// Conditional-rescale threshold of the forward's online softmax, log2 units (process-wide).
std::atomic<float> g_rescale_tau{8.0f};

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
// Strides in elements: non-negative, 16-byte multiples (8 bf16 or, with f32, 4 fp32).
bool stride_ok(int64_t s, bool f32 = false) { return s >= 0 && (s & (f32 ? 3 : 7)) == 0; }

bsfa_status check_slices(const bsfa_slice *s, int32_t n, int32_t sq, int32_t sk)
{
    for (int32_t t = 0; t < n; ++t) {
        const bsfa_slice &x = s[t];
        if (x.type != BSFA_FULL && x.type != BSFA_CAUSAL) return BSFA_ERR_MASK;
        if (x.q0 < 0 || x.k0 < 0 || x.q1 < x.q0 || x.k1 < x.k0) return BSFA_ERR_MASK;
        if (x.q1 > sq || x.k1 > sk) return BSFA_ERR_MASK;
    }
    return BSFA_OK;
}

// Plans past the kernels' addressing limits (kMaxEntries, kMaxPieces) are refused.
bsfa_status check_plan_limits(size_t nnz, size_t n_pieces)
{
    return nnz >= kMaxEntries || n_pieces >= kMaxPieces ? BSFA_ERR_UNSUPPORTED : BSFA_OK;
}

// Internal consistency of a plan before its metadata reaches a kernel, which trusts it
// completely: CSR offsets monotone and in range, every entry's key tile and piece range
// in range (full tiles without pieces, partial tiles with at least one), pieces inside
// the extents, units inside their query tile's CSR row, every unit in exactly one bin,
// split slots and the column view and launch orders in range.  Host-only, linear in the
// plan's size.
bool plan_consistent(const bsfa_plan &p)
{
    const size_t nnz = p.nnz(), npc = p.npieces();
    const int64_t n_items = (int64_t)p.hq * p.n_qt;
    if (p.row_ptr.size() != (size_t)p.n_qt + 1) return false;
    if (p.row_ptr[0] != 0 || (size_t)p.row_ptr[(size_t)p.n_qt] != nnz) return false;
    for (int32_t t = 0; t < p.n_qt; ++t)
        if (p.row_ptr[(size_t)t + 1] < p.row_ptr[(size_t)t]) return false;
    if (!p.device_built) {
        // the CSR arrays (a device-built plan has them only in its device image)
        if (p.tag.size() != nnz || p.piece_ptr.size() != nnz + 1) return false;
        if (p.piece_ptr[0] != 0 || (size_t)p.piece_ptr[nnz] != npc) return false;
        for (size_t e = 0; e < nnz; ++e) {
            const int32_t np = p.piece_ptr[e + 1] - p.piece_ptr[e];
            if (np < 0 || p.col[e] < 0 || p.col[e] >= p.n_kt) return false;
            if (p.tag[e] == BSFA_TILE_FULL ? np != 0 : (p.tag[e] != BSFA_TILE_PARTIAL || np < 1)) return false;
        }
        for (const Piece &pc : p.pieces)
            if (pc.q_lo < 0 || pc.q_lo > pc.q_hi || pc.q_hi > p.sq || pc.k_lo < 0 || pc.k_lo > pc.k_hi ||
                pc.k_hi > p.sk)
                return false;
    }
    if ((int64_t)p.item_cost.size() != n_items || p.unit_cost.size() != p.units.size()) return false;
    const size_t n_units = p.units.size();
    for (const Unit &u : p.units) {
        if (u.item < 0 || u.item >= n_items || u.slot < -1 || u.slot >= p.n_slots) return false;
        const int32_t qt = u.item % p.n_qt;
        if (u.eb < p.row_ptr[(size_t)qt] || u.eb > u.ee || u.ee > p.row_ptr[(size_t)qt + 1]) return false;
    }
    if (p.bin_ptr.empty() || p.bin_ptr[0] != 0 || (size_t)p.bin_ptr.back() != p.bin_items.size() ||
        p.bin_items.size() != n_units)
        return false;
    for (size_t b = 0; b + 1 < p.bin_ptr.size(); ++b)
        if (p.bin_ptr[b + 1] < p.bin_ptr[b]) return false;
    std::vector<uint8_t> seen(n_units, 0);
    for (int32_t u : p.bin_items) {
        if (u < 0 || (size_t)u >= n_units || seen[(size_t)u]) return false;
        seen[(size_t)u] = 1;
    }
    for (const Split &sp : p.splits)
        if (sp.item < 0 || sp.item >= n_items || sp.first < 0 || sp.parts < 1 || sp.first + sp.parts > p.n_slots)
            return false;
    if (p.t_ptr.size() != (size_t)p.n_kt + 1 || p.t_ptr[0] != 0 || (size_t)p.t_ptr[(size_t)p.n_kt] != nnz)
        return false;
    for (int32_t t = 0; t < p.n_kt; ++t)
        if (p.t_ptr[(size_t)t + 1] < p.t_ptr[(size_t)t]) return false;
    if (!p.device_built) {
        if (p.t_list.size() != 2 * nnz) return false;
        for (size_t i = 0; i < nnz; ++i) {
            const int32_t qt = p.t_list[2 * i], e = p.t_list[2 * i + 1];
            if (qt < 0 || qt >= p.n_qt || e < 0 || (size_t)e >= nnz) return false;
        }
    }
    if ((int64_t)p.dq_order.size() != n_items || (int64_t)p.dkv_order.size() != (int64_t)p.hkv * p.n_kt) return false;
    for (int32_t it : p.dq_order)
        if (it < 0 || it >= n_items) return false;
    for (int32_t it : p.dkv_order)
        if (it < 0 || (int64_t)it >= (int64_t)p.hkv * p.n_kt) return false;
    return true;
}

// Column view and schedule of a compiled plan.  They read the same CSR and write
// disjoint fields, so a large plan builds them on two threads (each is a few passes over
// the entries: tens of milliseconds at millions of tiles); a small one, or a host where
// no thread can be started, builds them one after the other.
bsfa_status finish_plan(bsfa_plan &p)
{
    constexpr size_t kThreadedNnz = (size_t)1 << 20;
    std::thread tr;
    bool tr_oom = false;
    if (p.col.size() >= kThreadedNnz) {
        try {
            tr = std::thread([&p, &tr_oom] {
                try {
                    build_transpose(p);
                } catch (const std::bad_alloc &) {
                    tr_oom = true;
                }
            });
        } catch (const std::exception &) {
            // no thread: build the column view below
        }
    }
    bool oom = false;
    try {
        if (!tr.joinable()) build_transpose(p);
        RowSteps rs;
        row_steps_host(p, rs);
        build_schedule(p, kNumCu * kBinsPerCu, rs,
                       [&p](int32_t e0, int32_t e1, std::vector<double> &out) { entry_costs_host(p, e0, e1, out); });
    } catch (const std::bad_alloc &) {
        oom = true;
    }
    if (tr.joinable()) tr.join();
    return oom || tr_oom ? BSFA_ERR_OOM : BSFA_OK;
}

bsfa_status build_plan(const bsfa_slice *slices, int32_t n_slices, int32_t sq, int32_t sk,
                       int32_t hq, int32_t hkv, int32_t d, int32_t bq, int32_t bk, bsfa_plan **out)
{
    if (!out) return BSFA_ERR_ARG;
    *out = nullptr;
    if (n_slices < 0 || (n_slices > 0 && !slices)) return BSFA_ERR_ARG;
    if (sq < 0 || sk < 0 || hq <= 0 || hkv <= 0 || d <= 0 || bq <= 0 || bk <= 0) return BSFA_ERR_ARG;
    if (sq >= (1 << 30) || sk >= (1 << 30)) return BSFA_ERR_ARG;
    if (hq % hkv != 0) return BSFA_ERR_SHAPE;
    if ((int64_t)hq * ((sq + bq - 1) / bq) >= (int64_t)1 << 31) return BSFA_ERR_ARG;
    bsfa_status st = check_slices(slices, n_slices, sq, sk);
    if (st != BSFA_OK) return st;
    bsfa_plan *p = new (std::nothrow) bsfa_plan;
    if (!p) return BSFA_ERR_OOM;
    p->sq = sq;
    p->sk = sk;
    p->hq = hq;
    p->hkv = hkv;
    p->d = d;
    p->bq = bq;
    p->bk = bk;
    st = compile_mask(slices, n_slices, *p);
    if (st == BSFA_OK) st = check_plan_limits(p->col.size(), p->pieces.size());
    if (st == BSFA_OK) st = finish_plan(*p);
    if (st != BSFA_OK) {
        delete p;
        return st;
    }
    *out = p;
    return BSFA_OK;
}

// Partial results of one part: O [kKernelBq][d] then LSE [kKernelBq], fp32.
size_t slot_floats(int32_t d) { return (size_t)kKernelBq * ((size_t)d + 1); }
size_t workspace_bytes(const bsfa_plan &p) { return (size_t)p.n_slots * slot_floats(p.d) * sizeof(float); }

template <class T>
size_t place(size_t &off, size_t count)
{
    off = (off + 255) & ~size_t(255);
    const size_t at = off;
    off += count * sizeof(T);
    return at;
}

// Byte offsets of the sections of a plan's device image (256-byte aligned): row_ptr |
// entries | pieces | bin_ptr | bin_items | units | splits | t_ptr | t_list | dq_order |
// dkv_order.
struct ImageLayout {
    size_t row, ent, pc, bp, bi, un, sp, tp, tl, oq, ok, bytes;
};

ImageLayout image_layout(const bsfa_plan &p)
{
    ImageLayout L;
    size_t off = 0;
    L.row = place<int32_t>(off, p.row_ptr.size());
    L.ent = place<Entry>(off, p.nnz());
    L.pc = place<Piece>(off, p.npieces());
    L.bp = place<int32_t>(off, p.bin_ptr.size());
    L.bi = place<int32_t>(off, p.bin_items.size());
    L.un = place<Unit>(off, p.units.size());
    L.sp = place<Split>(off, p.splits.size());
    L.tp = place<int32_t>(off, p.t_ptr.size());
    L.tl = place<int32_t>(off, 2 * p.nnz());
    L.oq = place<int32_t>(off, p.dq_order.size());
    L.ok = place<int32_t>(off, p.dkv_order.size());
    L.bytes = (off + 255) & ~size_t(255);
    return L;
}

// Pinned host images of plan metadata, reused across uploads.  An image is taken by
// one caller from its acquisition until the copy recorded behind it has run: while
// the caller fills it and enqueues the copy (`filling`) nobody else may look at its
// event, which still belongs to an earlier copy; after that (`busy`) it is free again
// once the event reports the copy done.  Uploads never wait for an image, they take
// another one (or pin a new one).  Images live until process exit.
struct Staging {
    void *host = nullptr;
    size_t cap = 0;
    int device = -1;
    hipEvent_t copied = nullptr;
    bool busy = false;
    bool filling = false;
};
std::mutex g_staging_mu;
std::vector<Staging *> g_staging;

bsfa_status staging_acquire(int dev, size_t bytes, Staging **out)
{
    std::lock_guard<std::mutex> lk(g_staging_mu);
    for (Staging *st : g_staging) {
        if (st->device != dev || st->cap < bytes || st->filling) continue;
        if (st->busy && hipEventQuery(st->copied) != hipSuccess) continue;
        st->busy = true;
        st->filling = true;
        *out = st;
        return BSFA_OK;
    }
    Staging *st = new (std::nothrow) Staging;
    if (!st) return BSFA_ERR_OOM;
    size_t cap = 64 * 1024;
    while (cap < bytes) cap *= 2;
    if (hipHostMalloc(&st->host, cap, hipHostMallocDefault) != hipSuccess) {
        delete st;
        return BSFA_ERR_OOM;
    }
    if (hipEventCreateWithFlags(&st->copied, hipEventDisableTiming) != hipSuccess) {
        (void)hipHostFree(st->host);
        delete st;
        return BSFA_ERR_HIP;
    }
    st->cap = cap;
    st->device = dev;
    st->busy = true;
    st->filling = true;
    try {
        g_staging.push_back(st);
    } catch (const std::bad_alloc &) {
        (void)hipEventDestroy(st->copied);
        (void)hipHostFree(st->host);
        delete st;
        return BSFA_ERR_OOM;
    }
    *out = st;
    return BSFA_OK;
}

void staging_release_now(Staging *st)
{
    std::lock_guard<std::mutex> lk(g_staging_mu);
    st->busy = false;
    st->filling = false;
}

// The copy out of the image and its event are enqueued: from now on the event tells
// when the image is free.
void staging_in_flight(Staging *st)
{
    std::lock_guard<std::mutex> lk(g_staging_mu);
    st->filling = false;
}

// One internal copy stream per device (default priority, non-blocking): metadata
// copies run there, beside the kernels of earlier steps, and the caller's stream waits
// for them with an event.
std::mutex g_cs_mu;
std::vector<hipStream_t> g_copy_streams;

hipStream_t copy_stream(int dev)
{
    std::lock_guard<std::mutex> lk(g_cs_mu);
    if ((size_t)dev >= g_copy_streams.size()) g_copy_streams.resize((size_t)dev + 1, nullptr);
    if (!g_copy_streams[(size_t)dev]) {
        hipStream_t s = nullptr;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
        g_copy_streams[(size_t)dev] = s;
    }
    return g_copy_streams[(size_t)dev];
}

// Device buffers for plan metadata, reused across plans.  A buffer is lent to one
// plan from its upload to its destruction; destruction records one event per stream
// the plan was used on, and the buffer is lent again only once all of them have
// completed.  Nothing waits and nothing is freed: buffers live until process exit.
struct DevSlot {
    void *ptr = nullptr;
    size_t cap = 0;
    int device = -1;
    bool lent = false;
    std::vector<hipEvent_t> released;   // recorded at destruction, one per stream
    int n_released = 0;                 // how many of them the last destruction recorded
    hipEvent_t ready = nullptr;         // recorded on the copy stream behind the upload
    std::atomic<bool> ready_seen{false};  // the upload is known to have completed
};
std::mutex g_dev_mu;
std::vector<DevSlot *> g_dev;

bool slot_idle(const DevSlot *d)
{
    for (int i = 0; i < d->n_released; ++i)
        if (hipEventQuery(d->released[(size_t)i]) != hipSuccess) return false;
    return true;
}

bsfa_status dev_acquire(int dev, size_t bytes, DevSlot **out)
{
    std::lock_guard<std::mutex> lk(g_dev_mu);
    for (DevSlot *d : g_dev) {
        if (d->device != dev || d->cap < bytes || d->lent || !slot_idle(d)) continue;
        d->lent = true;
        d->n_released = 0;
        d->ready_seen = false;
        *out = d;
        return BSFA_OK;
    }
    DevSlot *d = new (std::nothrow) DevSlot;
    if (!d) return BSFA_ERR_OOM;
    size_t cap = 64 * 1024;
    while (cap < bytes) cap *= 2;
    const hipError_t e = hipMalloc(&d->ptr, cap);
    if (e != hipSuccess) {
        delete d;
        return e == hipErrorOutOfMemory ? BSFA_ERR_OOM : BSFA_ERR_HIP;
    }
    if (hipEventCreateWithFlags(&d->ready, hipEventDisableTiming) != hipSuccess) {
        (void)hipFree(d->ptr);
        delete d;
        return BSFA_ERR_HIP;
    }
    d->cap = cap;
    d->device = dev;
    d->lent = true;
    try {
        g_dev.push_back(d);
    } catch (const std::bad_alloc &) {
        (void)hipEventDestroy(d->ready);
        (void)hipFree(d->ptr);
        delete d;
        return BSFA_ERR_OOM;
    }
    *out = d;
    return BSFA_OK;
}

// Orders a launch that reads the plan's device metadata after the copy that filled
// it: nothing to do once the copy is known to have completed (then no cross-stream
// dependency is enqueued at all), else the launch stream waits for it.
bsfa_status meta_ready(const bsfa_plan *p, hipStream_t s)
{
    DevSlot *d = (DevSlot *)p->slot;
    if (d->ready_seen.load(std::memory_order_acquire)) return BSFA_OK;
    const hipError_t q = hipEventQuery(d->ready);
    if (q == hipSuccess) {
        d->ready_seen.store(true, std::memory_order_release);
        return BSFA_OK;
    }
    if (q != hipErrorNotReady) return BSFA_ERR_HIP;
    return hipStreamWaitEvent(s, d->ready, 0) == hipSuccess ? BSFA_OK : BSFA_ERR_HIP;
}

// Hands the buffer back behind the work already enqueued on the given streams.  If an
// event cannot be made or recorded, the buffer is never lent again (leaked, not reused
// early).
void dev_release(DevSlot *d, const std::vector<hipStream_t> &streams)
{
    std::lock_guard<std::mutex> lk(g_dev_mu);
    bool ok = true;
    d->n_released = 0;
    for (hipStream_t s : streams) {
        if ((size_t)d->n_released == d->released.size()) {
            hipEvent_t ev = nullptr;
            if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
                ok = false;
                break;
            }
            try {
                d->released.push_back(ev);
            } catch (const std::bad_alloc &) {
                (void)hipEventDestroy(ev);
                ok = false;
                break;
            }
        }
        if (hipEventRecord(d->released[(size_t)d->n_released], s) != hipSuccess) {
            ok = false;
            break;
        }
        ++d->n_released;
    }
    if (ok) d->lent = false;
}

// A device-compiled CSR with the extents it was compiled for (a plan built from it
// needs them).  Created and destroyed only in this file.
struct DcsrEx : bsfa_dcsr {
    int32_t sq = 0, sk = 0, bq = 0, bk = 0;
};

}  // namespace

extern "C" {

bsfa_status bsfa_plan_create(const bsfa_slice *slices, int32_t n_slices, int32_t sq, int32_t sk,
                             int32_t hq, int32_t hkv, int32_t d, int32_t bq, int32_t bk,
                             bsfa_plan **out)
{
    return build_plan(slices, n_slices, sq, sk, hq, hkv, d, bq, bk, out);
}

bsfa_status bsfa_plan_from_varlen(const int32_t *cu_seqlens, int32_t n_docs, int32_t causal,
                                  int32_t hq, int32_t hkv, int32_t d, int32_t bq, int32_t bk,
                                  bsfa_plan **out)
{
    if (!out) return BSFA_ERR_ARG;
    *out = nullptr;
    if (!cu_seqlens || n_docs < 0) return BSFA_ERR_ARG;
    if (cu_seqlens[0] != 0) return BSFA_ERR_MASK;
    std::vector<bsfa_slice> sl;
    try {
        sl.reserve((size_t)n_docs);
        for (int32_t t = 0; t < n_docs; ++t) {
            const int32_t a = cu_seqlens[t], b = cu_seqlens[t + 1];
            if (b < a) return BSFA_ERR_MASK;
            if (b > a) sl.push_back({a, b, a, b, causal ? BSFA_CAUSAL : BSFA_FULL});
        }
    } catch (const std::bad_alloc &) {
        return BSFA_ERR_OOM;
    }
    const int32_t total = cu_seqlens[n_docs];
    return build_plan(sl.data(), (int32_t)sl.size(), total, total, hq, hkv, d, bq, bk, out);
}

bsfa_status bsfa_plan_from_blocks(const uint8_t *codes, int32_t nbq, int32_t nbk,
                                  int32_t block_q, int32_t block_k, int32_t sq, int32_t sk,
                                  int32_t hq, int32_t hkv, int32_t d, int32_t bq, int32_t bk,
                                  bsfa_plan **out)
{
    if (!out) return BSFA_ERR_ARG;
    *out = nullptr;
    if (nbq < 0 || nbk < 0 || block_q <= 0 || block_k <= 0 || sq < 0 || sk < 0) return BSFA_ERR_ARG;
    if ((int64_t)nbq * nbk > 0 && !codes) return BSFA_ERR_ARG;
    std::vector<bsfa_slice> sl;
    try {
        for (int64_t i = 0; i < nbq; ++i)
            for (int64_t j = 0; j < nbk; ++j) {
                const uint8_t c = codes[i * nbk + j];
                if (c == 0) continue;
                if (c > 2) return BSFA_ERR_MASK;
                const int64_t q0 = i * block_q, k0 = j * block_k;
                const int64_t q1 = std::min<int64_t>(q0 + block_q, sq), k1 = std::min<int64_t>(k0 + block_k, sk);
                if (q0 >= sq || k0 >= sk) continue;
                sl.push_back({(int32_t)q0, (int32_t)q1, (int32_t)k0, (int32_t)k1,
                              c == 1 ? BSFA_FULL : BSFA_CAUSAL});
            }
    } catch (const std::bad_alloc &) {
        return BSFA_ERR_OOM;
    }
    return build_plan(sl.data(), (int32_t)sl.size(), sq, sk, hq, hkv, d, bq, bk, out);
}

bsfa_status bsfa_plan_upload(bsfa_plan *p, void *stream)
{
    if (!p) return BSFA_ERR_ARG;
    if (p->device_built) {
        // built on the device and resident there: nothing to copy; the stream is only
        // remembered as one to release the buffer behind
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return BSFA_ERR_HIP;
        if (cur != p->device) return BSFA_ERR_STATE;
        const hipStream_t s = (hipStream_t)stream;
        std::lock_guard<std::mutex> lk(p->streams_mu);
        if (s != p->ustream && std::find(p->used_streams.begin(), p->used_streams.end(), s) == p->used_streams.end()) {
            try {
                p->used_streams.push_back(s);
            } catch (const std::bad_alloc &) {
                return BSFA_ERR_OOM;
            }
        }
        return BSFA_OK;
    }
    if (p->dbuf) return BSFA_ERR_STATE;
    if (!plan_consistent(*p)) return BSFA_ERR_PLAN;
    hipStream_t s = (hipStream_t)stream;
    // one image: row_ptr | entries | pieces | bin_ptr | bin_items | units | splits | column
    // view | launch orders
    const size_t nnz = p->col.size();
    const ImageLayout L = image_layout(*p);
    const size_t o_row = L.row, o_ent = L.ent, o_pc = L.pc, o_bp = L.bp, o_bi = L.bi, o_un = L.un, o_sp = L.sp,
                 o_tp = L.tp, o_tl = L.tl, o_oq = L.oq, o_ok = L.ok, bytes = L.bytes;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BSFA_ERR_HIP;
    Staging *stg = nullptr;
    bsfa_status st = staging_acquire(dev, bytes, &stg);
    if (st != BSFA_OK) return st;
    uint8_t *h = (uint8_t *)stg->host;
    std::memcpy(h + o_row, p->row_ptr.data(), p->row_ptr.size() * sizeof(int32_t));
    Entry *ent = (Entry *)(h + o_ent);
    for (size_t e = 0; e < nnz; ++e)
        ent[e] = Entry{p->col[e], p->piece_ptr[e], p->piece_ptr[e + 1] - p->piece_ptr[e], p->tag[e]};
    if (!p->pieces.empty()) std::memcpy(h + o_pc, p->pieces.data(), p->pieces.size() * sizeof(Piece));
    std::memcpy(h + o_bp, p->bin_ptr.data(), p->bin_ptr.size() * sizeof(int32_t));
    if (!p->bin_items.empty())
        std::memcpy(h + o_bi, p->bin_items.data(), p->bin_items.size() * sizeof(int32_t));
    if (!p->units.empty()) std::memcpy(h + o_un, p->units.data(), p->units.size() * sizeof(Unit));
    if (!p->splits.empty()) std::memcpy(h + o_sp, p->splits.data(), p->splits.size() * sizeof(Split));
    std::memcpy(h + o_tp, p->t_ptr.data(), p->t_ptr.size() * sizeof(int32_t));
    if (!p->t_list.empty()) std::memcpy(h + o_tl, p->t_list.data(), p->t_list.size() * sizeof(int32_t));
    if (!p->dq_order.empty())
        std::memcpy(h + o_oq, p->dq_order.data(), p->dq_order.size() * sizeof(int32_t));
    if (!p->dkv_order.empty())
        std::memcpy(h + o_ok, p->dkv_order.data(), p->dkv_order.size() * sizeof(int32_t));

    DevSlot *slot = nullptr;
    st = dev_acquire(dev, bytes, &slot);
    if (st != BSFA_OK) {
        staging_release_now(stg);
        return st;
    }
    void *d = slot->ptr;
    // The copy runs on the internal copy stream (the buffer is idle, nothing earlier on
    // s touches it); the pinned image stays reserved until it has run.  Launches that
    // read the metadata are ordered after it (meta_ready): a plan built ahead of its
    // launch costs the launch stream no cross-stream dependency.
    hipStream_t cs = nullptr;
    try {
        cs = copy_stream(dev);
    } catch (const std::bad_alloc &) {
        cs = nullptr;
    }
    const bool copied = cs && hipMemcpyAsync(d, h, bytes, hipMemcpyHostToDevice, cs) == hipSuccess;
    if (!copied || hipEventRecord(stg->copied, cs) != hipSuccess || hipEventRecord(slot->ready, cs) != hipSuccess) {
        // an enqueued copy may still read the image: let it finish before the image is
        // handed out again (error path only)
        if (copied) (void)hipStreamSynchronize(cs);
        std::vector<hipStream_t> rel;
        if (cs) rel.push_back(cs);
        rel.push_back(s);
        dev_release(slot, rel);
        staging_release_now(stg);
        return BSFA_ERR_HIP;
    }
    staging_in_flight(stg);
    uint8_t *base = (uint8_t *)d;
    p->dev.row_ptr = (const int32_t *)(base + o_row);
    p->dev.entries = (const Entry *)(base + o_ent);
    p->dev.pieces = (const Piece *)(base + o_pc);
    p->dev.bin_ptr = (const int32_t *)(base + o_bp);
    p->dev.bin_items = (const int32_t *)(base + o_bi);
    p->dev.units = (const Unit *)(base + o_un);
    p->dev.splits = (const Split *)(base + o_sp);
    p->dev.t_ptr = (const int32_t *)(base + o_tp);
    p->dev.t_list = (const int32_t *)(base + o_tl);
    p->dev.dq_order = (const int32_t *)(base + o_oq);
    p->dev.dkv_order = (const int32_t *)(base + o_ok);
    p->dbuf = d;
    p->slot = slot;
    p->device = dev;
    p->ustream = s;
    return BSFA_OK;
}

void bsfa_plan_destroy(bsfa_plan *p)
{
    if (!p) return;
    if (p->slot) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        if (cur != p->device) (void)hipSetDevice(p->device);
        std::vector<hipStream_t> streams;
        try {
            streams.push_back(p->ustream);
            std::lock_guard<std::mutex> lk(p->streams_mu);
            streams.insert(streams.end(), p->used_streams.begin(), p->used_streams.end());
            dev_release((DevSlot *)p->slot, streams);
        } catch (const std::bad_alloc &) {
            // the buffer stays lent forever rather than being reused too early
        }
        if (cur != p->device) (void)hipSetDevice(cur);
    }
    delete p;
}

bsfa_status bsfa_plan_get_info(const bsfa_plan *p, bsfa_plan_info *info)
{
    if (!p || !info) return BSFA_ERR_ARG;
    info->sq = p->sq;
    info->sk = p->sk;
    info->hq = p->hq;
    info->hkv = p->hkv;
    info->d = p->d;
    info->bq = p->bq;
    info->bk = p->bk;
    info->n_qtiles = p->n_qt;
    info->n_ktiles = p->n_kt;
    info->nnz = (int64_t)p->nnz();
    info->n_full = p->n_full;
    info->n_partial = p->n_partial;
    info->n_pieces = (int64_t)p->npieces();
    info->pairs = p->pairs;
    info->n_items = (int32_t)p->item_cost.size();
    info->n_bins = (int32_t)p->bin_ptr.size() - 1;
    info->makespan = p->makespan;
    info->total_cost = p->total_cost;
    info->uploaded = p->dbuf ? 1 : 0;
    info->n_units = (int32_t)p->units.size();
    info->n_splits = (int32_t)p->splits.size();
    info->workspace_bytes = (int64_t)workspace_bytes(*p);
    return BSFA_OK;
}

// Entry records (and pieces) of a device-built plan, copied back from its device image
// once the image is complete.
static bsfa_status device_entries(const bsfa_plan &p, std::vector<Entry> &ent, std::vector<Piece> *pcs)
{
    try {
        ent.resize(p.nnz());
        if (pcs) pcs->resize(p.npieces());
    } catch (const std::bad_alloc &) {
        return BSFA_ERR_OOM;
    }
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return BSFA_ERR_HIP;
    if (cur != p.device && hipSetDevice(p.device) != hipSuccess) return BSFA_ERR_HIP;
    bool ok = hipEventSynchronize(((DevSlot *)p.slot)->ready) == hipSuccess;
    const uint8_t *base = (const uint8_t *)p.dbuf;
    if (ok && !ent.empty())
        ok = hipMemcpy(ent.data(), base + p.off_entries, ent.size() * sizeof(Entry), hipMemcpyDeviceToHost) ==
             hipSuccess;
    if (ok && pcs && !pcs->empty())
        ok = hipMemcpy(pcs->data(), base + p.off_pieces, pcs->size() * sizeof(Piece), hipMemcpyDeviceToHost) ==
             hipSuccess;
    if (cur != p.device) (void)hipSetDevice(cur);
    return ok ? BSFA_OK : BSFA_ERR_HIP;
}

bsfa_status bsfa_plan_export_csr(const bsfa_plan *p, int32_t *row_ptr, int32_t *col, uint8_t *tag,
                                 int64_t cap, int64_t *nnz)
{
    if (!p || !nnz) return BSFA_ERR_ARG;
    *nnz = (int64_t)p->nnz();
    if (cap < *nnz) return BSFA_ERR_ARG;
    if (!row_ptr || (*nnz > 0 && (!col || !tag))) return BSFA_ERR_ARG;
    std::memcpy(row_ptr, p->row_ptr.data(), p->row_ptr.size() * sizeof(int32_t));
    if (*nnz == 0) return BSFA_OK;
    if (p->device_built) {
        std::vector<Entry> ent;
        const bsfa_status st = device_entries(*p, ent, nullptr);
        if (st != BSFA_OK) return st;
        for (size_t e = 0; e < ent.size(); ++e) {
            col[e] = ent[e].col;
            tag[e] = (uint8_t)ent[e].tag;
        }
        return BSFA_OK;
    }
    std::memcpy(col, p->col.data(), p->col.size() * sizeof(int32_t));
    std::memcpy(tag, p->tag.data(), p->tag.size());
    return BSFA_OK;
}

bsfa_status bsfa_plan_export_pieces(const bsfa_plan *p, int32_t *piece_ptr, int32_t *pieces, int64_t cap)
{
    if (!p || !piece_ptr) return BSFA_ERR_ARG;
    const int64_t n = (int64_t)p->npieces();
    if (cap < n || (n > 0 && !pieces)) return BSFA_ERR_ARG;
    const Piece *src = p->pieces.data();
    std::vector<Entry> ent;
    std::vector<Piece> pcs;
    if (p->device_built) {
        const bsfa_status st = device_entries(*p, ent, &pcs);
        if (st != BSFA_OK) return st;
        for (size_t e = 0; e < ent.size(); ++e) piece_ptr[e] = ent[e].piece_begin;
        piece_ptr[ent.size()] = (int32_t)n;
        src = pcs.data();
    } else {
        std::memcpy(piece_ptr, p->piece_ptr.data(), p->piece_ptr.size() * sizeof(int32_t));
    }
    for (int64_t t = 0; t < n; ++t) {
        const Piece &pc = src[(size_t)t];
        int32_t *o = pieces + 5 * t;
        o[0] = pc.q_lo;
        o[1] = pc.q_hi;
        o[2] = pc.k_lo;
        o[3] = pc.k_hi;
        o[4] = pc.diag;
    }
    return BSFA_OK;
}

bsfa_status bsfa_plan_export_schedule(const bsfa_plan *p, int32_t *bin_ptr, int32_t *units,
                                      float *unit_cost)
{
    if (!p) return BSFA_ERR_ARG;
    if (bin_ptr) std::memcpy(bin_ptr, p->bin_ptr.data(), p->bin_ptr.size() * sizeof(int32_t));
    if (units && !p->bin_items.empty())
        std::memcpy(units, p->bin_items.data(), p->bin_items.size() * sizeof(int32_t));
    if (unit_cost && !p->unit_cost.empty())
        std::memcpy(unit_cost, p->unit_cost.data(), p->unit_cost.size() * sizeof(float));
    return BSFA_OK;
}

bsfa_status bsfa_plan_export_units(const bsfa_plan *p, int32_t *units)
{
    if (!p || !units) return BSFA_ERR_ARG;
    if (!p->units.empty()) std::memcpy(units, p->units.data(), p->units.size() * sizeof(Unit));
    return BSFA_OK;
}

bsfa_status bsfa_attn_fwd(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                          const bsfa_plan *p, float scale, bsfa_tensor *o, float *lse,
                          int64_t lse_stride_head, void *workspace, int64_t workspace_bytes_cap,
                          void *stream)
{
    return bsfa_attn_fwd_typed(q, k, v, p, scale, o, BSFA_DTYPE_BF16, lse, lse_stride_head, workspace,
                               workspace_bytes_cap, stream);
}

bsfa_status bsfa_attn_fwd_typed(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                                const bsfa_plan *p, float scale, bsfa_tensor *o, int32_t o_dtype, float *lse,
                                int64_t lse_stride_head, void *workspace, int64_t workspace_bytes_cap,
                                void *stream)
{
    if (!q || !k || !v || !p || !o) return BSFA_ERR_ARG;
    if (o_dtype != BSFA_DTYPE_BF16 && o_dtype != BSFA_DTYPE_F32) return BSFA_ERR_ARG;
    const bool o32 = o_dtype == BSFA_DTYPE_F32;
    if (workspace_bytes_cap < 0) return BSFA_ERR_ARG;
    if (p->n_slots > 0) {
        // split rows: their parts write partial results into the caller's workspace
        if (!workspace || (size_t)workspace_bytes_cap < workspace_bytes(*p)) return BSFA_ERR_ARG;
        if (!aligned16(workspace)) return BSFA_ERR_ALIGN;
    }
    if (!lse && p->sq > 0) return BSFA_ERR_ARG;   // no query: nothing is written
    if (!(scale > 0.f) || !std::isfinite(scale)) return BSFA_ERR_ARG;
    if (p->d != 64 && p->d != 128) return BSFA_ERR_UNSUPPORTED;
    if (p->bq != kKernelBq || p->bk % kKernelBk != 0) return BSFA_ERR_UNSUPPORTED;
    if (!p->dbuf) return BSFA_ERR_STATE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BSFA_ERR_HIP;
    if (dev != p->device) return BSFA_ERR_STATE;
    if (lse_stride_head < p->sq) return BSFA_ERR_ARG;
    const bool need_q = p->sq > 0, need_k = p->sk > 0;
    if ((need_q && (!q->ptr || !o->ptr)) || (need_k && (!k->ptr || !v->ptr))) return BSFA_ERR_ARG;
    // Strides: multiples of 8 elements (16-byte rows), a token row never overlapped by
    // the next token's row (stride_tok >= d), and small enough for 32-bit offsets.
    const int32_t n_tok[4] = {p->sq, p->sk, p->sk, p->sq};
    const int32_t n_head[4] = {p->hq, p->hkv, p->hkv, p->hq};
    const bsfa_tensor *ts[4] = {q, k, v, o};
    for (int t = 0; t < 4; ++t) {
        // 16-byte rows: strides in multiples of 8 bf16 (4 fp32 for an fp32 O)
        const bool f32 = t == 3 && o32;
        if (ts[t]->ptr && !aligned16(ts[t]->ptr)) return BSFA_ERR_ALIGN;
        if (!stride_ok(ts[t]->stride_tok, f32) || !stride_ok(ts[t]->stride_head, f32)) return BSFA_ERR_ALIGN;
        // the kernels size their buffer ranges as rows x stride_tok: a tensor with a token
        // needs stride_tok >= d even when it has only one
        if (n_tok[t] > 0 && ts[t]->stride_tok < p->d) return BSFA_ERR_SHAPE;
        if (n_head[t] > 1 && ts[t]->stride_head < p->d) return BSFA_ERR_SHAPE;
        if (ts[t]->stride_tok > (1 << 24) || ts[t]->stride_head > INT32_MAX) return BSFA_ERR_UNSUPPORTED;
    }
    if (lse_stride_head > INT32_MAX) return BSFA_ERR_UNSUPPORTED;
    FwdArgs a{};
    a.q = q->ptr;
    a.k = k->ptr;
    a.v = v->ptr;
    a.o = o->ptr;
    a.lse = lse;
    a.q_st = (int32_t)q->stride_tok;
    a.q_sh = (int32_t)q->stride_head;
    a.k_st = (int32_t)k->stride_tok;
    a.k_sh = (int32_t)k->stride_head;
    a.v_st = (int32_t)v->stride_tok;
    a.v_sh = (int32_t)v->stride_head;
    a.o_st = (int32_t)o->stride_tok;
    a.o_sh = (int32_t)o->stride_head;
    a.lse_sh = (int32_t)lse_stride_head;
    a.sq = p->sq;
    a.sk = p->sk;
    a.hq = p->hq;
    a.hkv = p->hkv;
    a.n_qt = p->n_qt;
    a.bk_plan = p->bk;
    a.c = scale * 1.4426950408889634f;
    a.tau = g_rescale_tau.load(std::memory_order_relaxed);
    a.rsum = std::exp2(a.tau);
    a.meta = p->dev;
    a.ws = p->n_slots > 0 ? (float *)workspace : nullptr;
    a.n_bins = (int32_t)p->bin_ptr.size() - 1;
    a.n_entries = (int32_t)p->nnz();
    a.n_pieces = (int32_t)p->npieces();
    a.o_f32 = o32 ? 1 : 0;
    if (p->sq == 0) return BSFA_OK;
    const hipStream_t s = (hipStream_t)stream;
    if (s != p->ustream) {
        // remember the stream: the plan's device buffer is released behind it
        std::lock_guard<std::mutex> lk(p->streams_mu);
        if (std::find(p->used_streams.begin(), p->used_streams.end(), s) == p->used_streams.end()) {
            try {
                p->used_streams.push_back(s);
            } catch (const std::bad_alloc &) {
                return BSFA_ERR_OOM;
            }
        }
    }
    const bsfa_status rs = meta_ready(p, s);
    if (rs != BSFA_OK) return rs;
    if (launch_attn_fwd(a, p->d, s) != hipSuccess) return BSFA_ERR_HIP;
    if (!p->splits.empty()) {
        SplitMergeArgs m;
        m.ws = a.ws;
        m.splits = p->dev.splits;
        m.n_splits = (int32_t)p->splits.size();
        m.n_qt = p->n_qt;
        m.sq = p->sq;
        m.o = o->ptr;
        m.lse = lse;
        m.o_st = a.o_st;
        m.o_sh = a.o_sh;
        m.lse_sh = a.lse_sh;
        m.o_f32 = a.o_f32;
        if (launch_split_merge(m, p->d, s) != hipSuccess) return BSFA_ERR_HIP;
    }
    return BSFA_OK;
}

static_assert(kStaticWorkspaceBytes == (size_t)BSFA_STATIC_WORKSPACE_BYTES, "one static workspace size");

bsfa_status bsfa_attn_fwd_noalloc(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                                  const bsfa_plan *p, float scale, bsfa_tensor *o, float *lse,
                                  int64_t lse_stride_head, void *stream)
{
    if (!p) return BSFA_ERR_ARG;
    if (workspace_bytes(*p) > kStaticWorkspaceBytes) return BSFA_ERR_UNSUPPORTED;
    float *ws = nullptr;
    if (static_workspace(&ws) != hipSuccess) return BSFA_ERR_HIP;
    return bsfa_attn_fwd(q, k, v, p, scale, o, lse, lse_stride_head, ws, (int64_t)kStaticWorkspaceBytes, stream);
}

namespace {

// The backward; o (the forward's fp32 O) may be null: D then comes from its own pass.
bsfa_status attn_bwd_impl(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                          const bsfa_tensor *dout, const bsfa_tensor *o, const float *lse, int64_t lse_stride_head,
                          const bsfa_plan *p, float scale, float *dq, float *dk, float *dv, float *delta,
                          void *stream)
{
    if (!q || !k || !v || !dout || !p) return BSFA_ERR_ARG;
    if (p->sq > 0 && (!lse || !delta)) return BSFA_ERR_ARG;   // no query: neither is read
    if (!(scale > 0.f) || !std::isfinite(scale)) return BSFA_ERR_ARG;
    if (p->d != 64 && p->d != 128) return BSFA_ERR_UNSUPPORTED;
    if (p->bq != kKernelBq || p->bk != 2 * kKernelBk) return BSFA_ERR_UNSUPPORTED;
    if (!p->dbuf) return BSFA_ERR_STATE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BSFA_ERR_HIP;
    if (dev != p->device) return BSFA_ERR_STATE;
    if (lse_stride_head < p->sq || lse_stride_head > INT32_MAX) return BSFA_ERR_ARG;
    if ((p->sq > 0 && !dq) || (p->sk > 0 && (!dk || !dv))) return BSFA_ERR_ARG;
    if ((int64_t)p->n_kt * p->hkv >= INT32_MAX) return BSFA_ERR_UNSUPPORTED;   // one workgroup each
    const int32_t n_tok[4] = {p->sq, p->sk, p->sk, p->sq};
    const int32_t n_head[4] = {p->hq, p->hkv, p->hkv, p->hq};
    const bsfa_tensor *ts[4] = {q, k, v, dout};
    for (int t = 0; t < 4; ++t) {
        if (n_tok[t] > 0 && !ts[t]->ptr) return BSFA_ERR_ARG;
        if (ts[t]->ptr && !aligned16(ts[t]->ptr)) return BSFA_ERR_ALIGN;
        if (!stride_ok(ts[t]->stride_tok) || !stride_ok(ts[t]->stride_head)) return BSFA_ERR_ALIGN;
        if (n_tok[t] > 0 && ts[t]->stride_tok < p->d) return BSFA_ERR_SHAPE;
        if (n_head[t] > 1 && ts[t]->stride_head < p->d) return BSFA_ERR_SHAPE;
        if (ts[t]->stride_tok > (1 << 24) || ts[t]->stride_head > INT32_MAX) return BSFA_ERR_UNSUPPORTED;
    }
    if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(delta)) return BSFA_ERR_ALIGN;
    if (o && p->sq > 0) {
        // fp32 [sq, hq, d]: 16-byte rows, a row never overlapped by the next
        if (!o->ptr) return BSFA_ERR_ARG;
        if (!aligned16(o->ptr) || !stride_ok(o->stride_tok, true) || !stride_ok(o->stride_head, true))
            return BSFA_ERR_ALIGN;
        if (o->stride_tok < p->d || (p->hq > 1 && o->stride_head < p->d)) return BSFA_ERR_SHAPE;
        if (o->stride_tok > (1 << 24) || o->stride_head > INT32_MAX) return BSFA_ERR_UNSUPPORTED;
    }
    BwdArgs a{};
    a.q = q->ptr;
    a.k = k->ptr;
    a.v = v->ptr;
    a.dout = dout->ptr;
    a.lse = lse;
    a.delta = delta;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.q_st = (int32_t)q->stride_tok;
    a.q_sh = (int32_t)q->stride_head;
    a.k_st = (int32_t)k->stride_tok;
    a.k_sh = (int32_t)k->stride_head;
    a.v_st = (int32_t)v->stride_tok;
    a.v_sh = (int32_t)v->stride_head;
    a.do_st = (int32_t)dout->stride_tok;
    a.do_sh = (int32_t)dout->stride_head;
    a.lse_sh = (int32_t)lse_stride_head;
    a.sq = p->sq;
    a.sk = p->sk;
    a.hq = p->hq;
    a.hkv = p->hkv;
    a.n_qt = p->n_qt;
    a.n_kt = p->n_kt;
    a.bk_plan = p->bk;
    a.scale = scale;
    a.c = scale * 1.4426950408889634f;
    a.meta = p->dev;
    a.n_entries = (int32_t)p->nnz();
    a.n_pieces = (int32_t)p->npieces();
    if (o && p->sq > 0) {
        a.o = (const float *)o->ptr;
        a.o_st = (int32_t)o->stride_tok;
        a.o_sh = (int32_t)o->stride_head;
    }
    const hipStream_t s = (hipStream_t)stream;
    if (s != p->ustream) {
        std::lock_guard<std::mutex> lk(p->streams_mu);
        if (std::find(p->used_streams.begin(), p->used_streams.end(), s) == p->used_streams.end()) {
            try {
                p->used_streams.push_back(s);
            } catch (const std::bad_alloc &) {
                return BSFA_ERR_OOM;
            }
        }
    }
    const bsfa_status rs = meta_ready(p, s);
    if (rs != BSFA_OK) return rs;
    if (launch_attn_bwd(a, p->d, s) != hipSuccess) return BSFA_ERR_HIP;
    return BSFA_OK;
}

}  // namespace

bsfa_status bsfa_attn_bwd(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                          const bsfa_tensor *dout, const float *lse, int64_t lse_stride_head,
                          const bsfa_plan *p, float scale, float *dq, float *dk, float *dv, float *delta,
                          void *stream)
{
    return attn_bwd_impl(q, k, v, dout, nullptr, lse, lse_stride_head, p, scale, dq, dk, dv, delta, stream);
}

bsfa_status bsfa_attn_bwd_o32(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                              const bsfa_tensor *dout, const bsfa_tensor *o, const float *lse,
                              int64_t lse_stride_head, const bsfa_plan *p, float scale, float *dq, float *dk,
                              float *dv, float *delta, void *stream)
{
    if (!o) return BSFA_ERR_ARG;
    return attn_bwd_impl(q, k, v, dout, o, lse, lse_stride_head, p, scale, dq, dk, dv, delta, stream);
}

bsfa_status bsfa_attn_merge(const void *const *o_parts, const float *const *lse_parts, int32_t n,
                            int64_t part_stride_tok, int64_t part_stride_head,
                            int64_t lse_stride_head, int32_t n_tok, int32_t n_head, int32_t d,
                            bsfa_tensor *o, float *lse, void *stream)
{
    return bsfa_attn_merge_typed(o_parts, BSFA_DTYPE_BF16, lse_parts, n, part_stride_tok, part_stride_head,
                                 lse_stride_head, n_tok, n_head, d, o, BSFA_DTYPE_BF16, lse, stream);
}

bsfa_status bsfa_attn_merge_typed(const void *const *o_parts, int32_t parts_dtype, const float *const *lse_parts,
                                  int32_t n, int64_t part_stride_tok, int64_t part_stride_head,
                                  int64_t lse_stride_head, int32_t n_tok, int32_t n_head, int32_t d,
                                  bsfa_tensor *o, int32_t o_dtype, float *lse, void *stream)
{
    if (!o_parts || !lse_parts || !o) return BSFA_ERR_ARG;
    if ((parts_dtype != BSFA_DTYPE_BF16 && parts_dtype != BSFA_DTYPE_F32) ||
        (o_dtype != BSFA_DTYPE_BF16 && o_dtype != BSFA_DTYPE_F32))
        return BSFA_ERR_ARG;
    const bool p32 = parts_dtype == BSFA_DTYPE_F32, o32 = o_dtype == BSFA_DTYPE_F32;
    if (n < 1 || n > BSFA_MERGE_MAX_PARTS || n_tok < 0 || n_head < 0 || n_head > 65535)
        return BSFA_ERR_ARG;
    if (d != 64 && d != 128) return BSFA_ERR_UNSUPPORTED;
    if (n_tok == 0 || n_head == 0) return BSFA_OK;   // nothing to merge; pointers may be NULL
    if (!lse) return BSFA_ERR_ARG;
    // one workgroup per (16 tokens, head) at d 128 with bf16 partials (8 with fp32
    // partials; twice as many at d 64) in a 1-D grid
    const int64_t rpb = p32 ? 8 : 16;
    if (((int64_t)n_tok + rpb - 1) / rpb * n_head >= INT32_MAX) return BSFA_ERR_UNSUPPORTED;
    if (lse_stride_head < n_tok) return BSFA_ERR_ARG;
    if (!stride_ok(part_stride_tok, p32) || !stride_ok(part_stride_head, p32) || !stride_ok(o->stride_tok, o32) ||
        !stride_ok(o->stride_head, o32))
        return BSFA_ERR_ALIGN;
    if (!o->ptr) return BSFA_ERR_ARG;
    if (!aligned16(o->ptr)) return BSFA_ERR_ALIGN;
    MergeArgs a{};
    for (int32_t t = 0; t < n; ++t) {
        if (!o_parts[t] || !lse_parts[t]) return BSFA_ERR_ARG;
        if (!aligned16(o_parts[t]) || ((uintptr_t)lse_parts[t] & 3u)) return BSFA_ERR_ALIGN;
        a.o_parts[t] = o_parts[t];
        a.lse_parts[t] = lse_parts[t];
    }
    a.n = n;
    a.p_st = part_stride_tok;
    a.p_sh = part_stride_head;
    a.lse_sh = lse_stride_head;
    a.n_tok = n_tok;
    a.n_head = n_head;
    a.o = o->ptr;
    a.lse = lse;
    a.o_st = o->stride_tok;
    a.o_sh = o->stride_head;
    a.parts_f32 = p32 ? 1 : 0;
    a.o_f32 = o32 ? 1 : 0;
    if (launch_attn_merge(a, d, (hipStream_t)stream) != hipSuccess) return BSFA_ERR_HIP;
    return BSFA_OK;
}

bsfa_status bsfa_dcsr_build(const bsfa_slice *slices, int32_t n_slices, int32_t sq, int32_t sk, int32_t bq,
                            int32_t bk, void *stream, bsfa_dcsr **out)
{
    if (!out) return BSFA_ERR_ARG;
    *out = nullptr;
    if (n_slices < 0 || (n_slices > 0 && !slices)) return BSFA_ERR_ARG;
    if (sq < 0 || sk < 0 || bq <= 0 || bk <= 0 || sq >= (1 << 30) || sk >= (1 << 30)) return BSFA_ERR_ARG;
    bsfa_status st = check_slices(slices, n_slices, sq, sk);
    if (st != BSFA_OK) return st;
    if (bk > 256 || n_slices >= (1 << 24)) return BSFA_ERR_UNSUPPORTED;
    const int32_t n_qt = (int32_t)(((int64_t)sq + bq - 1) / bq), n_kt = (int32_t)(((int64_t)sk + bk - 1) / bk);
    int32_t sbits = 1;
    while (sbits < 24 && (1 << sbits) < n_slices) ++sbits;
    int32_t tbits = 1;
    const uint64_t n_tiles = (uint64_t)n_qt * (uint64_t)n_kt;
    while (tbits < 63 && (1ull << tbits) < n_tiles) ++tbits;
    if (tbits + sbits > 64) return BSFA_ERR_UNSUPPORTED;
    // (slice, query tile) pairs and the key tiles each reaches (the host compiler's walk):
    // counted first, then written straight into a pinned staging image
    auto walk = [&](auto &&emit) {
        for (int32_t sx = 0; sx < n_slices; ++sx) {
            const bsfa_slice &sl = slices[sx];
            if (sl.q0 >= sl.q1 || sl.k0 >= sl.k1) continue;
            const int64_t diag = sl.type == BSFA_CAUSAL ? (int64_t)sl.k1 - sl.q1 : kDiagFull;
            for (int64_t qt = sl.q0 / bq; qt * bq < sl.q1; ++qt) {
                const int64_t r1 = std::min<int64_t>(qt * bq + bq, sq);
                const int64_t b = std::min<int64_t>(sl.q1, r1);
                const int64_t j_lo = sl.k0, j_hi = std::min<int64_t>(b - 1 + diag + 1, sl.k1);
                if (j_lo >= j_hi) continue;
                emit(sx, qt, j_lo / bk, (j_hi + bk - 1) / bk);
            }
        }
    };
    int64_t n_pairs = 0, n = 0;
    walk([&](int32_t, int64_t, int64_t lo, int64_t hi) {
        ++n_pairs;
        n += hi - lo;
    });
    if (n >= INT32_MAX) return BSFA_ERR_UNSUPPORTED;
    // staging image = the head of the device buffer: slices | pair_info | pair_off
    size_t off = 0;
    auto place = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    const size_t o_sl = place((size_t)std::max(n_slices, 1) * sizeof(bsfa_slice));
    const size_t o_pi = place((size_t)std::max<int64_t>(n_pairs, 1) * 16);
    const size_t o_po = place((size_t)std::max<int64_t>(n_pairs, 1) * 8);
    const size_t image_bytes = off;
    const size_t nn = (size_t)std::max<int64_t>(n, 1);
    const size_t o_tot = place(8 * sizeof(unsigned long long));
    const size_t o_row = place(((size_t)n_qt + 1) * 4), o_col = place(nn * 4), o_tag = place(nn);
    const size_t o_pp = place((nn + 1) * 4), o_pc = place(nn * sizeof(Piece));
    const size_t o_k0 = place(nn * 8), o_k1 = place(nn * 8);
    const size_t o_fl = place(nn * 4), o_sg = place(nn * 4), o_ef = place(nn * 4), o_en = place(nn * 4);
    const size_t o_ep = place(nn * 4), o_po2 = place(nn * 4), o_eu = place(nn);
    const size_t temp = n > 0 ? dcsr_sort_temp_bytes(n, tbits + sbits) : 0;
    const size_t o_tmp = place(std::max<size_t>(temp, 1));
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BSFA_ERR_HIP;
    Staging *stg = nullptr;
    bsfa_status sst = staging_acquire(dev, image_bytes, &stg);
    if (sst != BSFA_OK) return sst;
    {
        uint8_t *h = (uint8_t *)stg->host;
        if (n_slices > 0) std::memcpy(h + o_sl, slices, (size_t)n_slices * sizeof(bsfa_slice));
        int32_t *pi = (int32_t *)(h + o_pi);
        int64_t *po = (int64_t *)(h + o_po);
        int64_t k = 0, total = 0;
        walk([&](int32_t sx, int64_t qt, int64_t lo, int64_t hi) {
            pi[4 * k] = sx;
            pi[4 * k + 1] = (int32_t)qt;
            pi[4 * k + 2] = (int32_t)lo;
            pi[4 * k + 3] = (int32_t)hi;
            po[k++] = total;
            total += hi - lo;
        });
    }
    DcsrEx *c = new (std::nothrow) DcsrEx;
    if (!c) {
        staging_release_now(stg);
        return BSFA_ERR_OOM;
    }
    c->device = dev;
    c->sq = sq;
    c->sk = sk;
    c->bq = bq;
    c->bk = bk;
    c->n_qt = n_qt;
    c->n_kt = n_kt;
    c->n_touch = n;
    void *buf = nullptr;
    if (hipMalloc(&buf, off) != hipSuccess) {
        (void)hipGetLastError();
        staging_release_now(stg);
        delete c;
        return BSFA_ERR_OOM;
    }
    c->buf = buf;
    char *b = (char *)buf;
    if (hipEventCreateWithFlags(&c->done, hipEventDisableTiming) != hipSuccess) {
        staging_release_now(stg);
        bsfa_dcsr_destroy(c);
        return BSFA_ERR_HIP;
    }
    const hipStream_t s = (hipStream_t)stream;
    DcsrArgs a{};
    a.sq = sq;
    a.sk = sk;
    a.bq = bq;
    a.bk = bk;
    a.n_qt = n_qt;
    a.n_kt = n_kt;
    a.sbits = sbits;
    a.end_bit = tbits + sbits;
    a.n_touch = n;
    a.n_pairs = n_pairs;
    a.slices = (const bsfa_slice *)(b + o_sl);
    a.pair_info = (const int32_t *)(b + o_pi);
    a.pair_off = (const int64_t *)(b + o_po);
    a.keys_in = (uint64_t *)(b + o_k0);
    a.keys = (uint64_t *)(b + o_k1);
    a.flag = (int32_t *)(b + o_fl);
    a.seg = (int32_t *)(b + o_sg);
    a.e_first = (int32_t *)(b + o_ef);
    a.e_n = (int32_t *)(b + o_en);
    a.e_pieces = (int32_t *)(b + o_ep);
    a.p_off = (int32_t *)(b + o_po2);
    a.e_full = (uint8_t *)(b + o_eu);
    a.temp = b + o_tmp;
    a.temp_bytes = temp;
    a.row_ptr = (int32_t *)(b + o_row);
    a.col = (int32_t *)(b + o_col);
    a.tag = (uint8_t *)(b + o_tag);
    a.piece_ptr = (int32_t *)(b + o_pp);
    a.pieces = (Piece *)(b + o_pc);
    a.totals = (unsigned long long *)(b + o_tot);
    c->row_ptr = a.row_ptr;
    c->col = a.col;
    c->tag = a.tag;
    c->piece_ptr = a.piece_ptr;
    c->pieces = (const int32_t *)a.pieces;
    c->totals_dev = a.totals;
    // the pinned image stays reserved until the copy recorded behind it has run
    const bool copied = hipMemcpyAsync(b, stg->host, image_bytes, hipMemcpyHostToDevice, s) == hipSuccess;
    bool ok = copied && hipEventRecord(stg->copied, s) == hipSuccess;
    if (ok) {
        staging_in_flight(stg);
    } else {
        if (copied) (void)hipStreamSynchronize(s);   // error path: the copy may still read the image
        staging_release_now(stg);
    }
    ok = ok && launch_dcsr(a, s) == hipSuccess;
    ok = ok && hipEventRecord(c->done, s) == hipSuccess;
    if (!ok) {
        (void)hipGetLastError();
        bsfa_dcsr_destroy(c);
        return BSFA_ERR_HIP;
    }
    *out = c;
    return BSFA_OK;
}

bsfa_status bsfa_dcsr_build_blocks(const uint8_t *codes, int32_t nbq, int32_t nbk, int32_t sq, int32_t sk,
                                   int32_t bq, int32_t bk, void *stream, bsfa_dcsr **out)
{
    if (!out) return BSFA_ERR_ARG;
    *out = nullptr;
    if (nbq < 0 || nbk < 0 || sq < 0 || sk < 0 || bq <= 0 || bk <= 0 || sq >= (1 << 30) || sk >= (1 << 30))
        return BSFA_ERR_ARG;
    const int64_t n_codes = (int64_t)nbq * nbk;
    if (n_codes > 0 && !codes) return BSFA_ERR_ARG;
    const int32_t n_qt = (int32_t)(((int64_t)sq + bq - 1) / bq), n_kt = (int32_t)(((int64_t)sk + bk - 1) / bk);
    // codes must be 0, 1 or 2 everywhere (as for bsfa_plan_from_blocks); entries and pieces
    // are counted over the blocks that exist, so the buffers are sized exactly
    const int32_t rq = std::min(nbq, n_qt), rk = std::min(nbk, n_kt);
    uint8_t worst = 0;
    int64_t nnz = 0, n_pieces = 0;
    for (int32_t i = 0; i < nbq; ++i) {
        const uint8_t *r = codes + (int64_t)i * nbk;
        const int32_t jc = i < rq ? rk : 0;   // blocks of this row that exist
        int64_t nz = 0, n2 = 0;
        // byte-wide counters over chunks of 255 blocks (they cannot wrap), so that the
        // compiler keeps the loop in vector registers
        for (int32_t j0 = 0; j0 < jc; j0 += 255) {
            const int32_t j1 = std::min(j0 + 255, jc);
            uint8_t cz = 0, c2 = 0, mx = 0;
            for (int32_t j = j0; j < j1; ++j) {
                cz += r[j] != 0;
                c2 += r[j] == 2;
                mx = std::max(mx, r[j]);
            }
            nz += cz;
            n2 += c2;
            worst = std::max(worst, mx);
        }
        for (int32_t j = jc; j < nbk; ++j) worst = std::max(worst, r[j]);
        nnz += nz;
        if (std::min<int64_t>((int64_t)i * bq + bq, sq) - (int64_t)i * bq > 1) n_pieces += n2;
    }
    if (worst > 2) return BSFA_ERR_MASK;
    if (nnz >= INT32_MAX || n_pieces >= INT32_MAX) return BSFA_ERR_UNSUPPORTED;
    size_t off = 0;
    auto place = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    const size_t o_codes = place((size_t)std::max<int64_t>(n_codes, 1));
    const size_t image_bytes = off;
    const size_t rows = (size_t)n_qt + 1;
    const size_t o_rc = place(rows * 4), o_rp = place(rows * 4), o_row = place(rows * 4), o_po = place(rows * 4);
    const size_t nn = (size_t)std::max<int64_t>(nnz, 1);
    const size_t o_col = place(nn * 4), o_tag = place(nn), o_pp = place((nn + 1) * 4);
    const size_t o_pc = place((size_t)std::max<int64_t>(n_pieces, 1) * sizeof(Piece));
    const size_t o_tot = place(8 * sizeof(unsigned long long));
    const size_t temp = dcsr_blocks_scan_temp_bytes(n_qt + 1);
    const size_t o_tmp = place(std::max<size_t>(temp, 1));
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BSFA_ERR_HIP;
    Staging *stg = nullptr;
    bsfa_status sst = staging_acquire(dev, image_bytes, &stg);
    if (sst != BSFA_OK) return sst;
    if (n_codes > 0) std::memcpy((uint8_t *)stg->host + o_codes, codes, (size_t)n_codes);
    DcsrEx *c = new (std::nothrow) DcsrEx;
    if (!c) {
        staging_release_now(stg);
        return BSFA_ERR_OOM;
    }
    c->device = dev;
    c->sq = sq;
    c->sk = sk;
    c->bq = bq;
    c->bk = bk;
    c->n_qt = n_qt;
    c->n_kt = n_kt;
    c->n_touch = nnz;   // one (tile, block) incidence per entry
    void *buf = nullptr;
    if (hipMalloc(&buf, off) != hipSuccess) {
        (void)hipGetLastError();
        staging_release_now(stg);
        delete c;
        return BSFA_ERR_OOM;
    }
    c->buf = buf;
    char *b = (char *)buf;
    if (hipEventCreateWithFlags(&c->done, hipEventDisableTiming) != hipSuccess) {
        staging_release_now(stg);
        bsfa_dcsr_destroy(c);
        return BSFA_ERR_HIP;
    }
    const hipStream_t s = (hipStream_t)stream;
    DcsrBlockArgs a{};
    a.sq = sq;
    a.sk = sk;
    a.bq = bq;
    a.bk = bk;
    a.n_qt = n_qt;
    a.n_kt = n_kt;
    a.nbq = nbq;
    a.nbk = nbk;
    a.codes = (const uint8_t *)(b + o_codes);
    a.row_cnt = (int32_t *)(b + o_rc);
    a.row_pcnt = (int32_t *)(b + o_rp);
    a.row_ptr = (int32_t *)(b + o_row);
    a.row_poff = (int32_t *)(b + o_po);
    a.temp = b + o_tmp;
    a.temp_bytes = temp;
    a.col = (int32_t *)(b + o_col);
    a.tag = (uint8_t *)(b + o_tag);
    a.piece_ptr = (int32_t *)(b + o_pp);
    a.pieces = (Piece *)(b + o_pc);
    a.totals = (unsigned long long *)(b + o_tot);
    c->row_ptr = a.row_ptr;
    c->col = a.col;
    c->tag = a.tag;
    c->piece_ptr = a.piece_ptr;
    c->pieces = (const int32_t *)a.pieces;
    c->totals_dev = a.totals;
    // the pinned image stays reserved until the copy recorded behind it has run
    const bool copied = hipMemcpyAsync(b, stg->host, image_bytes, hipMemcpyHostToDevice, s) == hipSuccess;
    bool ok = copied && hipEventRecord(stg->copied, s) == hipSuccess;
    if (ok) {
        staging_in_flight(stg);
    } else {
        if (copied) (void)hipStreamSynchronize(s);   // error path: the copy may still read the image
        staging_release_now(stg);
    }
    ok = ok && launch_dcsr_blocks(a, s) == hipSuccess;
    ok = ok && hipEventRecord(c->done, s) == hipSuccess;
    if (!ok) {
        (void)hipGetLastError();
        bsfa_dcsr_destroy(c);
        return BSFA_ERR_HIP;
    }
    *out = c;
    return BSFA_OK;
}

bsfa_status bsfa_dcsr_view_get(bsfa_dcsr *c, bsfa_dcsr_view *v)
{
    if (!c || !v) return BSFA_ERR_ARG;
    if (!c->have_totals) {
        if (hipEventSynchronize(c->done) != hipSuccess) return BSFA_ERR_HIP;
        if (hipMemcpy(c->totals, c->totals_dev, sizeof(c->totals), hipMemcpyDeviceToHost) != hipSuccess)
            return BSFA_ERR_HIP;
        c->have_totals = true;
    }
    v->row_ptr = c->row_ptr;
    v->col = c->col;
    v->tag = c->tag;
    v->piece_ptr = c->piece_ptr;
    v->pieces = c->pieces;
    v->n_qtiles = c->n_qt;
    v->n_ktiles = c->n_kt;
    v->nnz = (int64_t)c->totals[0];
    v->n_full = (int64_t)c->totals[1];
    v->n_partial = (int64_t)c->totals[2];
    v->n_pieces = (int64_t)c->totals[3];
    v->pairs = (int64_t)c->totals[4];
    v->touches = c->n_touch;
    return BSFA_OK;
}

bsfa_status bsfa_dcsr_export(bsfa_dcsr *c, int32_t *row_ptr, int32_t *col, uint8_t *tag, int32_t *piece_ptr,
                             int32_t *pieces, int64_t cap_nnz, int64_t cap_pieces)
{
    bsfa_dcsr_view v;
    const bsfa_status st = bsfa_dcsr_view_get(c, &v);
    if (st != BSFA_OK) return st;
    if (!row_ptr || !piece_ptr || cap_nnz < v.nnz || cap_pieces < v.n_pieces) return BSFA_ERR_ARG;
    if (v.nnz > 0 && (!col || !tag)) return BSFA_ERR_ARG;
    if (v.n_pieces > 0 && !pieces) return BSFA_ERR_ARG;
    bool ok = hipMemcpy(row_ptr, v.row_ptr, ((size_t)v.n_qtiles + 1) * 4, hipMemcpyDeviceToHost) == hipSuccess;
    ok = ok && hipMemcpy(piece_ptr, v.piece_ptr, ((size_t)v.nnz + 1) * 4, hipMemcpyDeviceToHost) == hipSuccess;
    if (v.nnz > 0) {
        ok = ok && hipMemcpy(col, v.col, (size_t)v.nnz * 4, hipMemcpyDeviceToHost) == hipSuccess;
        ok = ok && hipMemcpy(tag, v.tag, (size_t)v.nnz, hipMemcpyDeviceToHost) == hipSuccess;
    }
    if (v.n_pieces > 0) {
        std::vector<int32_t> raw;
        try {
            raw.resize((size_t)v.n_pieces * 8);
        } catch (const std::bad_alloc &) {
            return BSFA_ERR_OOM;
        }
        ok = ok && hipMemcpy(raw.data(), v.pieces, raw.size() * 4, hipMemcpyDeviceToHost) == hipSuccess;
        for (int64_t t = 0; ok && t < v.n_pieces; ++t)
            for (int f = 0; f < 5; ++f) pieces[5 * t + f] = raw[(size_t)(8 * t + f)];
    }
    return ok ? BSFA_OK : BSFA_ERR_HIP;
}

bsfa_status bsfa_plan_from_dcsr(bsfa_dcsr *csr, int32_t hq, int32_t hkv, int32_t d, bsfa_plan **out)
{
    if (!out) return BSFA_ERR_ARG;
    *out = nullptr;
    if (!csr || hq <= 0 || hkv <= 0 || d <= 0) return BSFA_ERR_ARG;
    if (hq % hkv != 0) return BSFA_ERR_SHAPE;
    const DcsrEx *x = static_cast<const DcsrEx *>(csr);
    if ((int64_t)hq * x->n_qt >= (int64_t)1 << 31) return BSFA_ERR_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BSFA_ERR_HIP;
    if (dev != x->device) return BSFA_ERR_STATE;
    bsfa_dcsr_view v;
    bsfa_status st = bsfa_dcsr_view_get(csr, &v);   // waits for the compile
    if (st != BSFA_OK) return st;
    st = check_plan_limits((size_t)v.nnz, (size_t)v.n_pieces);
    if (st != BSFA_OK) return st;
    const hipStream_t cs = copy_stream(dev);
    if (!cs) return BSFA_ERR_HIP;
    bsfa_plan *p = new (std::nothrow) bsfa_plan;
    if (!p) return BSFA_ERR_OOM;
    p->sq = x->sq;
    p->sk = x->sk;
    p->hq = hq;
    p->hkv = hkv;
    p->d = d;
    p->bq = x->bq;
    p->bk = x->bk;
    p->n_qt = x->n_qt;
    p->n_kt = x->n_kt;
    p->device_built = true;
    p->dev_nnz = v.nnz;
    p->dev_npieces = v.n_pieces;
    p->n_full = v.n_full;
    p->n_partial = v.n_partial;
    p->pairs = v.pairs;
    const int64_t nnz = v.nnz;
    int end_bit = 1;
    while ((1ll << end_bit) < (int64_t)std::max(p->n_kt, 1)) ++end_bit;

    // device scratch (stream-ordered, freed behind the image's kernels): per-row steps,
    // per-key-tile counts, then the sort's arrays
    const size_t sort_temp = nnz > 0 ? plan_sort_temp_bytes(nnz, end_bit) : 0;
    size_t off = 0;
    const size_t o_full = place<int64_t>(off, (size_t)p->n_qt), o_part = place<int64_t>(off, (size_t)p->n_qt);
    const size_t o_cnt = place<int32_t>(off, (size_t)p->n_kt);
    const size_t o_iota = place<int32_t>(off, (size_t)nnz), o_keys = place<int32_t>(off, (size_t)nnz);
    const size_t o_sorted = place<int32_t>(off, (size_t)nnz), o_rowof = place<int32_t>(off, (size_t)nnz);
    const size_t o_temp = place<uint8_t>(off, sort_temp);
    const size_t scratch_bytes = off + 256;
    void *scratch = nullptr;
    if (hipMallocAsync(&scratch, scratch_bytes, cs) != hipSuccess) {
        delete p;
        return BSFA_ERR_OOM;
    }
    uint8_t *sb = (uint8_t *)scratch;
    DevPlanArgs a{};
    a.row_ptr = v.row_ptr;
    a.col = v.col;
    a.piece_ptr = v.piece_ptr;
    a.tag = v.tag;
    a.n_qt = p->n_qt;
    a.n_kt = p->n_kt;
    a.bk = p->bk;
    a.sk = p->sk;
    a.end_bit = end_bit;
    a.nnz = nnz;
    a.row_full = (int64_t *)(sb + o_full);
    a.row_partial = (int64_t *)(sb + o_part);
    a.col_count = (int32_t *)(sb + o_cnt);
    a.iota = (int32_t *)(sb + o_iota);
    a.keys_out = (int32_t *)(sb + o_keys);
    a.sorted_e = (int32_t *)(sb + o_sorted);
    a.row_of = (int32_t *)(sb + o_rowof);
    a.temp = sb + o_temp;
    a.temp_bytes = sort_temp;
    auto fail = [&](bsfa_status code) {
        (void)hipFreeAsync(scratch, cs);
        delete p;
        return code;
    };

    // 1. counts on the device; the host receives row_ptr and n_qt + n_kt counts
    RowSteps rs;
    std::vector<int32_t> col_count;
    try {
        p->row_ptr.resize((size_t)p->n_qt + 1);
        rs.full.resize((size_t)p->n_qt);
        rs.partial.resize((size_t)p->n_qt);
        col_count.resize((size_t)p->n_kt);
    } catch (const std::bad_alloc &) {
        return fail(BSFA_ERR_OOM);
    }
    bool ok = launch_plan_counts(a, cs) == hipSuccess;
    ok = ok && hipMemcpyAsync(p->row_ptr.data(), v.row_ptr, p->row_ptr.size() * 4, hipMemcpyDeviceToHost, cs) ==
                   hipSuccess;
    if (p->n_qt > 0) {
        ok = ok && hipMemcpyAsync(rs.full.data(), a.row_full, rs.full.size() * 8, hipMemcpyDeviceToHost, cs) ==
                       hipSuccess;
        ok = ok && hipMemcpyAsync(rs.partial.data(), a.row_partial, rs.partial.size() * 8, hipMemcpyDeviceToHost,
                                  cs) == hipSuccess;
    }
    if (p->n_kt > 0)
        ok = ok && hipMemcpyAsync(col_count.data(), a.col_count, col_count.size() * 4, hipMemcpyDeviceToHost, cs) ==
                       hipSuccess;
    ok = ok && hipStreamSynchronize(cs) == hipSuccess;
    if (!ok) return fail(BSFA_ERR_HIP);

    // 2. column offsets, schedule and launch orders on the host (sizes n_qt, n_kt, items);
    //    a split row's entry costs come from its CSR entries (copied for that row only)
    try {
        p->t_ptr.assign((size_t)p->n_kt + 1, 0);
        for (int32_t kt = 0; kt < p->n_kt; ++kt) p->t_ptr[(size_t)kt + 1] = p->t_ptr[kt] + col_count[kt];
        bool copy_ok = true;
        build_schedule(*p, kNumCu * kBinsPerCu, rs, [&](int32_t e0, int32_t e1, std::vector<double> &outc) {
            std::vector<int32_t> c((size_t)(e1 - e0));
            std::vector<uint8_t> t((size_t)(e1 - e0));
            copy_ok = copy_ok && hipMemcpy(c.data(), v.col + e0, c.size() * 4, hipMemcpyDeviceToHost) == hipSuccess &&
                      hipMemcpy(t.data(), v.tag + e0, t.size(), hipMemcpyDeviceToHost) == hipSuccess;
            outc.resize(c.size());
            for (size_t i = 0; i < c.size(); ++i)
                outc[i] = (double)entry_steps(*p, c[i]) * bsfa_tile_cost(t[i], kCostPartial);
        });
        if (!copy_ok) return fail(BSFA_ERR_HIP);
        build_orders(*p);
    } catch (const std::bad_alloc &) {
        return fail(BSFA_ERR_OOM);
    }

    // 3. the device image: the host-built sections go through one compact pinned image,
    //    the CSR sections (entries, pieces, column view) are written on the device
    const ImageLayout L = image_layout(*p);
    struct Sec {
        size_t at;          // offset in the device image
        const void *src;
        size_t bytes;
        size_t staged = 0;  // offset in the compact host image
    };
    Sec secs[] = {{L.row, p->row_ptr.data(), p->row_ptr.size() * 4},
                  {L.bp, p->bin_ptr.data(), p->bin_ptr.size() * 4},
                  {L.bi, p->bin_items.data(), p->bin_items.size() * 4},
                  {L.un, p->units.data(), p->units.size() * sizeof(Unit)},
                  {L.sp, p->splits.data(), p->splits.size() * sizeof(Split)},
                  {L.tp, p->t_ptr.data(), p->t_ptr.size() * 4},
                  {L.oq, p->dq_order.data(), p->dq_order.size() * 4},
                  {L.ok, p->dkv_order.data(), p->dkv_order.size() * 4}};
    size_t staged = 0;
    for (Sec &x : secs) x.staged = place<uint8_t>(staged, x.bytes);
    Staging *stg = nullptr;
    st = staging_acquire(dev, staged + 256, &stg);
    if (st != BSFA_OK) return fail(st);
    uint8_t *h = (uint8_t *)stg->host;
    for (const Sec &x : secs)
        if (x.bytes) std::memcpy(h + x.staged, x.src, x.bytes);
    DevSlot *slot = nullptr;
    st = dev_acquire(dev, L.bytes, &slot);
    if (st != BSFA_OK) {
        staging_release_now(stg);
        return fail(st);
    }
    uint8_t *base = (uint8_t *)slot->ptr;
    for (const Sec &x : secs)
        ok = ok && (x.bytes == 0 ||
                    hipMemcpyAsync(base + x.at, h + x.staged, x.bytes, hipMemcpyHostToDevice, cs) == hipSuccess);
    if (ok && v.n_pieces > 0)
        ok = hipMemcpyAsync(base + L.pc, v.pieces, (size_t)v.n_pieces * sizeof(Piece), hipMemcpyDeviceToDevice, cs) ==
             hipSuccess;
    a.entries = (Entry *)(base + L.ent);
    a.t_list = (int32_t *)(base + L.tl);
    ok = ok && launch_plan_image(a, cs) == hipSuccess;
    ok = ok && hipEventRecord(stg->copied, cs) == hipSuccess && hipEventRecord(slot->ready, cs) == hipSuccess;
    // the image's kernels and copies read the compiled CSR's buffer: its completion event
    // now stands behind them, so destroying the CSR waits for them
    ok = ok && hipEventRecord(csr->done, cs) == hipSuccess;
    (void)hipFreeAsync(scratch, cs);
    if (!ok) {
        (void)hipStreamSynchronize(cs);
        std::vector<hipStream_t> rel{cs};
        dev_release(slot, rel);
        staging_release_now(stg);
        delete p;
        return BSFA_ERR_HIP;
    }
    staging_in_flight(stg);
    p->dev.row_ptr = (const int32_t *)(base + L.row);
    p->dev.entries = (const Entry *)(base + L.ent);
    p->dev.pieces = (const Piece *)(base + L.pc);
    p->dev.bin_ptr = (const int32_t *)(base + L.bp);
    p->dev.bin_items = (const int32_t *)(base + L.bi);
    p->dev.units = (const Unit *)(base + L.un);
    p->dev.splits = (const Split *)(base + L.sp);
    p->dev.t_ptr = (const int32_t *)(base + L.tp);
    p->dev.t_list = (const int32_t *)(base + L.tl);
    p->dev.dq_order = (const int32_t *)(base + L.oq);
    p->dev.dkv_order = (const int32_t *)(base + L.ok);
    p->off_entries = L.ent;
    p->off_pieces = L.pc;
    p->dbuf = base;
    p->slot = slot;
    p->device = dev;
    p->ustream = cs;
    if (!plan_consistent(*p)) {
        // an internal error: the metadata must never reach a kernel
        bsfa_plan_destroy(p);
        return BSFA_ERR_PLAN;
    }
    *out = p;
    return BSFA_OK;
}

void bsfa_dcsr_destroy(bsfa_dcsr *c)
{
    if (!c) return;
    if (c->done) {
        (void)hipEventSynchronize(c->done);
        (void)hipEventDestroy(c->done);
    }
    if (c->buf) (void)hipFree(c->buf);
    delete static_cast<DcsrEx *>(c);
}

bsfa_status bsfa_set_rescale_threshold(float tau_log2)
{
    if (!(tau_log2 >= 0.f && tau_log2 <= 64.f)) return BSFA_ERR_ARG;
    g_rescale_tau.store(tau_log2, std::memory_order_relaxed);
    return BSFA_OK;
}

float bsfa_get_rescale_threshold(void) { return g_rescale_tau.load(std::memory_order_relaxed); }

const char *bsfa_status_str(bsfa_status s)
{
    switch (s) {
    case BSFA_OK: return "ok";
    case BSFA_ERR_ARG: return "invalid argument";
    case BSFA_ERR_SHAPE: return "shape mismatch";
    case BSFA_ERR_ALIGN: return "misaligned pointer or stride";
    case BSFA_ERR_UNSUPPORTED: return "unsupported head dim or tile size";
    case BSFA_ERR_MASK: return "invalid mask";
    case BSFA_ERR_OOM: return "out of memory";
    case BSFA_ERR_HIP: return "HIP runtime error";
    case BSFA_ERR_STATE: return "plan not uploaded to the current device";
    case BSFA_ERR_PLAN: return "plan metadata failed its consistency check";
    }
    return "unknown status";
}

}  // extern "C"

