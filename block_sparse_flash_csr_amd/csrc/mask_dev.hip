// Device mask compiler: a slice list -> the tile CSR (row_ptr, col, tag, piece_ptr,
// pieces) in device memory, equal entry for entry to the host compiler.
//
// Follows the MagiAttention v1.1.0 news ("Blackwell adaptation" list: block-sparse mask
// generation without a dense mask, CSR mask metadata) and the UltraAttn blog, 3 (Full /
// Causal / Empty blocks) and 3.3 (Empty blocks are skipped).  The rule is the host
// compiler's: a tile is an entry when some slice reaches it; it is full when one slice
// alone admits every in-range pair or the union of the clipped slices does, partial
// otherwise, and a partial tile keeps its clipped slices in ascending slice order.
//
// Steps (one stream, no host synchronisation):
//   1. expand: the host lists every (slice, query tile) pair with the key-tile range the
//      slice reaches there and the pair's output offset (O(sum of query tiles per
//      slice)); one wave per pair writes the keys (tile << sbits) | slice;
//   2. stable radix sort of the keys (dev_sort.hip), so a tile's incidences are adjacent and in
//      slice order, tiles in (query tile, key tile) order;
//   3. heads of equal-tile runs -> entry numbers (exclusive scan);
//   4. per entry: full / partial, admitted pairs (closed form for one slice, a per-row
//      bitmap union for several), piece count;
//   5. piece offsets (exclusive scan), then col, tag, piece_ptr, pieces, row_ptr and the
//      totals.
#include <algorithm>

#include "dev_sort.h"

#include "bsfa_internal.h"

namespace bsfa {
namespace {

constexpr int kThreadsDev = 256;

struct Geometry {
    int32_t sq, sk, bq, bk, n_qt, n_kt, sbits;
};

__device__ __forceinline__ int64_t diag_of(const bsfa_slice &s)
{
    return s.type == BSFA_CAUSAL ? (int64_t)s.k1 - s.q1 : (int64_t)kDiagFull;
}

__global__ void expand_kernel(const int32_t *__restrict__ pair_info, const int64_t *__restrict__ pair_off,
                              int64_t n_pairs, Geometry g, uint64_t *__restrict__ keys)
{
    const int64_t pr = (int64_t)blockIdx.x * (kThreadsDev / 64) + (threadIdx.x >> 6);
    if (pr >= n_pairs) return;
    const int lane = threadIdx.x & 63;
    const int32_t s = pair_info[4 * pr], qt = pair_info[4 * pr + 1];
    const int32_t kt_lo = pair_info[4 * pr + 2], kt_hi = pair_info[4 * pr + 3];
    const int64_t off = pair_off[pr];
    for (int32_t kt = kt_lo + lane; kt < kt_hi; kt += 64) {
        const uint64_t tile = (uint64_t)qt * (uint64_t)g.n_kt + (uint64_t)kt;
        keys[off + (kt - kt_lo)] = (tile << g.sbits) | (uint64_t)s;
    }
}

__global__ void head_kernel(const uint64_t *__restrict__ keys, int64_t n, int32_t sbits, int32_t *__restrict__ flag)
{
    const int64_t t = (int64_t)blockIdx.x * kThreadsDev + threadIdx.x;
    if (t >= n) return;
    flag[t] = (t == 0 || (keys[t] >> sbits) != (keys[t - 1] >> sbits)) ? 1 : 0;
}

// Admitted pairs of one clipped slice in rows [r0, r1) x keys [c0, c1): row i admits
// [lo, min(hi, i + diag + 1)), an arithmetic ramp then a plateau.
__device__ int64_t piece_pairs(const bsfa_slice &s, int64_t r0, int64_t r1, int64_t c0, int64_t c1)
{
    const int64_t diag = diag_of(s);
    const int64_t a = max((int64_t)s.q0, r0), b = min((int64_t)s.q1, r1);
    const int64_t lo = max((int64_t)s.k0, c0), hi = min((int64_t)s.k1, c1);
    if (a >= b || lo >= hi) return 0;
    const int64_t i0 = lo - diag, i1 = hi - diag - 1;
    int64_t total = 0;
    const int64_t ra = max(a, i0), rb = min(b, i1);
    if (ra < rb) {
        const int64_t w0 = ra + diag + 1 - lo, w1 = rb - 1 + diag + 1 - lo;
        total += (w0 + w1) * (rb - ra) / 2;
    }
    const int64_t fa = max(a, max(i1, i0));
    if (fa < b) total += (b - fa) * (hi - lo);
    return total;
}

__device__ void entry_one(const uint64_t *__restrict__ keys, const int32_t *__restrict__ seg, int64_t t, int64_t n,
                          const Geometry &g, const bsfa_slice *__restrict__ slices, int32_t *__restrict__ e_first,
                          int32_t *__restrict__ e_n, uint8_t *__restrict__ e_full, int32_t *__restrict__ e_pieces,
                          unsigned long long &n_full, unsigned long long &n_part, unsigned long long &n_pairs)
{
    const uint64_t smask = (1ull << g.sbits) - 1ull;
    const uint64_t tile = keys[t] >> g.sbits;
    const int64_t qt = (int64_t)(tile / (uint64_t)g.n_kt), kt = (int64_t)(tile % (uint64_t)g.n_kt);
    const int64_t r0 = qt * g.bq, r1 = min(r0 + g.bq, (int64_t)g.sq);
    const int64_t c0 = kt * g.bk, c1 = min(c0 + g.bk, (int64_t)g.sk);
    const int64_t area = (r1 - r0) * (c1 - c0);
    int64_t u = t;
    bool covered = false;
    while (u < n && (keys[u] >> g.sbits) == tile) {
        const bsfa_slice s = slices[keys[u] & smask];
        const int64_t a = max((int64_t)s.q0, r0), b = min((int64_t)s.q1, r1);
        const bool rows_all = a == r0 && b == r1;
        covered |= rows_all && s.k0 <= c0 && s.k1 >= c1 && (c1 - 1) <= r0 + diag_of(s);
        ++u;
    }
    const int32_t cnt = (int32_t)(u - t);
    int64_t pairs = area;
    if (!covered) {
        if (cnt == 1) {
            pairs = piece_pairs(slices[keys[t] & smask], r0, r1, c0, c1);
        } else {
            // union of the clipped slices, row by row, as a bitmap of the tile's keys
            pairs = 0;
            for (int64_t i = r0; i < r1; ++i) {
                uint64_t m[4] = {0, 0, 0, 0};
                for (int64_t x = t; x < u; ++x) {
                    const bsfa_slice s = slices[keys[x] & smask];
                    if (i < s.q0 || i >= s.q1) continue;
                    const int64_t lo = max((int64_t)s.k0, c0) - c0;
                    const int64_t hi = min(min((int64_t)s.k1, i + diag_of(s) + 1), c1) - c0;
                    for (int w = 0; w < 4; ++w) {
                        const int64_t wl = max(lo, (int64_t)(64 * w)), wh = min(hi, (int64_t)(64 * w + 64));
                        if (wl >= wh) continue;
                        const int bl = (int)(wl - 64 * w), bh = (int)(wh - 64 * w);
                        const uint64_t upto = bh >= 64 ? ~0ull : ((1ull << bh) - 1ull);
                        m[w] |= upto & ~((1ull << bl) - 1ull);
                    }
                }
                pairs += __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]);
            }
        }
    }
    const bool full = covered || pairs == area;
    const int32_t e = seg[t];
    e_first[e] = (int32_t)t;
    e_n[e] = cnt;
    e_full[e] = full ? 1 : 0;
    e_pieces[e] = full ? 0 : cnt;
    (full ? n_full : n_part) = 1;
    n_pairs = (unsigned long long)pairs;
}

// Sum over the workgroup, left in thread 0 (every thread must call it).
__device__ void block_sum(unsigned long long &x)
{
    __shared__ unsigned long long part[kThreadsDev / 64];
    for (int w = 32; w >= 1; w >>= 1) x += __shfl_xor(x, w, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0)
        for (int w = 1; w < kThreadsDev / 64; ++w) x += part[w];
}

// Per entry (one thread per head of an equal-tile run): full / partial and counts.
__global__ void entry_kernel(const uint64_t *__restrict__ keys, const int32_t *__restrict__ flag,
                             const int32_t *__restrict__ seg, int64_t n, Geometry g,
                             const bsfa_slice *__restrict__ slices, int32_t *__restrict__ e_first,
                             int32_t *__restrict__ e_n, uint8_t *__restrict__ e_full,
                             int32_t *__restrict__ e_pieces, unsigned long long *__restrict__ totals)
{
    const int64_t t = (int64_t)blockIdx.x * kThreadsDev + threadIdx.x;
    unsigned long long n_full = 0, n_part = 0, n_pairs = 0;
    if (t < n && flag[t]) entry_one(keys, seg, t, n, g, slices, e_first, e_n, e_full, e_pieces, n_full, n_part, n_pairs);
    // one atomic per workgroup and total (8 million heads on one address serialise)
    block_sum(n_full);
    block_sum(n_part);
    block_sum(n_pairs);
    if (threadIdx.x == 0) {
        if (n_full) atomicAdd(&totals[1], n_full);
        if (n_part) atomicAdd(&totals[2], n_part);
        if (n_pairs) atomicAdd(&totals[4], n_pairs);
    }
}

// Output of entry e (one thread each): col, tag, piece_ptr, pieces, row_ptr.
__global__ void write_kernel(const uint64_t *__restrict__ keys, const int32_t *__restrict__ flag,
                             const int32_t *__restrict__ seg, int64_t n, Geometry g,
                             const bsfa_slice *__restrict__ slices, const int32_t *__restrict__ e_first,
                             const int32_t *__restrict__ e_n, const uint8_t *__restrict__ e_full,
                             const int32_t *__restrict__ e_pieces, const int32_t *__restrict__ p_off,
                             int32_t *__restrict__ row_ptr, int32_t *__restrict__ col, uint8_t *__restrict__ tag,
                             int32_t *__restrict__ piece_ptr, Piece *__restrict__ pieces,
                             unsigned long long *__restrict__ totals)
{
    const int64_t e = (int64_t)blockIdx.x * kThreadsDev + threadIdx.x;
    const int64_t nnz = n > 0 ? (int64_t)seg[n - 1] + flag[n - 1] : 0;
    if (e >= nnz) return;
    const uint64_t smask = (1ull << g.sbits) - 1ull;
    const int64_t t = e_first[e];
    const uint64_t tile = keys[t] >> g.sbits;
    const int32_t qt = (int32_t)(tile / (uint64_t)g.n_kt), kt = (int32_t)(tile % (uint64_t)g.n_kt);
    col[e] = kt;
    tag[e] = e_full[e] ? BSFA_TILE_FULL : BSFA_TILE_PARTIAL;
    piece_ptr[e] = p_off[e];
    if (!e_full[e]) {
        const int32_t r0 = qt * g.bq, r1 = min(r0 + g.bq, g.sq);
        const int32_t c0 = kt * g.bk, c1 = min(c0 + g.bk, g.sk);
        for (int32_t x = 0; x < e_n[e]; ++x) {
            const bsfa_slice s = slices[keys[t + x] & smask];
            Piece pc;
            pc.q_lo = max(s.q0, r0);
            pc.q_hi = min(s.q1, r1);
            pc.k_lo = max(s.k0, c0);
            pc.k_hi = min(s.k1, c1);
            pc.diag = s.type == BSFA_CAUSAL ? s.k1 - s.q1 : kDiagFull;
            pc.pad0 = pc.pad1 = pc.pad2 = 0;
            pieces[p_off[e] + x] = pc;
        }
    }
    // row_ptr[r] = first entry of a query tile >= r
    const int32_t prev = e == 0 ? -1 : (int32_t)((keys[e_first[e - 1]] >> g.sbits) / (uint64_t)g.n_kt);
    for (int32_t r = prev + 1; r <= qt; ++r) row_ptr[r] = (int32_t)e;
    if (e == nnz - 1) {
        for (int32_t r = qt + 1; r <= g.n_qt; ++r) row_ptr[r] = (int32_t)nnz;
        piece_ptr[nnz] = p_off[e] + e_pieces[e];
        totals[0] = (unsigned long long)nnz;
        totals[3] = (unsigned long long)(p_off[e] + e_pieces[e]);
    }
}

__global__ void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v)
{
    const int64_t t = (int64_t)blockIdx.x * kThreadsDev + threadIdx.x;
    if (t < n) p[t] = v;
}

__global__ void fill_u64_kernel(unsigned long long *__restrict__ p, int64_t n)
{
    const int64_t t = (int64_t)blockIdx.x * kThreadsDev + threadIdx.x;
    if (t < n) p[t] = 0ull;
}

inline unsigned grid_of(int64_t n) { return (unsigned)((n + kThreadsDev - 1) / kThreadsDev); }

}  // namespace

size_t dcsr_sort_temp_bytes(int64_t n, int32_t end_bit)
{
    return std::max(dev_sort_keys_temp_bytes(n, end_bit), dev_scan_temp_bytes(n));
}

hipError_t launch_dcsr(const DcsrArgs &a, hipStream_t stream)
{
    const Geometry g{a.sq, a.sk, a.bq, a.bk, a.n_qt, a.n_kt, a.sbits};
    const int64_t n = a.n_touch;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(kThreadsDev), 0, stream, a.totals, (int64_t)8);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_of(a.n_qt + 1)), dim3(kThreadsDev), 0, stream, a.row_ptr,
                       (int64_t)a.n_qt + 1, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(kThreadsDev), 0, stream, a.piece_ptr, (int64_t)1, 0);
    if (n == 0) return hipGetLastError();
    hipLaunchKernelGGL(expand_kernel, dim3((unsigned)((a.n_pairs + 3) / 4)), dim3(kThreadsDev), 0, stream,
                       a.pair_info, a.pair_off, a.n_pairs, g, a.keys_in);
    hipError_t err = dev_sort_keys_u64((const uint64_t *)a.keys_in, a.keys, n, a.end_bit, a.temp, a.temp_bytes,
                                       stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(head_kernel, dim3(grid_of(n)), dim3(kThreadsDev), 0, stream, (const uint64_t *)a.keys, n,
                       a.sbits, a.flag);
    err = dev_exclusive_scan((const int32_t *)a.flag, a.seg, n, a.temp, a.temp_bytes, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_of(n)), dim3(kThreadsDev), 0, stream, a.e_pieces, n, 0);
    hipLaunchKernelGGL(entry_kernel, dim3(grid_of(n)), dim3(kThreadsDev), 0, stream, (const uint64_t *)a.keys,
                       (const int32_t *)a.flag, (const int32_t *)a.seg, n, g, a.slices, a.e_first, a.e_n, a.e_full,
                       a.e_pieces, a.totals);
    err = dev_exclusive_scan((const int32_t *)a.e_pieces, a.p_off, n, a.temp, a.temp_bytes, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(write_kernel, dim3(grid_of(n)), dim3(kThreadsDev), 0, stream, (const uint64_t *)a.keys,
                       (const int32_t *)a.flag, (const int32_t *)a.seg, n, g, a.slices, (const int32_t *)a.e_first,
                       (const int32_t *)a.e_n, (const uint8_t *)a.e_full, (const int32_t *)a.e_pieces,
                       (const int32_t *)a.p_off, a.row_ptr, a.col, a.tag, a.piece_ptr, a.pieces, a.totals);
    return hipGetLastError();
}

}  // namespace bsfa
