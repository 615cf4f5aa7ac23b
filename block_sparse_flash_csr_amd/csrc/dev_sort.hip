// Device exclusive scan and stable LSD radix sort for the device mask compiler and the
// device-built plans (MagiAttention v1.1.0 news, "Blackwell adaptation" list: block-sparse
// mask metadata generated on the device and kept as a CSR).
//
// Scan: one workgroup per 4096 values.  The workgroups' sums are scanned the same way
// (recursively, in the caller's temp), then every workgroup scans its own values in 16
// rounds of 256 (one value per thread, coalesced) with its carry added.
//
// Sort, one pass per 8-bit digit: (1) each workgroup counts the digits of its 4096 keys
// into a digit-major table (digit d of workgroup b at d * n_blocks + b); (2) that table is
// exclusive-scanned, which gives every (digit, workgroup) its first output slot; (3) each
// workgroup walks its keys in index order, 256 at a time: the lanes of a wave holding
// the same digit find one another with 8 ballots (a key's rank = lanes below it with
// that digit), the waves are ordered through their digit counts in LDS, and the key is
// staged in LDS at its digit's start + its rank; the staged keys then go out in order,
// each digit's run to consecutive slots from the digit's first slot.  Keys with equal
// digits keep their order, so the passes compose to a stable sort.  No atomics outside
// LDS counters; results do not depend on timing.
#include "dev_sort.h"

#include <climits>

namespace bsfa {
namespace {

constexpr int kT = 256;               // threads per workgroup (4 waves)
constexpr int kItems = 16;            // values per thread
constexpr int kTile = kT * kItems;    // values per workgroup
constexpr int kWaves = kT / 64;
constexpr size_t kAlign = 256;
static_assert(kT == 256, "one thread per digit value in the sort kernels");

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t n_tiles(int64_t n) { return (n + kTile - 1) / kTile; }

// Inclusive scan of one value per lane over the wave.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Exclusive scan of one value per thread over the workgroup; total receives the sum.
// Every thread of the workgroup must call it (it holds two barriers).
__device__ __forceinline__ int32_t block_excl_scan(int32_t x, int32_t *wsum, int32_t &total)
{
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int32_t inc = wave_incl_scan(x, lane);
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int32_t before = 0;
    total = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
        const int32_t s = wsum[ww];
        if (ww < w) before += s;
        total += s;
    }
    __syncthreads();   // wsum is rewritten by the next call
    return before + inc - x;
}

__global__ void __launch_bounds__(kT) scan_sums_kernel(const int32_t *__restrict__ in, int64_t n,
                                                       int32_t *__restrict__ sums)
{
    __shared__ int32_t wsum[kWaves];
    const int64_t base = (int64_t)blockIdx.x * kTile;
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t k = base + i * kT + threadIdx.x;
        if (k < n) s += in[k];
    }
    int32_t total;
    block_excl_scan(s, wsum, total);
    if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

// in may equal out: every thread reads its value before the barriers that precede its
// write, and no other thread touches that element.
__global__ void __launch_bounds__(kT) scan_apply_kernel(const int32_t *in, int64_t n,
                                                        const int32_t *__restrict__ carry, int32_t *out)
{
    __shared__ int32_t wsum[kWaves];
    const int64_t base = (int64_t)blockIdx.x * kTile;
    int32_t run = carry ? carry[blockIdx.x] : 0;
    for (int i = 0; i < kItems; ++i) {
        const int64_t k = base + i * kT + threadIdx.x;
        const int32_t x = k < n ? in[k] : 0;
        int32_t total;
        const int32_t ex = block_excl_scan(x, wsum, total);
        if (k < n) out[k] = run + ex;
        run += total;
    }
}

size_t scan_temp_elems(int64_t n)
{
    const int64_t nb = n_tiles(n);
    return nb > 1 ? (size_t)nb + scan_temp_elems(nb) : 0;
}

hipError_t scan_rec(const int32_t *in, int32_t *out, int64_t n, int32_t *temp, hipStream_t s)
{
    const int64_t nb = n_tiles(n);
    if (nb > 1) {
        hipLaunchKernelGGL(scan_sums_kernel, dim3((unsigned)nb), dim3(kT), 0, s, in, n, temp);
        const hipError_t e = scan_rec(temp, temp, nb, temp + nb, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)nb), dim3(kT), 0, s, in, n, nb > 1 ? temp : nullptr,
                       out);
    return hipGetLastError();
}

// Per-workgroup digit counts, digit-major.
template <typename K>
__global__ void __launch_bounds__(kT) rs_hist_kernel(const K *__restrict__ keys, int64_t n, int shift,
                                                     int32_t *__restrict__ hist, int32_t nblk)
{
    __shared__ int32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kTile;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t k = base + i * kT + threadIdx.x;
        if (k < n) atomicAdd(&h[(int)((keys[k] >> shift) & 0xFFu)], 1);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter of one digit pass; off holds the exclusive scan of the digit table.
// The workgroup first orders its keys by digit in LDS (stable), then writes each digit's
// run to consecutive output slots, so that neighbouring threads store to neighbouring
// addresses.
template <typename K, bool PAIRS>
__global__ void __launch_bounds__(kT) rs_scatter_kernel(const K *__restrict__ keys, const int32_t *__restrict__ vals,
                                                        int64_t n, int shift, const int32_t *__restrict__ off,
                                                        int32_t nblk, K *__restrict__ keys_out,
                                                        int32_t *__restrict__ vals_out)
{
    __shared__ K skey[kTile];                       // the tile's keys in digit order
    __shared__ int32_t sval[PAIRS ? kTile : 1];
    __shared__ int32_t gslot[256];                  // first output slot of every digit
    __shared__ int32_t lstart[256];                 // first staged position of every digit
    __shared__ int32_t run[256];                    // keys of every digit staged so far
    __shared__ int32_t wcnt[kWaves][256];           // per-wave digit counts of the current round
    __shared__ int32_t wsum[kWaves];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int64_t base = (int64_t)blockIdx.x * kTile;
    const int32_t count = (int32_t)(n - base < kTile ? n - base : kTile);   // keys of this tile

    // this tile's digit counts -> where each digit starts in the staged order
    run[t] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t k = base + i * kT + t;
        if (k < n) atomicAdd(&run[(int)((keys[k] >> shift) & 0xFFu)], 1);
    }
    __syncthreads();
    int32_t total;
    const int32_t c = run[t];
    lstart[t] = block_excl_scan(c, wsum, total);
    run[t] = 0;
    gslot[t] = off[(int64_t)t * nblk + blockIdx.x];
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) wcnt[ww][t] = 0;
    __syncthreads();

    // stage the keys in index order within each digit
    const uint64_t below = (1ull << lane) - 1ull;
    for (int i = 0; i < kItems; ++i) {
        const int64_t k = base + i * kT + t;
        const bool valid = k < n;
        const K key = valid ? keys[k] : (K)0;
        const int32_t val = (PAIRS && valid) ? vals[k] : 0;
        const int d = (int)((key >> shift) & 0xFFu);
        // lanes of this wave that hold a key with the same digit
        uint64_t same = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1;
            const uint64_t ones = __builtin_amdgcn_ballot_w64(bit);
            same &= bit ? ones : ~ones;
        }
        const int rank = __popcll(same & below);
        if (valid && rank == 0) wcnt[w][d] = __popcll(same);
        __syncthreads();
        if (valid) {
            int32_t lp = lstart[d] + run[d] + rank;
            for (int ww = 0; ww < w; ++ww) lp += wcnt[ww][d];
            if (lp >= 0 && lp < count) {   // always true when the counts agree
                skey[lp] = key;
                if (PAIRS) sval[lp] = val;
            }
        }
        __syncthreads();
        int32_t cw = 0;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            cw += wcnt[ww][t];
            wcnt[ww][t] = 0;
        }
        run[t] += cw;
        __syncthreads();
    }

    // write the staged keys: digit d's j-th key goes to gslot[d] + j
    for (int i = 0; i < kItems; ++i) {
        const int32_t j = i * kT + t;
        if (j < count) {
            const K key = skey[j];
            const int d = (int)((key >> shift) & 0xFFu);
            const int64_t pos = (int64_t)gslot[d] + (j - lstart[d]);
            if (pos >= 0 && pos < n) {   // always true when the counts agree
                keys_out[pos] = key;
                if (PAIRS) vals_out[pos] = sval[j];
            }
        }
    }
}

template <typename K>
__global__ void __launch_bounds__(kT) copy_kernel(const K *__restrict__ in, K *__restrict__ out, int64_t n)
{
    const int64_t k = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (k < n) out[k] = in[k];
}

// Temp layout of a sort: the second key buffer, the second value buffer (pairs), the
// digit table and the scan's temp.
struct SortLayout {
    size_t alt_keys, alt_vals, hist, scan, total;
};

template <typename K, bool PAIRS>
SortLayout sort_layout(int64_t n)
{
    SortLayout L{};
    const int64_t nblk = n_tiles(n);
    size_t p = 0;
    L.alt_keys = p;
    p += align_up((size_t)n * sizeof(K));
    L.alt_vals = p;
    if (PAIRS) p += align_up((size_t)n * sizeof(int32_t));
    L.hist = p;
    p += align_up((size_t)nblk * 256 * sizeof(int32_t));
    L.scan = p;
    p += dev_scan_temp_bytes(nblk * 256);
    L.total = p;
    return L;
}

template <typename K, bool PAIRS>
hipError_t radix_sort(const K *kin, K *kout, const int32_t *vin, int32_t *vout, int64_t n, int32_t end_bit,
                      void *temp, size_t temp_bytes, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    if (n >= INT32_MAX || end_bit < 0 || end_bit > 8 * (int32_t)sizeof(K)) return hipErrorInvalidValue;
    if (!kin || !kout || (PAIRS && (!vin || !vout))) return hipErrorInvalidValue;
    const int passes = (end_bit + 7) / 8;
    if (passes == 0) {
        const dim3 g((unsigned)((n + kT - 1) / kT));
        hipLaunchKernelGGL(copy_kernel<K>, g, dim3(kT), 0, s, kin, kout, n);
        if (PAIRS) hipLaunchKernelGGL(copy_kernel<int32_t>, g, dim3(kT), 0, s, vin, vout, n);
        return hipGetLastError();
    }
    const SortLayout L = sort_layout<K, PAIRS>(n);
    if (!temp || temp_bytes < L.total) return hipErrorInvalidValue;
    char *tb = (char *)temp;
    K *alt_k = (K *)(tb + L.alt_keys);
    int32_t *alt_v = (int32_t *)(tb + L.alt_vals);
    int32_t *hist = (int32_t *)(tb + L.hist);
    const int64_t nblk = n_tiles(n);
    if (nblk * 256 >= INT32_MAX) return hipErrorInvalidValue;
    const K *src_k = kin;
    const int32_t *src_v = vin;
    for (int p = 0; p < passes; ++p) {
        // the last pass writes the output; earlier ones alternate so that it does
        const bool to_out = ((passes - 1 - p) & 1) == 0;
        K *dst_k = to_out ? kout : alt_k;
        int32_t *dst_v = to_out ? vout : alt_v;
        hipLaunchKernelGGL(rs_hist_kernel<K>, dim3((unsigned)nblk), dim3(kT), 0, s, src_k, n, 8 * p, hist,
                           (int32_t)nblk);
        const hipError_t e = dev_exclusive_scan(hist, hist, nblk * 256, tb + L.scan, L.total - L.scan, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((rs_scatter_kernel<K, PAIRS>), dim3((unsigned)nblk), dim3(kT), 0, s, src_k, src_v, n,
                           8 * p, (const int32_t *)hist, (int32_t)nblk, dst_k, dst_v);
        src_k = dst_k;
        src_v = dst_v;
    }
    return hipGetLastError();
}

}  // namespace

size_t dev_scan_temp_bytes(int64_t n) { return n > 0 ? align_up(scan_temp_elems(n) * sizeof(int32_t)) : 0; }

hipError_t dev_exclusive_scan(const int32_t *in, int32_t *out, int64_t n, void *temp, size_t temp_bytes,
                              hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    if (n >= INT32_MAX || !in || !out) return hipErrorInvalidValue;
    const size_t need = dev_scan_temp_bytes(n);
    if (need > 0 && (!temp || temp_bytes < need)) return hipErrorInvalidValue;
    return scan_rec(in, out, n, (int32_t *)temp, stream);
}

size_t dev_sort_keys_temp_bytes(int64_t n, int32_t /*end_bit*/)
{
    return n > 0 ? sort_layout<uint64_t, false>(n).total : 0;
}

hipError_t dev_sort_keys_u64(const uint64_t *keys_in, uint64_t *keys_out, int64_t n, int32_t end_bit, void *temp,
                             size_t temp_bytes, hipStream_t stream)
{
    return radix_sort<uint64_t, false>(keys_in, keys_out, nullptr, nullptr, n, end_bit, temp, temp_bytes, stream);
}

size_t dev_sort_pairs_temp_bytes(int64_t n, int32_t /*end_bit*/)
{
    return n > 0 ? sort_layout<uint32_t, true>(n).total : 0;
}

hipError_t dev_sort_pairs_u32(const uint32_t *keys_in, uint32_t *keys_out, const int32_t *vals_in, int32_t *vals_out,
                              int64_t n, int32_t end_bit, void *temp, size_t temp_bytes, hipStream_t stream)
{
    return radix_sort<uint32_t, true>(keys_in, keys_out, vals_in, vals_out, n, end_bit, temp, temp_bytes, stream);
}

}  // namespace bsfa
