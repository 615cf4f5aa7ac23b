// The device part of a plan built over a device-compiled tile CSR: the per-row step
// counts the scheduler weighs, the key-tile histogram of the column view, the kernels'
// entry records and the column view itself, all from the CSR arrays in device memory;
// only n_qt + n_kt counts travel to the host (for the min-heap schedule and the gradient
// launch orders), and the plan's device image is assembled where the CSR already is
// (MagiAttention v1.1.0 news, "Blackwell adaptation": block-sparse mask metadata built
// without a round trip through a dense or host form; UltraAttn blog 3.3: the 2-D block
// view of the mask, read by rows for queries and by columns for keys).
//
// The column view is the host's counting sort by key tile in a device form: a stable
// radix sort of the entries' key tiles (values: entry numbers), so within one key tile
// the entries stay in ascending entry order, i.e. ascending query tile, exactly as the
// host builds it.
#include "dev_sort.h"

#include "bsfa_internal.h"

namespace bsfa {
namespace {

constexpr int kThreadsPlan = 256;

inline unsigned grid_of(int64_t n) { return (unsigned)((n + kThreadsPlan - 1) / kThreadsPlan); }

// One wave per query tile: its full and partial 64-key steps.
__global__ void row_steps_kernel(const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col,
                                 const uint8_t *__restrict__ tag, int32_t n_qt, int32_t bk, int32_t sk,
                                 int64_t *__restrict__ full, int64_t *__restrict__ partial)
{
    const int32_t qt = (int32_t)blockIdx.x * (kThreadsPlan / 64) + (int32_t)(threadIdx.x >> 6);
    if (qt >= n_qt) return;
    const int lane = threadIdx.x & 63;
    long long f = 0, pa = 0;
    for (int32_t e = row_ptr[qt] + lane; e < row_ptr[qt + 1]; e += 64) {
        const int64_t c0 = (int64_t)col[e] * bk;
        const int64_t keys = min(c0 + (int64_t)bk, (int64_t)sk) - c0;
        const long long steps = (keys + kKernelBk - 1) / kKernelBk;
        if (tag[e] == BSFA_TILE_FULL) f += steps;
        else pa += steps;
    }
    for (int off = 32; off > 0; off >>= 1) {
        f += __shfl_down(f, off);
        pa += __shfl_down(pa, off);
    }
    if (lane == 0) {
        full[qt] = f;
        partial[qt] = pa;
    }
}

__global__ void zero_i32_kernel(int32_t *__restrict__ p, int64_t n)
{
    const int64_t t = (int64_t)blockIdx.x * kThreadsPlan + threadIdx.x;
    if (t < n) p[t] = 0;
}

__global__ void col_count_kernel(const int32_t *__restrict__ col, int64_t nnz, int32_t *__restrict__ count)
{
    const int64_t e = (int64_t)blockIdx.x * kThreadsPlan + threadIdx.x;
    if (e < nnz) atomicAdd(&count[col[e]], 1);
}

// Entry records of the forward and backward kernels, and the entry numbers to sort.
__global__ void entries_kernel(const int32_t *__restrict__ col, const uint8_t *__restrict__ tag,
                               const int32_t *__restrict__ piece_ptr, int64_t nnz, Entry *__restrict__ out,
                               int32_t *__restrict__ iota)
{
    const int64_t e = (int64_t)blockIdx.x * kThreadsPlan + threadIdx.x;
    if (e >= nnz) return;
    out[e] = Entry{col[e], piece_ptr[e], piece_ptr[e + 1] - piece_ptr[e], (int32_t)tag[e]};
    iota[e] = (int32_t)e;
}

// Query tile of every entry (the row whose range [row_ptr[qt], row_ptr[qt + 1]) holds it).
__global__ void row_of_kernel(const int32_t *__restrict__ row_ptr, int32_t n_qt, int64_t nnz,
                              int32_t *__restrict__ row_of)
{
    const int64_t e = (int64_t)blockIdx.x * kThreadsPlan + threadIdx.x;
    if (e >= nnz) return;
    int32_t lo = 0, hi = n_qt;   // row_ptr[lo] <= e < row_ptr[hi]
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (row_ptr[mid] <= e) lo = mid;
        else hi = mid;
    }
    row_of[e] = lo;
}

__global__ void tlist_kernel(const int32_t *__restrict__ sorted_e, const int32_t *__restrict__ row_of, int64_t nnz,
                             int32_t *__restrict__ t_list)
{
    const int64_t i = (int64_t)blockIdx.x * kThreadsPlan + threadIdx.x;
    if (i >= nnz) return;
    const int32_t e = sorted_e[i];
    t_list[2 * i] = row_of[e];
    t_list[2 * i + 1] = e;
}

}  // namespace

hipError_t launch_plan_counts(const DevPlanArgs &a, hipStream_t stream)
{
    if (a.n_qt > 0)
        hipLaunchKernelGGL(row_steps_kernel, dim3((unsigned)((a.n_qt + 3) / 4)), dim3(kThreadsPlan), 0, stream,
                           a.row_ptr, a.col, a.tag, a.n_qt, a.bk, a.sk, a.row_full, a.row_partial);
    if (a.n_kt > 0) {
        hipLaunchKernelGGL(zero_i32_kernel, dim3(grid_of(a.n_kt)), dim3(kThreadsPlan), 0, stream, a.col_count,
                           (int64_t)a.n_kt);
        if (a.nnz > 0)
            hipLaunchKernelGGL(col_count_kernel, dim3(grid_of(a.nnz)), dim3(kThreadsPlan), 0, stream, a.col, a.nnz,
                               a.col_count);
    }
    return hipGetLastError();
}

size_t plan_sort_temp_bytes(int64_t nnz, int32_t end_bit) { return dev_sort_pairs_temp_bytes(nnz, end_bit); }

hipError_t launch_plan_image(const DevPlanArgs &a, hipStream_t stream)
{
    if (a.nnz <= 0) return hipSuccess;
    hipLaunchKernelGGL(entries_kernel, dim3(grid_of(a.nnz)), dim3(kThreadsPlan), 0, stream, a.col, a.tag,
                       a.piece_ptr, a.nnz, a.entries, a.iota);
    hipLaunchKernelGGL(row_of_kernel, dim3(grid_of(a.nnz)), dim3(kThreadsPlan), 0, stream, a.row_ptr, a.n_qt,
                       a.nnz, a.row_of);
    const hipError_t err = dev_sort_pairs_u32((const uint32_t *)a.col, (uint32_t *)a.keys_out, (const int32_t *)a.iota,
                                              a.sorted_e, a.nnz, a.end_bit, a.temp, a.temp_bytes, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(tlist_kernel, dim3(grid_of(a.nnz)), dim3(kThreadsPlan), 0, stream,
                       (const int32_t *)a.sorted_e, (const int32_t *)a.row_of, a.nnz, a.t_list);
    return hipGetLastError();
}

}  // namespace bsfa
