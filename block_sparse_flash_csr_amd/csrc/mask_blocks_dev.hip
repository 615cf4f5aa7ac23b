// Device mask compiler for block-code masks whose blocks are the tiles: a uint8 code
// map (0 empty, 1 full, 2 causal inside the block) -> the tile CSR in device memory,
// equal entry for entry to the host compiler run on the block slices.
//
// MagiAttention v1.1.0 news, "Blackwell adaptation" list: the block-sparse mask's
// metadata generated on the device without instantiating a dense mask, kept as a CSR;
// UltraAttn blog 3 (Full / Causal / Empty blocks) and 3.3 (Empty blocks are skipped).
// With blocks equal to tiles every non-empty block is exactly one entry of its row:
// a full block is a full tile; a causal block (bottom-right aligned in its clipped
// extent) admits every in-range pair only when it has a single row, so it is a
// partial tile carrying itself as its one piece otherwise.
//
// Steps (one stream, no host synchronisation): one wave per query tile counts its
// entries and pieces and adds the tile counts and admitted pairs to the totals; two
// exclusive scans give row_ptr and the rows' first pieces; one wave per query tile then
// writes its entries in key-tile order (a ballot per 64 blocks gives each block its
// slot).
#include "dcsr_blocks.h"
#include "dev_sort.h"

namespace bsfa {
namespace {

constexpr int kThreadsBlk = 256;

// Rows and keys of block (i, j) that exist: [q0, q1) x [k0, k1).
struct BlockExt {
    int32_t q0, q1, k0, k1;
};

__device__ __forceinline__ BlockExt block_ext(const DcsrBlockArgs &a, int32_t i, int32_t j)
{
    BlockExt e;
    e.q0 = i * a.bq;
    e.q1 = min(e.q0 + a.bq, a.sq);
    e.k0 = j * a.bk;
    e.k1 = min(e.k0 + a.bk, a.sk);
    return e;
}

// A causal block of L rows and W keys, bottom-right aligned: row r (0-based) admits
// min(W, max(0, W - L + 1 + r)) keys.
__device__ __forceinline__ unsigned long long causal_pairs(int64_t L, int64_t W)
{
    const int64_t a0 = W - L + 1;
    return (unsigned long long)(a0 >= 0 ? L * a0 + L * (L - 1) / 2 : W * (W + 1) / 2);
}

__global__ void blk_zero_kernel(unsigned long long *__restrict__ totals)
{
    if (threadIdx.x < 8) totals[threadIdx.x] = 0ull;
}

// One wave per query tile: entries and pieces of the row (into cnt[i], pcnt[i]; the
// extra slot n_qt gets 0 so that the scans also give the totals) and the totals.
__global__ void blk_count_kernel(const DcsrBlockArgs a)
{
    const int32_t i = (int32_t)blockIdx.x * (kThreadsBlk / 64) + (int32_t)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (i > a.n_qt) return;
    if (i == a.n_qt) {
        if (lane == 0) {
            a.row_cnt[i] = 0;
            a.row_pcnt[i] = 0;
        }
        return;
    }
    int32_t cnt = 0, pcnt = 0, full = 0;
    unsigned long long pairs = 0;
    if (i < a.nbq) {
        const int32_t jn = min(a.nbk, a.n_kt);
        const uint8_t *row = a.codes + (int64_t)i * a.nbk;
        for (int32_t j = lane; j < jn; j += 64) {
            const uint8_t c = row[j];
            if (c == 0) continue;
            const BlockExt e = block_ext(a, i, j);
            const int64_t L = e.q1 - e.q0, W = e.k1 - e.k0;
            ++cnt;
            if (c == 1 || L == 1) {
                ++full;
                pairs += (unsigned long long)(L * W);
            } else {
                ++pcnt;
                pairs += causal_pairs(L, W);
            }
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        cnt += __shfl_down(cnt, off);
        pcnt += __shfl_down(pcnt, off);
        full += __shfl_down(full, off);
        pairs += __shfl_down(pairs, off);
    }
    if (lane == 0) {
        a.row_cnt[i] = cnt;
        a.row_pcnt[i] = pcnt;
        if (cnt > 0) {
            atomicAdd(&a.totals[0], (unsigned long long)cnt);
            atomicAdd(&a.totals[1], (unsigned long long)full);
            atomicAdd(&a.totals[2], (unsigned long long)(cnt - full));
            atomicAdd(&a.totals[3], (unsigned long long)pcnt);
            atomicAdd(&a.totals[4], pairs);
        }
    }
}

// piece_ptr[nnz] = n_pieces (the scans' totals).
__global__ void blk_tail_kernel(const DcsrBlockArgs a)
{
    if (threadIdx.x == 0) a.piece_ptr[a.row_ptr[a.n_qt]] = a.row_poff[a.n_qt];
}

// One wave per query tile: its entries in key-tile order.
__global__ void blk_write_kernel(const DcsrBlockArgs a)
{
    const int32_t i = (int32_t)blockIdx.x * (kThreadsBlk / 64) + (int32_t)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (i >= a.n_qt || i >= a.nbq) return;
    const int32_t jn = min(a.nbk, a.n_kt);
    const uint8_t *row = a.codes + (int64_t)i * a.nbk;
    int32_t e = a.row_ptr[i], p = a.row_poff[i];
    const int32_t rows = min(i * a.bq + a.bq, a.sq) - i * a.bq;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int32_t j0 = 0; j0 < jn; j0 += 64) {
        const int32_t j = j0 + lane;
        const uint8_t c = j < jn ? row[j] : (uint8_t)0;
        const bool part = c == 2 && rows > 1;
        const uint64_t nz = __builtin_amdgcn_ballot_w64(c != 0);
        const uint64_t pz = __builtin_amdgcn_ballot_w64(part);
        if (c != 0) {
            const BlockExt ex = block_ext(a, i, j);
            const int32_t me = e + __popcll(nz & below), mp = p + __popcll(pz & below);
            a.col[me] = j;
            a.tag[me] = part ? (uint8_t)BSFA_TILE_PARTIAL : (uint8_t)BSFA_TILE_FULL;
            a.piece_ptr[me] = mp;
            if (part) a.pieces[mp] = Piece{ex.q0, ex.q1, ex.k0, ex.k1, ex.k1 - ex.q1, 0, 0, 0};
        }
        e += __popcll(nz);
        p += __popcll(pz);
    }
}

}  // namespace

size_t dcsr_blocks_scan_temp_bytes(int32_t n) { return dev_scan_temp_bytes(n); }

hipError_t launch_dcsr_blocks(const DcsrBlockArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL(blk_zero_kernel, dim3(1), dim3(64), 0, stream, a.totals);
    const unsigned rows = (unsigned)((a.n_qt + 1 + 3) / 4);
    hipLaunchKernelGGL(blk_count_kernel, dim3(rows), dim3(kThreadsBlk), 0, stream, a);
    hipError_t err = dev_exclusive_scan((const int32_t *)a.row_cnt, a.row_ptr, (int64_t)a.n_qt + 1, a.temp,
                                        a.temp_bytes, stream);
    if (err != hipSuccess) return err;
    err = dev_exclusive_scan((const int32_t *)a.row_pcnt, a.row_poff, (int64_t)a.n_qt + 1, a.temp, a.temp_bytes,
                             stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(blk_tail_kernel, dim3(1), dim3(64), 0, stream, a);
    if (a.n_qt > 0 && a.nbq > 0)
        hipLaunchKernelGGL(blk_write_kernel, dim3((unsigned)((min(a.n_qt, a.nbq) + 3) / 4)), dim3(kThreadsBlk), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace bsfa
