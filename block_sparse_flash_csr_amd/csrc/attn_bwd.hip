// Backward of the masked attention for gfx950 (MI355X): dQ, dK, dV over the same tile
// CSR the forward runs on.
//
// What is computed (MagiAttention v1.1.0 news: the same flexible-mask attention runs
// forward and backward; FlashAttention-T blog, lineage paragraph: the tiled pass
// recomputes the softmax from the saved log-sum-exp instead of storing it):
//   P_ij  = 2^(c s_ij - LSE_i log2 e) on admitted pairs, s_ij = q_i . k_j, c = scale log2 e
//   D_i   = sum_e dO_ie O_ie                       (kernel 1)
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dQ_i  = scale sum_j dS_ij k_j                  (kernel 2: by query tile, CSR row)
//   dK_j  = scale sum_(h,i) dS_ij q_i,  dV_j = sum_(h,i) P_ij dO_i
//                                                  (kernel 3: by key tile, CSR column,
//                                                   over the query heads of its kv head)
// No atomics: every output element has one writer, so the result is deterministic.
//
// Design (own, for CDNA4):
//   * Kernel 2 mirrors the forward's transposed products: S^T = K Q^T and
//     dP^T = V dO^T with Q and dO held as B operands, so a lane owns one query column
//     and its LSE_i, D_i are scalars; dQ^T += K^T dS^T takes K^T from the LDS tile with
//     ds_read_b64_tr_b16 and dS^T straight from the accumulator registers.
//   * Kernel 3 takes S = Q K^T and dP = dO V^T with K and V held as B operands (a lane
//     owns one key), dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
//     transposed from LDS; the per-query LSE and D come from LDS as broadcasts.
//   * Tiles go HBM -> LDS with direct buffer loads; 16-byte chunks of a row are
//     XOR-swizzled by the row's low bits so that row reads are conflict-free.
//   * A row without any admitted key (and a row past the end) has LSE = -inf: its
//     weights are taken against -inf and come out exactly 0.
#include <climits>

#include "bsfa_internal.h"

namespace bsfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t *cptr_i32;
typedef const __attribute__((address_space(4))) i32x4 *cptr_i32x4;
typedef __attribute__((address_space(3))) void *lds_ptr;
typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;

constexpr int kThreads = 256;
constexpr int kStep = 64;                 // keys (kernel 2) or queries (kernel 3) per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr int32_t kRsrcWord3 = 0x00020000;

template <int D>
struct BCfg {
    static constexpr int NCH = D / 8;           // 16-byte chunks per row
    static constexpr int ROWB = 2 * D;          // bytes per row in LDS
    static constexpr int TILE_B = kStep * ROWB; // bytes of a 64-row tile
    static constexpr int KS = D / 16;           // k-steps over the head dim
    static constexpr int DB = D / 32;           // 32-row blocks over the head dim
    static constexpr int NBLK = TILE_B / 1024;  // 1 KB direct-load blocks per tile
};

// Byte offset of 16-byte chunk c of row r in a swizzled tile.
template <int D>
__device__ __forceinline__ uint32_t toff(int r, int c)
{
    return (uint32_t)(r * BCfg<D>::ROWB + ((c ^ (r & (BCfg<D>::NCH - 1))) << 4));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t addr = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// Bytes from the first of n rows (row stride st elements) to the end of the last
// row's D elements; 0 when n <= 0, which makes every load of the range read zeros.
template <int D>
__device__ __forceinline__ uint32_t extent(int n, int32_t st)
{
    return n > 0 ? ((uint32_t)(n - 1) * (uint32_t)st + (uint32_t)D) * 2u : 0u;
}

__device__ __forceinline__ int32_t cload(const int32_t *p, int i) { return ((cptr_i32)p)[i]; }

// 64 rows of a [tokens, heads, D] bf16 tensor (row stride st elements, n rows in range)
// into an LDS tile; the waves share the 1 KB blocks, rows past n land as zeros.
template <int D>
__device__ __forceinline__ void load_rows(const void *base, int32_t st, int n, char *tile, int wave)
{
    using C = BCfg<D>;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, extent<D>(n, st));
    const int lane = threadIdx.x & 63;
    for (int b = wave; b < C::NBLK; b += kThreads / 64) {
        const int p = 64 * b + lane, row = p / C::NCH, phys = p % C::NCH;
        const uint32_t goff = (uint32_t)(row * st * 2 + ((phys ^ (row & (C::NCH - 1))) << 4));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(tile + b * 1024), 16, (int)goff, 0, 0, 0);
    }
}

// B-operand fragment of one token row (dims 16 ks + 8 hh .. + 7 for every ks) from a
// bf16 tensor in global memory; rows past the end read as zero.
template <int D>
__device__ __forceinline__ void load_frag(const void *row_base, int32_t st, int rows, int l32, int hh,
                                          bf16x8 (&f)[BCfg<D>::KS])
{
    const __amdgpu_buffer_rsrc_t r = make_rsrc(row_base, extent<D>(min(32, rows), st));
#pragma unroll
    for (int ks = 0; ks < BCfg<D>::KS; ++ks)
        f[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               r, (int)(l32 * st * 2 + 32 * ks + 16 * hh), 0, 0));
}

// A operand read along a tile row: row r, chunk c (8 elements).
template <int D>
__device__ __forceinline__ bf16x8 rd_row(const char *tile, int r, int c)
{
    return *(const bf16x8 *)(tile + toff<D>(r, c));
}

// A operand of X^T for a 64-row tile X: head dims 32 db .. + 31 (the A rows) against
// tile rows 16 ks .. + 15 (the k index), element e of lane (l32, hh) <-> tile row
// 16 ks + 8 (e >> 2) + 4 hh + (e & 3): two transpose reads of 4 rows each.
template <int D>
__device__ __forceinline__ bf16x8 rd_tr(const char *tile, int db, int ks, int lane)
{
    const int grp = lane >> 4, i16 = lane & 15, r = i16 >> 2, c4 = i16 & 3, hh = lane >> 5;
    const int chunk = 4 * db + 2 * (grp & 1) + (c4 >> 1);
    const int row0 = 16 * ks + 4 * hh + r, row1 = row0 + 8;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(tile + toff<D>(row0, chunk) + (c4 & 1) * 8));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(tile + toff<D>(row1, chunk) + (c4 & 1) * 8));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

__device__ __forceinline__ uint64_t range_bits(int lo, int hi)
{
    lo = max(lo, 0);
    hi = min(hi, 64);
    if (lo >= hi) return 0ull;
    const uint64_t upto_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
    return upto_hi & ~((1ull << lo) - 1ull);
}

// Accumulator element (block b, register r) sits at offset 32 b + 8 (r >> 2) + (r & 3)
// from base = first + 4 hh along the tile's 64-long axis.
__device__ __forceinline__ void mask_scores(uint64_t m, f32x16 (&s)[2])
{
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int32_t w = (int32_t)(b ? (uint32_t)(m >> 32) : (uint32_t)m);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            const int32_t keep = (w << (31 - off)) >> 31;
            s[b][r] = __int_as_float((keep & __float_as_int(s[b][r])) | (~keep & __float_as_int(-INFINITY)));
        }
    }
}

// bf16 B operands from 2 accumulator blocks (block b registers 0..7 -> k-step 2b,
// 8..15 -> 2b+1), the same k mapping rd_tr reads.
__device__ __forceinline__ void to_bf16_operands(const f32x16 (&x)[2], bf16x8 (&out)[4])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = x[j >> 1][(j & 1) * 8 + e];
        out[j] = __builtin_convertvector(t, bf16x8);
    }
}

// ---------------------------------------------------------------------------
// kernel 1: D = rowsum(dO * O), one lane group of D/8 per (token, head) row
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads) bwd_delta_kernel(const BwdArgs a)
{
    constexpr int TPR = D / 8, RPB = kThreads / TPR;
    const int h = blockIdx.y;
    const int i = (int)blockIdx.x * RPB + (int)threadIdx.x / TPR;
    const int c = ((int)threadIdx.x % TPR) * 8;
    float s = 0.f;
    if (i < a.sq) {
        const bf16x8 o = *(const bf16x8 *)((const __bf16 *)a.o + (int64_t)i * a.o_st + (int64_t)h * a.o_sh + c);
        const bf16x8 g = *(const bf16x8 *)((const __bf16 *)a.dout + (int64_t)i * a.do_st + (int64_t)h * a.do_sh + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += (float)o[e] * (float)g[e];
    }
    // reduce over the TPR lanes of the row (they are adjacent and TPR divides 64)
#pragma unroll
    for (int w = TPR / 2; w >= 1; w >>= 1) s += __shfl_xor(s, w, 64);
    if (i < a.sq && (threadIdx.x % TPR) == 0) a.delta[(int64_t)h * a.lse_sh + i] = s;
}

// ---------------------------------------------------------------------------
// kernel 2: dQ by query tile (grid n_qt x hq), 64-key steps over the CSR row
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq_kernel(const BwdArgs a)
{
    using C = BCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[2 * C::TILE_B];
    char *Kt = smem, *Vt = smem + C::TILE_B;
    const int qt = blockIdx.x, h = blockIdx.y, g = h / (a.hq / a.hkv);
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qrow0 = qt * kKernelBq + wave * 32, qrow = qrow0 + l32;
    const bool qvalid = qrow < a.sq;

    bf16x8 qf[C::KS], gf[C::KS];
    load_frag<D>((const __bf16 *)a.q + (int64_t)qrow0 * a.q_st + (int64_t)h * a.q_sh, a.q_st, a.sq - qrow0, l32, hh,
                 qf);
    load_frag<D>((const __bf16 *)a.dout + (int64_t)qrow0 * a.do_st + (int64_t)h * a.do_sh, a.do_st,
                 a.sq - qrow0, l32, hh, gf);
    const float lse = qvalid ? a.lse[(int64_t)h * a.lse_sh + qrow] : -INFINITY;
    const float nl = lse == -INFINITY ? -INFINITY : -lse * kLog2e;   // exponent offset
    const float dlt = qvalid ? a.delta[(int64_t)h * a.lse_sh + qrow] : 0.f;
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

    const int e0 = cload(a.meta.row_ptr, qt), e1 = cload(a.meta.row_ptr, qt + 1);
    for (int e = e0; e < e1; ++e) {
        const i32x4 en = ((cptr_i32x4)a.meta.entries)[e];   // col, piece_begin, piece_count, tag
        for (int sub = 0; sub < a.bk_plan / kStep; ++sub) {
            const int kv0 = en[0] * a.bk_plan + sub * kStep;
            const int kv_end = min(en[0] * a.bk_plan + a.bk_plan, a.sk);
            const int nk = min(kStep, kv_end - kv0);
            if (nk <= 0) continue;
            load_rows<D>((const __bf16 *)a.k + (int64_t)kv0 * a.k_st + (int64_t)g * a.k_sh, a.k_st, nk, Kt, wave);
            load_rows<D>((const __bf16 *)a.v + (int64_t)kv0 * a.v_st + (int64_t)g * a.v_sh, a.v_st, nk, Vt, wave);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            // S^T = K Q^T and dP^T = V dO^T (keys x queries, two 32-key blocks)
            f32x16 s[2], dp[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                s[b] = f32x16{};
                dp[b] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(Kt, 32 * b + l32, 2 * ks + hh), qf[ks],
                                                                   s[b], 0, 0, 0);
                    dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(Vt, 32 * b + l32, 2 * ks + hh), gf[ks],
                                                                    dp[b], 0, 0, 0);
                }
            }
            // mask (partial tiles and key tails): this lane's query row over the keys
            const int base = kv0 + 4 * hh;
            if (en[3] == BSFA_TILE_PARTIAL || nk < kStep) {
                uint64_t m = range_bits(0, kv0 + nk - base);
                if (en[3] == BSFA_TILE_PARTIAL) {
                    uint64_t u = 0;
                    for (int pi = 0; pi < en[2]; ++pi) {
                        const i32x4 pc = ((cptr_i32x4)a.meta.pieces)[2 * (en[1] + pi)];
                        const int diag = ((cptr_i32)a.meta.pieces)[8 * (en[1] + pi) + 4];
                        if (qrow < pc[0] || qrow >= pc[1]) continue;
                        u |= range_bits(pc[2] - base, min(pc[3], qrow + diag + 1) - base);
                    }
                    m &= u;
                }
                mask_scores(m, s);
            }
            // dS^T = P^T (dP^T - D_i), P^T = 2^(c s - LSE_i log2 e)
            f32x16 ds[2];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], a.c, nl));
                    ds[b][r] = p * (dp[b][r] - dlt);
                }
            bf16x8 dsb[4];
            to_bf16_operands(ds, dsb);
            // dQ^T += K^T dS^T
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr<D>(Kt, db, ks, lane), dsb[ks], acc[db], 0, 0,
                                                                      0);
            __syncthreads();   // every wave is done with the tiles before the next loads
        }
    }
    // lane (query l32, half hh) holds dims 32 db + 8 g4 + 4 hh + 0..3 of its query
    if (qvalid) {
        float *out = a.dq + ((int64_t)qrow * a.hq + h) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = a.scale * acc[db][4 * g4 + t];
                *(f32x4 *)(out + 32 * db + 8 * g4 + 4 * hh) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// kernel 3: dK, dV by key tile (grid n_kt x hkv); a wave owns 32 keys; 64-query
// steps over the CSR column, for every query head of the key/value head
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads, 1) bwd_dkdv_kernel(const BwdArgs a)
{
    using C = BCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[2 * C::TILE_B + 2 * kStep * 4];
    char *Qt = smem, *Gt = smem + C::TILE_B;
    float *lse_s = (float *)(smem + 2 * C::TILE_B), *dlt_s = lse_s + kStep;
    const int kt = blockIdx.x, g = blockIdx.y, group = a.hq / a.hkv;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int key0 = kt * a.bk_plan + wave * 32, key = key0 + l32;

    bf16x8 kf[C::KS], vf[C::KS];
    load_frag<D>((const __bf16 *)a.k + (int64_t)key0 * a.k_st + (int64_t)g * a.k_sh, a.k_st, a.sk - key0, l32, hh, kf);
    load_frag<D>((const __bf16 *)a.v + (int64_t)key0 * a.v_st + (int64_t)g * a.v_sh, a.v_st, a.sk - key0, l32, hh, vf);
    f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    const int t0 = cload(a.meta.t_ptr, kt), t1 = cload(a.meta.t_ptr, kt + 1);
    for (int h = g * group; h < (g + 1) * group; ++h)
        for (int t = t0; t < t1; ++t) {
            const int qt = cload(a.meta.t_list, 2 * t), e = cload(a.meta.t_list, 2 * t + 1);
            const i32x4 en = ((cptr_i32x4)a.meta.entries)[e];
            for (int sub = 0; sub < kKernelBq / kStep; ++sub) {
                const int q0 = qt * kKernelBq + sub * kStep;
                const int nq = min(kStep, a.sq - q0);
                if (nq <= 0) continue;
                load_rows<D>((const __bf16 *)a.q + (int64_t)q0 * a.q_st + (int64_t)h * a.q_sh, a.q_st, nq, Qt, wave);
                load_rows<D>((const __bf16 *)a.dout + (int64_t)q0 * a.do_st + (int64_t)h * a.do_sh, a.do_st, nq, Gt,
                             wave);
                if (tid < kStep) {
                    const int i = q0 + tid;
                    lse_s[tid] = i < a.sq ? a.lse[(int64_t)h * a.lse_sh + i] : -INFINITY;
                    dlt_s[tid] = i < a.sq ? a.delta[(int64_t)h * a.lse_sh + i] : 0.f;
                }
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                // S = Q K^T and dP = dO V^T (queries x keys, two 32-query blocks)
                f32x16 s[2], dp[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    s[b] = f32x16{};
                    dp[b] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < C::KS; ++ks) {
                        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(Qt, 32 * b + l32, 2 * ks + hh), kf[ks],
                                                                       s[b], 0, 0, 0);
                        dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_row<D>(Gt, 32 * b + l32, 2 * ks + hh),
                                                                        vf[ks], dp[b], 0, 0, 0);
                    }
                }
                // mask of partial tiles: this lane's key over the 64 query rows
                if (en[3] == BSFA_TILE_PARTIAL) {
                    const int base = q0 + 4 * hh;
                    uint64_t m = 0;
                    for (int pi = 0; pi < en[2]; ++pi) {
                        const i32x4 pc = ((cptr_i32x4)a.meta.pieces)[2 * (en[1] + pi)];
                        const int diag = ((cptr_i32)a.meta.pieces)[8 * (en[1] + pi) + 4];
                        if (key < pc[2] || key >= pc[3]) continue;
                        // rows i of the piece with key <= i + diag
                        m |= range_bits(max(pc[0], key - diag) - base, pc[1] - base);
                    }
                    mask_scores(m, s);
                }
                // P = 2^(c s - LSE_i log2 e), dS = P (dP - D_i); rows of the lane's
                // registers: 32 b + 8 g4 + 4 hh + t
                f32x16 p[2], ds[2];
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 l4 = *(const f32x4 *)(lse_s + 32 * b + 8 * g4 + 4 * hh);
                        const f32x4 d4 = *(const f32x4 *)(dlt_s + 32 * b + 8 * g4 + 4 * hh);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const float nl = l4[t] == -INFINITY ? -INFINITY : -l4[t] * kLog2e;
                            const int r = 4 * g4 + t;
                            p[b][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], a.c, nl));
                            ds[b][r] = p[b][r] * (dp[b][r] - d4[t]);
                        }
                    }
                bf16x8 pb[4], dsb[4];
                to_bf16_operands(p, pb);
                to_bf16_operands(ds, dsb);
                // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr<D>(Gt, db, ks, lane), pb[ks], dv[db], 0,
                                                                         0, 0);
                        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_tr<D>(Qt, db, ks, lane), dsb[ks], dk[db],
                                                                         0, 0, 0);
                    }
                __syncthreads();   // every wave is done with the tiles before the next loads
            }
        }
    // lane (key l32, half hh) holds dims 32 db + 8 g4 + 4 hh + 0..3 of its key
    if (key < a.sk) {
        float *ok = a.dk + ((int64_t)key * a.hkv + g) * D, *ov = a.dv + ((int64_t)key * a.hkv + g) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 wk, wv;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    wk[t] = a.scale * dk[db][4 * g4 + t];
                    wv[t] = dv[db][4 * g4 + t];
                }
                *(f32x4 *)(ok + 32 * db + 8 * g4 + 4 * hh) = wk;
                *(f32x4 *)(ov + 32 * db + 8 * g4 + 4 * hh) = wv;
            }
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t stream)
{
    constexpr int RPB = kThreads / (D / 8);
    if (a.sq > 0) {
        hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((a.sq + RPB - 1) / RPB, a.hq), dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(a.n_qt, a.hq), dim3(kThreads), 0, stream, a);
    }
    if (a.sk > 0) hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(a.n_kt, a.hkv), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs &a, int d, hipStream_t stream)
{
    return d == 128 ? launch_bwd_d<128>(a, stream) : launch_bwd_d<64>(a, stream);
}

}  // namespace bsfa
