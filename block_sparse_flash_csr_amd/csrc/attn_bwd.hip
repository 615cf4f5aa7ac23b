// Backward of the masked attention for gfx950 (MI355X): dQ, dK, dV over the same tile
// CSR the forward runs on.
//
// What is computed (MagiAttention v1.1.0 news: the same flexible-mask attention runs
// forward and backward; FlashAttention-T blog, lineage paragraph: the tiled pass
// recomputes the softmax from the saved log-sum-exp instead of storing it):
//   P_ij  = 2^(c s_ij - LSE_i log2 e) on admitted pairs, s_ij = q_i . k_j, c = scale log2 e
//   dP_ij = dO_i . v_j
//   D_i   = sum_j P_ij dP_ij                       (kernel 1: a first pass over the CSR
//                                                   row; equal to dO_i . O_i for the
//                                                   exact O, without the bf16 output's
//                                                   rounding)
//   dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = scale sum_j dS_ij k_j                  (kernel 2: by query tile, CSR row)
//   dK_j  = scale sum_(h,i) dS_ij q_i,  dV_j = sum_(h,i) P_ij dO_i
//                                                  (kernel 3: by key tile, CSR column,
//                                                   over the query heads of its kv head)
// No atomics: every output element has one writer, so the result is deterministic.
//
// Design (own, for CDNA4):
//   * Kernels 1 and 2 are one kernel body: kernel 1 forms only S^T and dP^T and sums
//     P dP per query row; kernel 2 reads that D and adds the dQ product.  A call that
//     passes the forward's fp32 O skips kernel 1: kernel 2 forms D_i = dO_i . O_i from
//     it (the fp32 value, without the bf16 output's rounding) and stores it for kernel 3.
//   * Kernel 2 mirrors the forward's transposed products: S^T = K Q^T and
//     dP^T = V dO^T with Q and dO held as B operands, so a lane owns one query column
//     and its LSE_i, D_i are scalars; dQ^T += K^T dS^T takes K^T from the LDS tile with
//     ds_read_b64_tr_b16 and dS^T straight from the accumulator registers.
//   * Kernel 3 takes S = Q K^T and dP = dO V^T with the key tile's K and V rows as B
//     operands read from LDS, where they stay for the whole workgroup (a lane owns one
//     key), dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read transposed from
//     LDS; the accumulators of S and dP start at -LSE / scale and -D, read from LDS as
//     broadcasts.  Eight waves, two per SIMD: a wave holds only its dK, dV partials.
//   * Tiles go HBM -> LDS with direct buffer loads; 16-byte chunks of a row are
//     XOR-swizzled by the row's low bits so that row reads are conflict-free.
//   * A row without any admitted key has LSE = -inf and only meets partial tiles, whose
//     mask gives its scores -inf: its weights come out exactly 0.  Rows past the end are
//     zero rows (with LSE = D = 0 in kernel 3, -inf in kernels 1 and 2) and contribute 0.
#include <climits>
#include <type_traits>

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
constexpr int kStep = 64;                 // keys (kernels 1, 2) or queries (kernel 3) per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr int32_t kRsrcWord3 = 0x00020000;

template <int D>
struct BCfg {
    static constexpr int NCH = D / 8;           // 16-byte chunks per row
    static constexpr int ROWB = 2 * D;          // bytes per row in LDS
    static constexpr int TILE_B = kStep * ROWB; // bytes of a 64-row tile
    static constexpr int KS = D / 16;           // k-steps over the head dim
    static constexpr int DB = D / 32;           // 32-row blocks over the head dim
};

// 16-byte chunk c of tile row r sits at chunk c ^ swz(r).  The pattern serves both reads
// of a tile: row reads (32 rows, one chunk each) see 16 (d 128) or 8 per row parity
// (d 64) different chunk positions, and transpose reads (rows 4 m .. 4 m + 3, a 4-chunk
// group each) put the 4 rows in 4 different 4-chunk groups of banks.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Byte offset of 16-byte chunk c of row r in a swizzled tile.
template <int D>
__device__ __forceinline__ uint32_t toff(int r, int c)
{
    return (uint32_t)(r * BCfg<D>::ROWB + ((c ^ swz<D>(r)) << 4));
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

// ROWS rows of a [tokens, heads, D] bf16 tensor (row stride st elements) from the
// buffer range r into an LDS tile; the NW waves share the 1 KB blocks, rows outside
// the range land as zeros.
template <int D, int ROWS = kStep, int NW = 4>
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t r, int32_t st, char *tile, int wave, int lane)
{
    using C = BCfg<D>;
    constexpr int NB = ROWS * C::ROWB / 1024;
    static_assert(NB % NW == 0, "the waves share the blocks evenly");
#pragma unroll
    for (int i = 0; i < NB / NW; ++i) {
        const int b = wave + NW * i;
        const int p = 64 * b + lane, row = p / C::NCH, phys = p % C::NCH;
        const uint32_t goff = (uint32_t)(row * st * 2 + ((phys ^ swz<D>(row)) << 4));
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

// Per-lane LDS offsets of the two tile reads, fixed for the whole kernel:
//   row[ks]    : chunk 2 ks + hh of tile row l32 (block b adds 32 b rows: the swizzle
//                depends on the row's low 4 bits only, so it is an immediate offset);
//   tr[db][j]  : the transpose read of head dims 32 db .. + 31, rows 4 hh + r + 8 j of
//                k-step 0 (k-step ks adds 16 ks rows, again an immediate).
template <int D>
struct Addr {
    uint32_t row[BCfg<D>::KS];
    uint32_t tr[BCfg<D>::DB][2];
};

template <int D>
__device__ __forceinline__ Addr<D> make_addr(int lane)
{
    using C = BCfg<D>;
    Addr<D> a;
    const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) a.row[ks] = toff<D>(l32, 2 * ks + hh);
    const int grp = lane >> 4, i16 = lane & 15, r = i16 >> 2, c4 = i16 & 3;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        const int chunk = 4 * db + 2 * (grp & 1) + (c4 >> 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) a.tr[db][j] = toff<D>(4 * hh + r + 8 * j, chunk) + (c4 & 1) * 8;
    }
    return a;
}

// A operand read along a tile row: rows 32 b + l32, chunk 2 ks + hh.
template <int D>
__device__ __forceinline__ bf16x8 rd_row(const char *tile, const Addr<D> &ad, int b, int ks)
{
    return *(const bf16x8 *)(tile + ad.row[ks] + 32 * b * BCfg<D>::ROWB);
}

// A operand of X^T for a 64-row tile X: head dims 32 db .. + 31 (the A rows) against
// tile rows 16 ks .. + 15 (the k index), element e of lane (l32, hh) <-> tile row
// 16 ks + 8 (e >> 2) + 4 hh + (e & 3): two transpose reads of 4 rows each.
template <int D>
__device__ __forceinline__ bf16x8 rd_tr(const char *tile, const Addr<D> &ad, int db, int ks)
{
    const char *p = tile + 16 * ks * BCfg<D>::ROWB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + ad.tr[db][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + ad.tr[db][1]));
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

// f(integral_constant<int, I>) for I = B .. E - 1, each with I a compile-time constant
// (long unrolled sequences of products exceed the unroller's limits; this never leaves
// one rolled with its accumulator arrays indexed at run time).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Operands are read this many products ahead of their MFMA (kernel 3, kernels 1 and 2).
constexpr int kAheadKv = 2, kAheadQ = 2;

// S += X Y^T and dP += Z W^T over one 64-row LDS tile pair (x_t, z_t) against the register
// fragments yf, wf (one 32-row block per wave): product i -> S (i even) or dP (i odd),
// row block (i >> 1) & 1, k-step i >> 2, so four independent accumulator chains rotate;
// the tile reads run AH products ahead.
template <int D, int AH>
__device__ __forceinline__ void score_products(const char *x_t, const char *z_t, const bf16x8 (&yf)[BCfg<D>::KS],
                                               const bf16x8 (&wf)[BCfg<D>::KS], const Addr<D> &ad, f32x16 (&s)[2],
                                               f32x16 (&dp)[2])
{
    constexpr int N1 = 4 * BCfg<D>::KS;
    auto rd1 = [&](int i) { return rd_row<D>((i & 1) ? z_t : x_t, ad, (i >> 1) & 1, i >> 2); };
    bf16x8 op[AH + 1];
#pragma unroll
    for (int i = 0; i < AH; ++i) op[i] = rd1(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N1; ++i) {
        if (i + AH < N1) op[(i + AH) % (AH + 1)] = rd1(i + AH);
        const int b = (i >> 1) & 1, ks = i >> 2;
        if (i & 1) dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (AH + 1)], wf[ks], dp[b], 0, 0, 0);
        else s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (AH + 1)], yf[ks], s[b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// kernels 1 and 2: D, then dQ, by query tile (one workgroup per (head, query tile), in
// the plan's launch order), 64-key steps over the CSR row; the K and V tiles of step
// j + 1 load (LDS double buffer) while step j computes
// ---------------------------------------------------------------------------
template <int D>
struct DqTiles {
    static constexpr int K0 = 0, V0 = BCfg<D>::TILE_B, BUF = 2 * BCfg<D>::TILE_B, BYTES = 2 * BUF;
};

// One dQ step: issue the next step's K/V loads into (kd, vd) when `issue`, then
// S^T = K Q^T, dP^T = V dO^T, dS^T = 2^(c S^T - LSE_i log2 e) (dP^T - D_i),
// dQ^T += K^T dS^T on (kt, vt).
// The restrict qualifiers tell the compiler that the loads in flight do not write the
// tiles this step reads.
template <int D>
__device__ __forceinline__ void dq_step(char *__restrict__ kd, char *__restrict__ vd, const char *__restrict__ kt,
                                        const char *__restrict__ vt, bool issue, __amdgpu_buffer_rsrc_t rk,
                                        __amdgpu_buffer_rsrc_t rv, int32_t k_st, int32_t v_st, int wave, int lane,
                                        const Addr<D> &ad, const bf16x8 (&qf)[BCfg<D>::KS], const bf16x8 (&gf)[BCfg<D>::KS], uint64_t m,
                                        bool masked_step, float c, float nl, float dlt,
                                        f32x16 (&acc)[BCfg<D>::DB])
{
    using C = BCfg<D>;
    if (issue) {
        tile_dma<D>(rk, k_st, kd, wave, lane);
        tile_dma<D>(rv, v_st, vd, wave, lane);
    }
    // a wave none of whose (query, key) pairs in this step is admitted adds nothing
    if (masked_step && __builtin_amdgcn_ballot_w64(m != 0ull) == 0ull) return;
    // (the dK/dV kernel starts its accumulators at -LSE / scale and -D; here, at two waves
    // per SIMD, those 64 live values would not fit beside Q, dO and dQ, so S and dP start
    // at 0 and the offsets are applied in the exponential)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        s[b] = f32x16{};
        dp[b] = f32x16{};
    }
    // The score products run at raised wave priority: the SIMD's other wave (of the other
    // resident workgroup, at its own point of the step) then gets the matrix unit back
    // while this wave exponentiates, instead of both waves contending for it in step.
    __builtin_amdgcn_s_setprio(1);
    score_products<D, kAheadQ>(kt, vt, qf, gf, ad, s, dp);
    __builtin_amdgcn_s_setprio(0);
    if (masked_step) mask_scores(m, s);
    f32x16 ds[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ds[b][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, nl)) * (dp[b][r] - dlt);
    bf16x8 dsb[4];
    to_bf16_operands(ds, dsb);
    // dQ^T += K^T dS^T: product i -> head-dim block i % DB, k-step i / DB
    constexpr int N2 = 4 * C::DB;
    bf16x8 op[kAheadQ + 1];
#pragma unroll
    for (int i = 0; i < kAheadQ; ++i) op[i] = rd_tr<D>(kt, ad, i % C::DB, i / C::DB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N2; ++i) {
        if (i + kAheadQ < N2) op[(i + kAheadQ) % (kAheadQ + 1)] = rd_tr<D>(kt, ad, (i + kAheadQ) % C::DB, (i + kAheadQ) / C::DB);
        acc[i % C::DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (kAheadQ + 1)], dsb[i / C::DB], acc[i % C::DB], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One step of the D pass: issue the next step's K/V loads, then S^T = K Q^T,
// dP^T = V dO^T and dsum += 2^(c S^T - LSE_i log2 e) dP^T over this lane's keys.
template <int D>
__device__ __forceinline__ void delta_step(char *__restrict__ kd, char *__restrict__ vd, const char *__restrict__ kt,
                                           const char *__restrict__ vt, bool issue, __amdgpu_buffer_rsrc_t rk,
                                           __amdgpu_buffer_rsrc_t rv, int32_t k_st, int32_t v_st, int wave, int lane,
                                           const Addr<D> &ad, const bf16x8 (&qf)[BCfg<D>::KS],
                                           const bf16x8 (&gf)[BCfg<D>::KS], uint64_t m, bool masked_step, float c,
                                           float nl, float &dsum)
{
    if (issue) {
        tile_dma<D>(rk, k_st, kd, wave, lane);
        tile_dma<D>(rv, v_st, vd, wave, lane);
    }
    if (masked_step && __builtin_amdgcn_ballot_w64(m != 0ull) == 0ull) return;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        s[b] = f32x16{};
        dp[b] = f32x16{};
    }
    __builtin_amdgcn_s_setprio(1);
    score_products<D, kAheadQ>(kt, vt, qf, gf, ad, s, dp);
    __builtin_amdgcn_s_setprio(0);
    if (masked_step) mask_scores(m, s);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dsum = __builtin_fmaf(__builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, nl)), dp[b][r], dsum);
}

// MODE 0: kernel 1 (D_i = sum_j P_ij dP_ij into `delta`); 1: kernel 2 (dQ, reading D);
// 2: kernel 2 taking D_i = dO_i . O_i from the forward's fp32 O (and storing it in
// `delta` for kernel 3), when the call has it.
template <int D, int MODE>
__device__ __forceinline__ void dq_body(const BwdArgs &a)
{
    constexpr bool DELTA = MODE == 0;
    using C = BCfg<D>;
    using L = DqTiles<D>;
    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
    const int item = cload(a.meta.dq_order, (int)blockIdx.x);
    const int h = item / a.n_qt, qt = item - h * a.n_qt, g = h / (a.hq / a.hkv);
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qrow0 = qt * kKernelBq + wave * 32, qrow = qrow0 + l32;
    const bool qvalid = qrow < a.sq;
    const int nsub = a.bk_plan / kStep;
    const Addr<D> ad = make_addr<D>(lane);

    bf16x8 qf[C::KS], gf[C::KS];
    load_frag<D>((const __bf16 *)a.q + (int64_t)qrow0 * a.q_st + (int64_t)h * a.q_sh, a.q_st, a.sq - qrow0, l32, hh,
                 qf);
    load_frag<D>((const __bf16 *)a.dout + (int64_t)qrow0 * a.do_st + (int64_t)h * a.do_sh, a.do_st,
                 a.sq - qrow0, l32, hh, gf);
    // exponent offset -LSE_i log2 e; a row with no key or past the end gets -inf, so its
    // P is 0 whatever the tile holds
    const float lse = qvalid ? a.lse[(int64_t)h * a.lse_sh + qrow] : -INFINITY;
    const float nl = lse == -INFINITY ? -INFINITY : -lse * kLog2e;
    // kernel 1: this lane's partial sum of P dP (lanes l and l ^ 32 cover the two halves
    // of each 64-key step); kernel 2: D_i of this lane's row as kernel 1 stored it
    float dlt = 0.f;
    if constexpr (MODE == 1) dlt = qvalid ? a.delta[(int64_t)h * a.lse_sh + qrow] : 0.f;
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

    const __bf16 *kh = (const __bf16 *)a.k + (int64_t)g * a.k_sh;
    const __bf16 *vh = (const __bf16 *)a.v + (int64_t)g * a.v_sh;
    const int e0 = cload(a.meta.row_ptr, qt), e1 = cload(a.meta.row_ptr, qt + 1);
    // steps (entry e, 64-key part sub); a part that starts past the last key is skipped
    auto kv_start = [&](int e, int sub) { return cload((const int32_t *)a.meta.entries, 4 * e) * a.bk_plan + sub * kStep; };
    auto advance = [&](int &e, int &sub) {
        ++sub;
        if (sub == nsub || kv_start(e, sub) >= a.sk) {
            ++e;
            sub = 0;
        }
    };
    auto rsrc_of = [&](const __bf16 *base, int32_t st, int kv0, int kend) {
        return make_rsrc(base + (int64_t)kv0 * st, extent<D>(min(kStep, kend - kv0), st));
    };
    int e = e0, sub = 0, buf = 0;
    if (e < e1) {
        const int kv0 = kv_start(e, 0);
        const int kend = min(kv0 + a.bk_plan, a.sk);
        tile_dma<D>(rsrc_of(kh, a.k_st, kv0, kend), a.k_st, smem + L::K0, wave, lane);
        tile_dma<D>(rsrc_of(vh, a.v_st, kv0, kend), a.v_st, smem + L::V0, wave, lane);
    }
    // (after the first tiles' loads are issued, so that the O rows arrive beside them)
    if constexpr (MODE == 2) {
        // this lane's half of the row's dims (16 ks + 8 hh .. + 7, as gf holds dO), then
        // the other half from lane l ^ 32
        float part = 0.f;
        if (qvalid) {
            const float *orow = a.o + (int64_t)qrow * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const f32x4 o0 = *(const f32x4 *)(orow + 16 * ks + 8 * hh);
                const f32x4 o1 = *(const f32x4 *)(orow + 16 * ks + 8 * hh + 4);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    part = __builtin_fmaf((float)gf[ks][x], o0[x], part);
                    part = __builtin_fmaf((float)gf[ks][4 + x], o1[x], part);
                }
            }
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(part), __float_as_int(part), false, false);
        dlt = __int_as_float(sw[0]) + __int_as_float(sw[1]);
        if (qvalid && hh == 0) a.delta[(int64_t)h * a.lse_sh + qrow] = dlt;
    }
    while (e < e1) {
        const i32x4 en = ((cptr_i32x4)a.meta.entries)[e];   // col, piece_begin, piece_count, tag
        const int kv0 = en[0] * a.bk_plan + sub * kStep;
        const int nk = min(kStep, min(en[0] * a.bk_plan + a.bk_plan, a.sk) - kv0);
        int ne = e, ns = sub;
        advance(ne, ns);
        const bool more = ne < e1;
        __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, 0u), rv = make_rsrc(vh, 0u);
        if (more) {
            const int nkv0 = kv_start(ne, ns);
            const int nkend = min(cload((const int32_t *)a.meta.entries, 4 * ne) * a.bk_plan + a.bk_plan, a.sk);
            rk = rsrc_of(kh, a.k_st, nkv0, nkend);
            rv = rsrc_of(vh, a.v_st, nkv0, nkend);
        }
        // mask (partial tiles and key tails): this lane's query row over the keys
        const int base = kv0 + 4 * hh;
        const bool masked_step = en[3] == BSFA_TILE_PARTIAL || nk < kStep;
        uint64_t m = ~0ull;
        if (masked_step) {
            m = range_bits(0, kv0 + nk - base);
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
        }
        __builtin_amdgcn_s_waitcnt(0);   // this step's tiles are in LDS (own loads) ...
        __syncthreads();                 // ... for every wave, and the other buffer is free
        char *cur = smem + buf * L::BUF, *nxt = smem + (buf ^ 1) * L::BUF;
        if constexpr (DELTA)
            delta_step<D>(nxt + L::K0, nxt + L::V0, cur + L::K0, cur + L::V0, more, rk, rv, a.k_st, a.v_st, wave,
                          lane, ad, qf, gf, m, masked_step, a.c, nl, dlt);
        else
            dq_step<D>(nxt + L::K0, nxt + L::V0, cur + L::K0, cur + L::V0, more, rk, rv, a.k_st, a.v_st, wave, lane,
                       ad, qf, gf, m, masked_step, a.c, nl, dlt, acc);
        e = ne;
        sub = ns;
        buf ^= 1;
    }
    if constexpr (DELTA) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(dlt), __float_as_int(dlt), false, false);
        const float dsum = __int_as_float(sw[0]) + __int_as_float(sw[1]);
        if (qvalid && hh == 0) a.delta[(int64_t)h * a.lse_sh + qrow] = dsum;
        return;
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

template <int D, bool DELTA>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq_kernel(const BwdArgs a)
{
    dq_body<D, DELTA ? 0 : 1>(a);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq_o32_kernel(const BwdArgs a)
{
    dq_body<D, 2>(a);
}

// ---------------------------------------------------------------------------
// kernel 3: dK, dV by key tile (one workgroup per (kv head, key tile), in the plan's
// launch order), 64-query steps over the CSR column for every query head of the key /
// value head; the Q, dO, LSE and D of step j + 1 load (LDS double buffer) while step j
// computes.  Two waves per SIMD: 8 waves per key tile; wave w owns keys 32 (w mod 4) ..
// + 31 and query half w div 4 of every 64-query step.  K and V stay in LDS for the whole
// workgroup and are read as MFMA operands (so a wave holds only its dK, dV partials and
// the step's scores); the two waves of a key block add their partials at the end.
// ---------------------------------------------------------------------------
// buffer ranges of one step's Q rows, dO rows, LSE and D
struct RowSrc {
    __amdgpu_buffer_rsrc_t q, g, l, d;
};

template <int D>
struct Kv2Tiles {
    static constexpr int K0 = 0, V0 = 2 * kStep * BCfg<D>::ROWB, T0 = 4 * kStep * BCfg<D>::ROWB;
    static constexpr int Q0 = 0, G0 = BCfg<D>::TILE_B, L0 = 2 * BCfg<D>::TILE_B, D0 = L0 + 4 * kStep;
    static constexpr int BUF = 2 * BCfg<D>::TILE_B + 1024, BYTES = T0 + 2 * BUF;
};

template <int D>
__device__ __forceinline__ void kv2_issue(char *__restrict__ dst, const RowSrc &r, int32_t q_st, int32_t do_st,
                                          int wave, int lane)
{
    using L = Kv2Tiles<D>;
    tile_dma<D, kStep, 8>(r.q, q_st, dst + L::Q0, wave, lane);
    tile_dma<D, kStep, 8>(r.g, do_st, dst + L::G0, wave, lane);
    if (wave == 6) __builtin_amdgcn_raw_ptr_buffer_load_lds(r.l, (lds_ptr)(dst + L::L0), 4, lane * 4, 0, 0, 0);
    if (wave == 7) __builtin_amdgcn_raw_ptr_buffer_load_lds(r.d, (lds_ptr)(dst + L::D0), 4, lane * 4, 0, 0, 0);
}

// One step of one wave on its 32 queries (half qh of the 64 in `cur`) against its 32 keys
// (block kb of the resident K, V): S = Q K^T - LSE / scale, dP = dO V^T - D, P = 2^(c S),
// dS = P dP, dV^T += dO^T P, dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void kv2_step(char *__restrict__ nxt, const char *__restrict__ cur,
                                         const char *__restrict__ kv, bool issue, const RowSrc &src, int32_t q_st,
                                         int32_t do_st, int wave, int lane, int kb, int qh, const Addr<D> &ad,
                                         uint32_t mw, bool masked_step, float c, float kneg,
                                         f32x16 (&dk)[BCfg<D>::DB], f32x16 (&dv)[BCfg<D>::DB])
{
    using C = BCfg<D>;
    using L = Kv2Tiles<D>;
    const int hh = lane >> 5;
    if (issue) kv2_issue<D>(nxt, src, q_st, do_st, wave, lane);
    // a block no pair of which is admitted adds nothing (every lane's mask word is empty)
    if (masked_step && __builtin_amdgcn_ballot_w64(mw != 0u) == 0ull) return;
    const char *qt_ = cur + L::Q0, *gt = cur + L::G0, *kt = kv + L::K0, *vt = kv + L::V0;
    const float *lse_s = (const float *)(cur + L::L0), *dlt_s = (const float *)(cur + L::D0);
    // accumulators start at -LSE / scale and -D of rows 32 qh + 8 g4 + 4 hh + t
    f32x16 s, dp;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 l4 = *(const f32x4 *)(lse_s + 32 * qh + 8 * g4 + 4 * hh);
        const f32x4 d4 = *(const f32x4 *)(dlt_s + 32 * qh + 8 * g4 + 4 * hh);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            s[4 * g4 + t] = l4[t] * kneg;
            dp[4 * g4 + t] = -d4[t];
        }
    }
    // score products: i -> S (even) / dP (odd), k-step i >> 1; A = query rows, B = key rows
    constexpr int N1 = 2 * C::KS;
    bf16x8 oa[kAheadKv + 1], ob[kAheadKv + 1];
    auto rd1 = [&](int i, bf16x8 &a_, bf16x8 &b_) {
        a_ = rd_row<D>((i & 1) ? gt : qt_, ad, qh, i >> 1);
        b_ = rd_row<D>((i & 1) ? vt : kt, ad, kb, i >> 1);
    };
    static_for<0, kAheadKv>([&](auto ic) { rd1(ic.value, oa[ic.value], ob[ic.value]); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N1>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + kAheadKv < N1)
            rd1(i + kAheadKv, oa[(i + kAheadKv) % (kAheadKv + 1)], ob[(i + kAheadKv) % (kAheadKv + 1)]);
        constexpr int r = i % (kAheadKv + 1);
        if constexpr (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[r], ob[r], dp, 0, 0, 0);
        else s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[r], ob[r], s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    });
    // gradient products: i -> dV (even) / dK (odd), block (i >> 1) % DB, k-step 2 qh + (i >> 1) / DB
    constexpr int N2 = 4 * C::DB;
    auto rd2 = [&](int i) { return rd_tr<D>((i & 1) ? qt_ : gt, ad, (i >> 1) % C::DB, 2 * qh + (i >> 1) / C::DB); };
    static_for<0, kAheadKv>([&](auto ic) { oa[ic.value] = rd2(ic.value); });
    __builtin_amdgcn_sched_barrier(0);
    if (masked_step) {
        const int32_t w = (int32_t)mw;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            const int32_t keep = (w << (31 - off)) >> 31;
            s[r] = __int_as_float((keep & __float_as_int(s[r])) | (~keep & __float_as_int(-INFINITY)));
        }
    }
    f32x8 tp[2], td[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[r] * c);
        tp[r >> 3][r & 7] = p;
        td[r >> 3][r & 7] = p * dp[r];
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        pb[k] = __builtin_convertvector(tp[k], bf16x8);
        dsb[k] = __builtin_convertvector(td[k], bf16x8);
    }
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, N2>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + kAheadKv < N2) oa[(i + kAheadKv) % (kAheadKv + 1)] = rd2(i + kAheadKv);
        constexpr int db = (i >> 1) % C::DB, kk = (i >> 1) / C::DB, r = i % (kAheadKv + 1);
        if constexpr (i & 1) dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[r], dsb[kk], dk[db], 0, 0, 0);
        else dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[r], pb[kk], dv[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int D>
__global__ void __launch_bounds__(2 * kThreads, 1) bwd_dkdv2_kernel(const BwdArgs a)
{
    using C = BCfg<D>;
    using L = Kv2Tiles<D>;
    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
    const int item = cload(a.meta.dkv_order, (int)blockIdx.x);
    const int g = item / a.n_kt, kt = item - g * a.n_kt, group = a.hq / a.hkv;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb = wave & 3, qh = wave >> 2;
    const int key = kt * a.bk_plan + 32 * kb + l32;
    const int nsub = kKernelBq / kStep;
    const Addr<D> ad = make_addr<D>(lane);

    // resident K and V rows of the key tile (rows past the end load as zeros)
    {
        const int k0 = kt * a.bk_plan, nk = min(2 * kStep, a.sk - k0);
        const __bf16 *kb_ = (const __bf16 *)a.k + (int64_t)k0 * a.k_st + (int64_t)g * a.k_sh;
        const __bf16 *vb_ = (const __bf16 *)a.v + (int64_t)k0 * a.v_st + (int64_t)g * a.v_sh;
        tile_dma<D, 2 * kStep, 8>(make_rsrc(kb_, extent<D>(nk, a.k_st)), a.k_st, smem + L::K0, wave, lane);
        tile_dma<D, 2 * kStep, 8>(make_rsrc(vb_, extent<D>(nk, a.v_st)), a.v_st, smem + L::V0, wave, lane);
    }
    f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }
    char *const tiles = smem + L::T0;
    const int t0 = cload(a.meta.t_ptr, kt), t1 = cload(a.meta.t_ptr, kt + 1);
    const int h_end = (g + 1) * group;
    auto q_start = [&](int t, int sub) { return cload(a.meta.t_list, 2 * t) * kKernelBq + sub * kStep; };
    auto advance = [&](int &h, int &t, int &sub) {
        ++sub;
        if (sub == nsub || q_start(t, sub) >= a.sq) {
            sub = 0;
            if (++t == t1) {
                t = t0;
                ++h;
            }
        }
    };
    auto sources = [&](int h, int q0) {
        const int nq = min(kStep, a.sq - q0);
        RowSrc r;
        r.q = make_rsrc((const __bf16 *)a.q + (int64_t)q0 * a.q_st + (int64_t)h * a.q_sh, extent<D>(nq, a.q_st));
        r.g = make_rsrc((const __bf16 *)a.dout + (int64_t)q0 * a.do_st + (int64_t)h * a.do_sh,
                        extent<D>(nq, a.do_st));
        r.l = make_rsrc(a.lse + (int64_t)h * a.lse_sh + q0, (uint32_t)nq * 4u);
        r.d = make_rsrc(a.delta + (int64_t)h * a.lse_sh + q0, (uint32_t)nq * 4u);
        return r;
    };
    int h = g * group, t = t0, sub = 0, buf = 0;
    if (t0 < t1) kv2_issue<D>(tiles, sources(h, q_start(t, 0)), a.q_st, a.do_st, wave, lane);
    else h = h_end;
    while (h < h_end) {
        const int e = cload(a.meta.t_list, 2 * t + 1);
        const i32x4 en = ((cptr_i32x4)a.meta.entries)[e];
        const int q0 = q_start(t, sub);
        int nh = h, ntt = t, ns = sub;
        advance(nh, ntt, ns);
        const bool more = nh < h_end;
        RowSrc src = sources(h, q0);   // placeholder when there is no next step
        if (more) src = sources(nh, q_start(ntt, ns));
        // mask of partial tiles: this lane's key over the wave's 32 query rows
        const bool masked_step = en[3] == BSFA_TILE_PARTIAL;
        uint32_t mw = ~0u;
        if (masked_step) {
            const int base = q0 + 4 * hh;
            uint64_t m = 0;
            for (int pi = 0; pi < en[2]; ++pi) {
                const i32x4 pc = ((cptr_i32x4)a.meta.pieces)[2 * (en[1] + pi)];
                const int diag = ((cptr_i32)a.meta.pieces)[8 * (en[1] + pi) + 4];
                if (key < pc[2] || key >= pc[3]) continue;
                m |= range_bits(max(pc[0], key - diag) - base, pc[1] - base);
            }
            mw = qh ? (uint32_t)(m >> 32) : (uint32_t)m;
        }
        __builtin_amdgcn_s_waitcnt(0);   // this step's rows (and the resident K, V) are in ...
        __syncthreads();                 // ... for every wave, and the other buffer is free
        kv2_step<D>(tiles + (buf ^ 1) * L::BUF, tiles + buf * L::BUF, smem, more, src, a.q_st, a.do_st, wave, lane,
                    kb, qh, ad, mw, masked_step, a.c, -1.f / a.scale, dk, dv);
        h = nh;
        t = ntt;
        sub = ns;
        buf ^= 1;
    }
    // the two waves of a key block add their partials: waves 4..7 pass theirs through LDS
    // (over the tiles; every load into them, the resident K and V included, has landed)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x4 *xch = (f32x4 *)smem + (size_t)kb * (2 * C::DB * 4) * 64 + lane;
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                xch[(2 * (4 * db + g4)) * 64] = f32x4{dk[db][4 * g4], dk[db][4 * g4 + 1], dk[db][4 * g4 + 2], dk[db][4 * g4 + 3]};
                xch[(2 * (4 * db + g4) + 1) * 64] = f32x4{dv[db][4 * g4], dv[db][4 * g4 + 1], dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]};
            }
    }
    __syncthreads();
    if (qh == 0 && key < a.sk) {
        float *ok = a.dk + ((int64_t)key * a.hkv + g) * D, *ov = a.dv + ((int64_t)key * a.hkv + g) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 pk = xch[(2 * (4 * db + g4)) * 64], pv = xch[(2 * (4 * db + g4) + 1) * 64];
                f32x4 wk, wv;
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    wk[t4] = a.scale * (dk[db][4 * g4 + t4] + pk[t4]);
                    wv[t4] = dv[db][4 * g4 + t4] + pv[t4];
                }
                *(f32x4 *)(ok + 32 * db + 8 * g4 + 4 * hh) = wk;
                *(f32x4 *)(ov + 32 * db + 8 * g4 + 4 * hh) = wv;
            }
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t stream)
{
    if (a.sq > 0 && a.o) {
        hipLaunchKernelGGL(bwd_dq_o32_kernel<D>, dim3(a.n_qt * a.hq), dim3(kThreads), 0, stream, a);
    } else if (a.sq > 0) {
        hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(a.n_qt * a.hq), dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3(a.n_qt * a.hq), dim3(kThreads), 0, stream, a);
    }
    if (a.sk > 0) hipLaunchKernelGGL(bwd_dkdv2_kernel<D>, dim3(a.n_kt * a.hkv), dim3(2 * kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs &a, int d, hipStream_t stream)
{
    return d == 128 ? launch_bwd_d<128>(a, stream) : launch_bwd_d<64>(a, stream);
}

}  // namespace bsfa
