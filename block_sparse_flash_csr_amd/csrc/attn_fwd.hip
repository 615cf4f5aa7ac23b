// Masked flash-attention forward for gfx950 (MI355X), driven by a tile CSR and a
// persistent schedule.
//
// What is computed (FlashAttention-T blog, FlashAttention lineage paragraph: tiles
// plus an incremental softmax kept on chip give the exact softmax; UltraAttn blog
// 3.2: the running (max, normaliser, rescaled sum) summary):
//   for every query row i of a work item and every admitted key j,
//   O_i = sum_j w_ij v_j / sum_j w_ij with w_ij = bf16(2^(t_ij - m_i)),
//   t_ij = scale*log2(e) * q_i.k_j, m_i a running maximum, and
//   LSE_i = ln2 * (m_i + log2 sum_j 2^(t_ij - m_i)) summed in fp32.
//
// Design (own, for CDNA4; the pages' Hopper/Blackwell kernels are prior art):
//   * Work item = (query head, 128-query tile); 4 waves, 32 query rows each.  A
//     persistent workgroup walks the items of its bin (min-heap greedy schedule).
//   * The CSR row of the query tile lists the non-empty key tiles; each is run in
//     64-key steps.  Empty tiles never appear (UltraAttn 3.3: skip Empty blocks).
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     the accumulator layout gives every lane one query column and 16 keys, so row
//     statistics and the O^T accumulator columns live in the same lane, the max
//     needs one cross-half exchange (v_permlane32_swap) and the exponentials feed
//     O^T = V^T P^T as its B operand without any shuffle.
//   * K and V tiles go from HBM straight into LDS (buffer loads with the LDS
//     destination: no staging registers, no LDS store instructions).  Both stay
//     row-major with 16-byte chunks XOR-swizzled per row; the V^T operand is read
//     with ds_read_b64_tr_b16, which hands each lane 4 keys of one head-dim column.
//     All operand reads are free of bank conflicts.
//   * Software pipeline over 64-key steps (FlashAttention-4 article: softmax
//     overlapped with the matrix products; FlashAttention-T: tensor/vector overlap,
//     double-buffered staging): while the exponentials of step j run on the vector
//     ALU, the matrix cores already form the scores of step j+1; while P_j V_j runs,
//     the vector ALU sums step j's weights and takes step j+1's row maximum.  K is
//     loaded two steps ahead and V one step ahead; one barrier per step.
//   * Softmax in base 2 with a single FMA for scale and shift, and conditional
//     rescaling (FlashAttention-4 article: rescale only when needed): a row's running
//     max moves only when its tile max exceeds it by more than tau = 8.
//   * The per-element mask runs only on partial tiles and on the key tail
//     (MagiAttention news: flexible masks at small cost; cheap boundary predicates):
//     each lane turns the tile's slice pieces into key intervals for its query row.
//   * A row with no admitted key ends with l = 0 and gets O = 0, LSE = -inf; the
//     running max starts at a finite floor so 2^(-inf - m) is exactly 0 and no NaN
//     can form (FlashAttention-T: a floor on the exponent).
#include <climits>
#include <type_traits>

#include "bsfa_internal.h"

namespace bsfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t *cptr_i32;
typedef const __attribute__((address_space(4))) i32x4 *cptr_i32x4;
typedef __attribute__((address_space(3))) void *lds_ptr;
typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;

constexpr int kThreads = 256;
constexpr int kBkS = kKernelBk;          // keys per step
constexpr float kTau = 8.0f;             // rescale threshold, log2 units
constexpr float kMFloor = -1.0e30f;      // finite start of the running max
constexpr float kLn2 = 0.693147180559945309f;
constexpr int32_t kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

template <int D>
struct Cfg {
    static constexpr int NCH = D / 8;              // 16-byte chunks per K/V row
    static constexpr int ROWB = 2 * D;             // bytes per K/V row in LDS
    static constexpr int TILE_B = kBkS * ROWB;     // bytes per K or V tile
    static constexpr int NLD = TILE_B / 1024 / 4;  // direct loads per wave per tile (1 KB each)
    static constexpr int KS = D / 16;              // k-steps of the score product
    static constexpr int DB = D / 32;              // 32-row blocks of O^T
    static constexpr int SWS = D == 128 ? 0 : 1;   // K swizzle shift
    // LDS: K0 | K1 | V0 | V1
    static constexpr int K_OFF0 = 0, K_OFF1 = TILE_B, V_OFF0 = 2 * TILE_B, V_OFF1 = 3 * TILE_B;
    static constexpr int LDS_B = 4 * TILE_B;
    static_assert(NLD * 4 * 1024 == TILE_B, "a tile is a whole number of wave loads");
};

// 16-byte chunk c of K row r sits at chunk c ^ kswz(r); of V row r at c ^ vswz(r).
template <int D>
__device__ __forceinline__ int kswz(int r) { return (r >> Cfg<D>::SWS) & (Cfg<D>::NCH - 1); }
// The V swizzle keeps transpose reads conflict-free in 32-lane phases: the 4 rows a
// 16-lane group reads land in 4 different 4-chunk groups of banks.
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 2 * (r & 3); }

__device__ __forceinline__ float wave_cross_half_max(float x)
{
    // lanes l and l ^ 32 hold the same query: swap halves and take the max
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float wave_cross_half_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Plan metadata is read-only for the whole launch: read it through the constant
// address space so uniform reads become scalar loads.
__device__ __forceinline__ int32_t cload(const int32_t *p, int i) { return ((cptr_i32)p)[i]; }

__device__ __forceinline__ Entry cload(const Entry *p, int i)
{
    return __builtin_bit_cast(Entry, ((cptr_i32x4)p)[i]);
}

__device__ __forceinline__ Piece cload(const Piece *p, int i)
{
    const i32x4 lo = ((cptr_i32x4)p)[2 * i], hi = ((cptr_i32x4)p)[2 * i + 1];
    Piece pc;
    pc.q_lo = lo[0];
    pc.q_hi = lo[1];
    pc.k_lo = lo[2];
    pc.k_hi = lo[3];
    pc.diag = hi[0];
    pc.pad0 = pc.pad1 = pc.pad2 = 0;
    return pc;
}

// One 64-key step of a CSR entry: keys [kv0, min(kv0 + 64, kv_end)) exist.  A step
// past the end of the keys (kv0 >= kv_end) is fully masked.
struct Step {
    int32_t kv0, kv_end, entry, partial;
};

__device__ __forceinline__ Step make_step(const FwdArgs &a, int e, int s)
{
    const Entry en = cload(a.meta.entries, e);
    Step st;
    const int32_t c0 = en.col * a.bk_plan;
    st.kv0 = c0 + s * kBkS;
    st.kv_end = min(c0 + a.bk_plan, a.sk);
    st.entry = e;
    st.partial = en.tag == BSFA_TILE_PARTIAL ? 1 : 0;
    return st;
}

// Per-lane constants for the whole launch.
template <int D>
struct Lane {
    uint32_t kg[Cfg<D>::NLD];   // global byte offsets (step-relative) of this lane's K chunks
    uint32_t vg[Cfg<D>::NLD];   // same for V
    uint32_t kr[Cfg<D>::KS];    // LDS byte offsets of the K operand for each k-step (block 0)
    uint32_t vr[Cfg<D>::DB];    // LDS byte offsets of the V^T transpose reads for each block
};

// Direct loads of one 64-key K or V tile into LDS.  Wave w fills 1 KB blocks
// b = w*NLD + i; lane l of a block fills 16-byte slot 64*b + l.  Rows past n are
// outside the buffer resource and land as zeros.
template <int D>
__device__ __forceinline__ void load_tile(const void *src, int32_t st_elems, int n, const uint32_t *goff,
                                          char *lds_tile, int wave)
{
    using C = Cfg<D>;
    // every operand of the resource is wave-uniform; say so, so that it lives in SGPRs
    const uint64_t addr = (uint64_t)src;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)max(n, 0) * (uint32_t)st_elems * 2u);
    const __amdgpu_buffer_rsrc_t r = rsrc((const void *)(((uint64_t)hi << 32) | lo), bytes);
#pragma unroll
    for (int i = 0; i < C::NLD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_ptr)(lds_tile + (wave * C::NLD + i) * 1024), 16, (int)goff[i], 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void load_k(const FwdArgs &a, const Step &st, int g, const Lane<D> &ln,
                                       char *lds_tile, int wave)
{
    const __bf16 *base = (const __bf16 *)a.k + (int64_t)g * a.k_sh + (int64_t)st.kv0 * a.k_st;
    load_tile<D>(base, a.k_st, min(kBkS, st.kv_end - st.kv0), ln.kg, lds_tile, wave);
}

template <int D>
__device__ __forceinline__ void load_v(const FwdArgs &a, const Step &st, int g, const Lane<D> &ln,
                                       char *lds_tile, int wave)
{
    const __bf16 *base = (const __bf16 *)a.v + (int64_t)g * a.v_sh + (int64_t)st.kv0 * a.v_st;
    load_tile<D>(base, a.v_st, min(kBkS, st.kv_end - st.kv0), ln.vg, lds_tile, wave);
}

// S^T (64 keys x 32 queries) = K Q^T from an LDS K tile, as two interleaved 32x32 chains.
template <int D>
__device__ __forceinline__ void scores(const char *ktile, const Lane<D> &ln, const bf16x8 (&qf)[Cfg<D>::KS],
                                       f32x16 (&s)[2])
{
    using C = Cfg<D>;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 ka = *(const bf16x8 *)(ktile + ln.kr[ks] + kb * 32 * C::ROWB);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
        }
    }
}

// Scores -inf where the step's mask rejects them.  off(kb, r) = kb*32 + 8*(r>>2) + (r&3)
// is the key offset from base = kv0 + 4*hh of accumulator register r of block kb.
__device__ __forceinline__ void apply_mask(const FwdArgs &a, const Step &cur, int qrow, int hh,
                                           f32x16 (&sacc)[2])
{
    const int base = cur.kv0 + 4 * hh;
    const int kv_hi = min(cur.kv0 + kBkS, cur.kv_end);
    const int tail = kv_hi - base;
    const Entry en = cload(a.meta.entries, cur.entry);
    if (!cur.partial || en.piece_count == 1) {
        int lo = INT_MIN / 2, hi = tail;
        if (cur.partial) {
            const Piece pc = cload(a.meta.pieces, en.piece_begin);
            const bool inq = qrow >= pc.q_lo && qrow < pc.q_hi;
            lo = pc.k_lo - base;
            hi = inq ? min(min(pc.k_hi, qrow + pc.diag + 1) - base, tail) : INT_MIN / 2;
        }
        if (__builtin_amdgcn_ballot_w64(lo > 0) == 0) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                    sacc[kb][r] = off < hi ? sacc[kb][r] : -INFINITY;
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                    sacc[kb][r] = (off >= lo && off < hi) ? sacc[kb][r] : -INFINITY;
                }
        }
        return;
    }
    // several pieces: union of their intervals as a 64-bit mask over the offsets
    uint64_t m = 0;
    for (int pi = 0; pi < en.piece_count; ++pi) {
        const Piece pc = cload(a.meta.pieces, en.piece_begin + pi);
        if (qrow < pc.q_lo || qrow >= pc.q_hi) continue;
        const int lo = max(pc.k_lo - base, 0);
        const int hi = min(min(pc.k_hi, qrow + pc.diag + 1) - base, 64);
        if (lo >= hi) continue;
        const uint64_t upto_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
        m |= upto_hi & ~((1ull << lo) - 1ull);
    }
    if (tail < 64) m &= tail <= 0 ? 0ull : ((1ull << tail) - 1ull);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
            sacc[kb][r] = ((m >> off) & 1ull) ? sacc[kb][r] : -INFINITY;
        }
}

__device__ __forceinline__ bool needs_mask(const Step &st) { return st.partial || st.kv_end - st.kv0 < kBkS; }

// Tile max of t = c * s for this lane's query (c > 0).
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2], float c)
{
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return wave_cross_half_max(mx) * c;
}

// Per-item running state of one wave (32 query rows).
template <int D>
struct Acc {
    f32x16 o[Cfg<D>::DB];
    float m, l, lb;   // running max, fp32 weight sum (LSE), bf16-weight sum (O's normaliser)
};

// Conditional rescale before step j (FlashAttention-4 article): each row moves its
// max only when its tile max exceeds it by more than tau; other rows keep m and get
// alpha = 2^0 = 1 exactly, so a row's result never depends on another row's scores.
template <int D>
__device__ __forceinline__ void rescale_for(float mx, Acc<D> &acc)
{
    const bool need = mx > acc.m + kTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = need ? fmaxf(acc.m, mx) : acc.m;
        const float alpha = __builtin_amdgcn_exp2f(acc.m - m_new);
#pragma unroll
        for (int db = 0; db < Cfg<D>::DB; ++db) acc.o[db] *= alpha;
        acc.l *= alpha;
        acc.lb *= alpha;
        acc.m = m_new;
    }
}

// Exponentials of step j against the running max: bf16 weights and their fp32 sum.
__device__ __forceinline__ void softmax_weights(const f32x16 (&s)[2], float c, float m_run, bf16x8 (&pb)[4],
                                                float &psum)
{
    float e0 = 0.f, e1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x8 pf;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            pf[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j >> 1][(j & 1) * 8 + r], c, -m_run));
            if (r & 1) e1 += pf[r]; else e0 += pf[r];
        }
        pb[j] = __builtin_convertvector(pf, bf16x8);   // v_cvt_pk_bf16_f32 x 4
    }
    psum = e0 + e1;
}

// Sum of the bf16 weights (O's normaliser: O is then an exact weighted average of
// the rounded weights, so in a peaked row the dominant weight's rounding cancels);
// v_dot2 adds two weights at once.
__device__ __forceinline__ float bf16_sum(const bf16x8 (&pb)[4])
{
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < 8; t += 4) {
            s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[j][t], pb[j][t + 1]}, ones, s0, false);
            s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[j][t + 2], pb[j][t + 3]}, ones, s1, false);
        }
    return s0 + s1;
}

// O^T += V^T P^T from an LDS V tile: A = V^T rows via transpose reads, B = P^T.
template <int D>
__device__ __forceinline__ void pv(const char *vtile, const Lane<D> &ln, const bf16x8 (&pb)[4],
                                   f32x16 (&o)[Cfg<D>::DB])
{
    using C = Cfg<D>;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const char *p = vtile + ln.vr[db] + 16 * ks * C::ROWB;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + 8 * C::ROWB));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], o[db], 0, 0, 0);
        }
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(const FwdArgs a)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_B];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform within a wave
    const int l32 = lane & 31, hh = lane >> 5;
    const int i0 = cload(a.meta.bin_ptr, (int)blockIdx.x), i1 = cload(a.meta.bin_ptr, (int)blockIdx.x + 1);
    const int group = a.hq / a.hkv;
    const float c = a.c;

    Lane<D> ln;
    {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int p = 64 * (wave * C::NLD + i) + lane;      // 16-byte slot in the tile
            const int row = p / C::NCH, phys = p % C::NCH;
            ln.kg[i] = (uint32_t)(row * a.k_st * 2 + ((phys ^ kswz<D>(row)) * 16));
            ln.vg[i] = (uint32_t)(row * a.v_st * 2 + ((phys ^ vswz<D>(row)) * 16));
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            ln.kr[ks] = (uint32_t)(l32 * C::ROWB + (((2 * ks + hh) ^ kswz<D>(l32)) * 16));
        // transpose reads: lanes 4r..4r+3 of a 16-lane group read key row 4*hh + r,
        // 16 consecutive head dims starting at 32*db + 16*(group & 1)
        const int grp = lane >> 4, i16 = lane & 15, r = i16 >> 2, c4 = i16 & 3;
        const int row = 4 * hh + r;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const int chunk = 4 * db + 2 * (grp & 1) + (c4 >> 1);
            ln.vr[db] = (uint32_t)(row * C::ROWB + ((chunk ^ vswz<D>(row)) * 16) + (c4 & 1) * 8);
        }
    }

    for (int it = i0; it < i1; ++it) {
        const int item = cload(a.meta.bin_items, it);
        const int h = item / a.n_qt, qt = item - h * a.n_qt;
        const int g = h / group;
        const int qrow0 = qt * kKernelBq + wave * 32;
        const int qrow = qrow0 + l32;
        const bool qvalid = qrow < a.sq;

        // Q operand (B of S^T = K Q^T): query qrow, dims 16*ks + 8*hh .. +7; rows past
        // the end read as zero
        bf16x8 qf[C::KS];
        {
            const int rows = max(0, min(32, a.sq - qrow0));
            const __bf16 *qb = (const __bf16 *)a.q + (int64_t)qrow0 * a.q_st + (int64_t)h * a.q_sh;
            const __amdgpu_buffer_rsrc_t rq = rsrc(qb, (uint32_t)rows * (uint32_t)a.q_st * 2u);
            const uint32_t qo = (uint32_t)(l32 * a.q_st * 2 + 16 * hh);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(rq, qo + 32 * ks));
        }
        Acc<D> acc;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc.o[db] = f32x16{};
        acc.m = kMFloor;
        acc.l = 0.f;
        acc.lb = 0.f;

        const int e0 = cload(a.meta.row_ptr, qt), e1 = cload(a.meta.row_ptr, qt + 1);
        const int spe = a.bk_plan / kBkS;     // steps per CSR entry
        const int n = (e1 - e0) * spe;        // steps of this item
        if (n > 0) {
            // step cursor: entry / sub-step of the next step to load
            int ce = e0, cs = 0;
            auto next_step = [&]() {
                const Step st = make_step(a, ce, cs);
                if (++cs == spe) {
                    cs = 0;
                    ++ce;
                }
                return st;
            };
            const Step st0 = next_step();
            const Step st1 = n > 1 ? next_step() : st0;
            // prologue: K0, V0 and K1 into LDS; S0 and its max
            load_k<D>(a, st0, g, ln, smem + C::K_OFF0, wave);
            load_v<D>(a, st0, g, ln, smem + C::V_OFF0, wave);
            if (n > 1) load_k<D>(a, st1, g, ln, smem + C::K_OFF1, wave);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            f32x16 sA[2], sB[2];
            scores<D>(smem + C::K_OFF0, ln, qf, sA);
            if (needs_mask(st0)) apply_mask(a, st0, qrow, hh, sA);
            float mxA = tile_max(sA, c), mxB = 0.f;

            // Pipelined step j (LDS buffers by parity P = j & 1): cur = S_j, nxt = S_{j+1}.
            auto step = [&](auto par_tag, f32x16(&cur)[2], const float mx_cur, f32x16(&nxt)[2], float &mx_nxt,
                            const Step &sj1, int j) -> Step {
                constexpr int P = decltype(par_tag)::value;
                constexpr int K_NEXT = P ? C::K_OFF0 : C::K_OFF1;   // holds K_{j+1}
                constexpr int K_FREE = P ? C::K_OFF1 : C::K_OFF0;   // receives K_{j+2}
                constexpr int V_CUR = P ? C::V_OFF1 : C::V_OFF0;    // holds V_j
                constexpr int V_NEXT = P ? C::V_OFF0 : C::V_OFF1;   // receives V_{j+1}
                const bool has1 = j + 1 < n, has2 = j + 2 < n;
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();   // K_{j+1}, V_j in LDS; every wave is done with step j-1
                Step sj2 = sj1;
                if (has2) {
                    sj2 = next_step();
                    load_k<D>(a, sj2, g, ln, smem + K_FREE, wave);
                }
                if (has1) load_v<D>(a, sj1, g, ln, smem + V_NEXT, wave);

                // rescale first (needs only step j's tile max), then one branch-free block:
                // exponentials of step j with the scores of step j+1 on the matrix cores,
                // P_j V_j with the weight sums
                rescale_for<D>(mx_cur, acc);
                float psum;
                bf16x8 pb[4];
                softmax_weights(cur, c, acc.m, pb, psum);
                // Unconditional so that it shares the block with the exponentials; on the
                // last step it reads a stale (valid) tile and is discarded.
                scores<D>(smem + K_NEXT, ln, qf, nxt);
                pv<D>(smem + V_CUR, ln, pb, acc.o);
                acc.l += psum;
                acc.lb += bf16_sum(pb);
                // step j+1's mask and row max
                if (has1) {
                    if (needs_mask(sj1)) apply_mask(a, sj1, qrow, hh, nxt);
                    mx_nxt = tile_max(nxt, c);
                }
                return sj2;
            };

            Step sj1 = st1;
            for (int j = 0; j < n; j += 2) {
                sj1 = step(std::integral_constant<int, 0>{}, sA, mxA, sB, mxB, sj1, j);
                if (j + 1 >= n) break;
                sj1 = step(std::integral_constant<int, 1>{}, sB, mxB, sA, mxA, sj1, j + 1);
            }
            __syncthreads();   // every wave is done with the LDS tiles before the next item
        }

        // ---- epilogue: O = O^T columns / (sum of bf16 weights), LSE = ln2 * (m + log2 l)
        const float l_tot = wave_cross_half_sum(acc.l);
        const float lb_tot = wave_cross_half_sum(acc.lb);
        if (qvalid) {
            const bool any = l_tot > 0.f;
            const float inv = any ? 1.0f / lb_tot : 0.f;
            __bf16 *op = (__bf16 *)a.o + (int64_t)qrow * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    bf16x4 w;
#pragma unroll
                    for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc.o[db][g4 * 4 + r] * inv);
                    *(bf16x4 *)(op + db * 32 + 8 * g4 + 4 * hh) = w;
                }
            if (hh == 0)
                a.lse[(int64_t)h * a.lse_sh + qrow] = any ? (acc.m + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs &a, int d, hipStream_t stream)
{
    if (a.n_bins <= 0) return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(a.n_bins), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(a.n_bins), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace bsfa
