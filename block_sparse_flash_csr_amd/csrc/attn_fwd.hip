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
//     persistent workgroup walks the units of its bin (min-heap greedy schedule); a
//     unit is an item over a range of its CSR row.  A row too costly for one bin is
//     split into parts (UltraAttn 3.2: key ranges merge exactly through their
//     summaries): a part writes its normalised fp32 O and LSE to a workspace slot and a
//     second kernel merges the parts.
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
//     loaded two steps ahead and V one step ahead; one barrier per step.  The step
//     body is straight-line, split into groups of one matrix product each (operands
//     read from LDS two products ahead, the vector work of the group beside it), and
//     its four LDS tiles are distinct restrict pointers, so no operand read waits for
//     the direct loads in flight into the other two tiles.
//   * Softmax in base 2 with a single FMA for scale and shift, and conditional
//     rescaling (FlashAttention-4 article: rescale only when needed): a row's running
//     max moves only when its tile max exceeds it by more than tau (8 unless set).  At head dim 64,
//     where the vector work binds, the tile max itself is skipped: a step's weights are
//     taken against the running max and checked afterwards (their sum over a lane's keys
//     at most 2^tau), with a recomputation only for the rare step that fails.
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
constexpr int kBkS = kKernelBk;          // keys per step
constexpr float kMFloor = -1.0e30f;      // finite start of the running max
constexpr float kLn2 = 0.693147180559945309f;
constexpr int32_t kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

// Head dim 64 runs the vector-bound form of the softmax step ("lazy max"): no tile max of
// the next step's scores; each step's weights are taken against the running max and only
// a lane whose weights exceed 2^tau (or overflowed) sends the wave through a recomputation
// with the true max.  At head dim 128 the extra branch costs more registers than the saved
// maxima are worth.
template <int D>
constexpr bool kLazyMax = D == 64;

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

// IEEE 754-2019 maximum (NaN-propagating): lowers to v_maximum3_f32 chains with no
// quieting of the matrix-core results that fmaxf would insert.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float wave_cross_half_max(float x)
{
    // lanes l and l ^ 32 hold the same query: swap halves and take the max
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return vmax(__int_as_float(r[0]), __int_as_float(r[1]));
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
// past the end of the keys (kv0 >= kv_end) is fully masked.  A partial step carries
// its tile's slice pieces [pbeg, pbeg + pcnt).
struct Step {
    int32_t kv0, kv_end, partial, pbeg, pcnt;
};

__device__ __forceinline__ Step make_step(const FwdArgs &a, const Entry &en, int s)
{
    Step st;
    const int32_t c0 = en.col * a.bk_plan;
    st.kv0 = c0 + s * kBkS;
    st.kv_end = min(c0 + a.bk_plan, a.sk);
    st.partial = en.tag == BSFA_TILE_PARTIAL ? 1 : 0;
    st.pbeg = en.piece_begin;
    st.pcnt = en.piece_count;
    return st;
}

// Entry and slice pieces fetched a step ahead with vector loads (the step's own wait
// for its K/V tiles covers them; a scalar load would have to be waited on at once).
__device__ __forceinline__ i32x4 vload16(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ Entry uniform_entry(const i32x4 v)
{
    Entry en;
    en.col = __builtin_amdgcn_readfirstlane(v[0]);
    en.piece_begin = __builtin_amdgcn_readfirstlane(v[1]);
    en.piece_count = __builtin_amdgcn_readfirstlane(v[2]);
    en.tag = __builtin_amdgcn_readfirstlane(v[3]);
    return en;
}

// Up to two pieces of a partial step held in registers: (q_lo, q_hi, k_lo, k_hi), diag.
struct PiecePair {
    i32x4 r0, r1;
    int32_t d0, d1;
};
constexpr int kPfPieces = 2;

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

// Buffer resource of one tile load (every operand wave-uniform, so it lives in SGPRs);
// n = 0 makes every lane out of range: the load then only writes zeros into LDS.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *src, int32_t st_elems, int n)
{
    const uint64_t addr = (uint64_t)src;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    // uniform first, so that the clamp and the product stay on the scalar unit
    const int32_t rows = max(__builtin_amdgcn_readfirstlane(n), 0);
    const uint32_t bytes = (uint32_t)rows * (uint32_t)__builtin_amdgcn_readfirstlane(st_elems) * 2u;
    return rsrc((const void *)(((uint64_t)hi << 32) | lo), bytes);
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

// S^T (64 keys x 32 queries) = K Q^T from an LDS K tile, as two interleaved 32x32
// chains (the first step's scores; later steps form theirs inside the pipeline).
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

// Mask of one step for this lane's query row as a bit set over the 64 key offsets
// from base = kv0 + 4*hh (bit o set: key base + o is admitted): the union of the
// tile's slice pieces, cut at the end of the keys.
__device__ __forceinline__ uint64_t range_bits(int lo, int hi)
{
    lo = max(lo, 0);
    hi = min(hi, 64);
    if (lo >= hi) return 0ull;
    const uint64_t upto_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
    return upto_hi & ~((1ull << lo) - 1ull);
}

// One score through the mask: bit off of w keeps it, else -inf.  At head dim 64, where
// the vector work binds, the bit is extracted sign-extended and a three-input bitwise
// select picks the score or -inf (two vector instructions, no compare through VCC and
// its wait state); at head dim 128 that form measured within noise, and the compiler's
// own compare-and-select stays.
template <int D>
__device__ __forceinline__ float masked(float x, int32_t w, int off)
{
    if constexpr (D == 64) {
        const int32_t keep = __builtin_amdgcn_sbfe(w, off, 1);
        // truth table 0xCA: keep ? x : -inf, bit by bit
        return __int_as_float(__builtin_amdgcn_bitop3_b32(keep, __float_as_int(x), __float_as_int(-INFINITY), 0xCA));
    } else {
        const int32_t keep = (w << (31 - off)) >> 31;
        return __int_as_float((keep & __float_as_int(x)) | (~keep & __float_as_int(-INFINITY)));
    }
}

__device__ __forceinline__ uint64_t piece_bits(int qrow, int base, int q_lo, int q_hi, int k_lo, int k_hi,
                                               int diag)
{
    if (qrow < q_lo || qrow >= q_hi) return 0ull;
    return range_bits(k_lo - base, min(k_hi, qrow + diag + 1) - base);
}

// Any number of pieces, read with scalar loads.
__device__ __forceinline__ uint64_t mask_bits(const FwdArgs &a, const Step &cur, int qrow, int hh)
{
    const int base = cur.kv0 + 4 * hh;
    const int tail = min(cur.kv0 + kBkS, cur.kv_end) - base;
    if (!cur.partial) return range_bits(0, tail);
    uint64_t m = 0;
    for (int pi = 0; pi < cur.pcnt; ++pi) {
        const Piece pc = cload(a.meta.pieces, cur.pbeg + pi);
        m |= piece_bits(qrow, base, pc.q_lo, pc.q_hi, pc.k_lo, pc.k_hi, pc.diag);
    }
    return m & range_bits(0, tail);
}

// At most kPfPieces pieces, already in registers.
__device__ __forceinline__ uint64_t mask_bits_pf(const Step &cur, const PiecePair &pp, int qrow, int hh)
{
    const int base = cur.kv0 + 4 * hh;
    const int tail = min(cur.kv0 + kBkS, cur.kv_end) - base;
    if (!cur.partial) return range_bits(0, tail);
    uint64_t m = piece_bits(qrow, base, pp.r0[0], pp.r0[1], pp.r0[2], pp.r0[3], pp.d0);
    if (cur.pcnt > 1) m |= piece_bits(qrow, base, pp.r1[0], pp.r1[1], pp.r1[2], pp.r1[3], pp.d1);
    return m & range_bits(0, tail);
}

// Rejected scores become -inf: bit off of the mask word selects between the score and
// -inf.  off(kb, r) = kb*32 + 8*(r>>2) + (r&3) is the offset of accumulator register r of
// block kb from base.
template <int D>
__device__ __forceinline__ void apply_bits(uint64_t m, f32x16 (&s)[2])
{
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int32_t w = (int32_t)(kb ? (uint32_t)(m >> 32) : (uint32_t)m);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[kb][r] = masked<D>(s[kb][r], w, 8 * (r >> 2) + (r & 3));
        }
    }
}

__device__ __forceinline__ bool needs_mask(const Step &st) { return st.partial || st.kv_end - st.kv0 < kBkS; }

// Group q of a running max over elements 0..14 of one score block: 3 elements per group.
__device__ __forceinline__ float max3_step(const f32x16 &b, int q, float mx)
{
    const float t = vmax(vmax(b[3 * q], b[3 * q + 1]), b[3 * q + 2]);
    return q == 0 ? t : vmax(mx, t);
}

// Tile max of t = c * s for this lane's query (c > 0).
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2], float c)
{
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = vmax(mx, s[kb][r]);
    return wave_cross_half_max(mx) * c;
}

// Per-item running state of one wave (32 query rows).
template <int D>
struct Acc {
    f32x16 o[Cfg<D>::DB];
    float m, l, lb;   // running max, fp32 weight sum (LSE), bf16-weight sum (O's normaliser)
    float tau, rsum;  // rescale threshold (log2 units) and 2^tau (the lazy max's bound)
};

// Conditional rescale before step j (FlashAttention-4 article): each row moves its
// max only when its tile max exceeds it by more than tau; other rows keep m and get
// alpha = 2^0 = 1 exactly, so a row's result never depends on another row's scores.
template <int D>
__device__ __forceinline__ void rescale_for(float mx, Acc<D> &acc)
{
    const bool need = mx > acc.m + acc.tau;
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

// O^T += V^T P^T from an LDS V tile: A = V^T rows via transpose reads, B = P^T.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const char *vtile, const Lane<D> &ln, int i)
{
    using C = Cfg<D>;
    // PV product i: k-step i / DB (16 keys), O^T block i % DB (32 head dims)
    const char *p = vtile + ln.vr[i % C::DB] + 16 * (i / C::DB) * C::ROWB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + 8 * C::ROWB));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// K operand of score product i: k-step i / 2 (16 head dims), key block i % 2.
template <int D>
__device__ __forceinline__ bf16x8 k_operand(const char *ktile, const Lane<D> &ln, int i)
{
    return *(const bf16x8 *)(ktile + ln.kr[i >> 1] + (i & 1) * 32 * Cfg<D>::ROWB);
}

// Global source of one step's K or V tile, with the number of keys that exist.
struct TileSrc {
    const void *base;
    int32_t st, n;
};

// The LDS-touching body of one pipelined step, straight-line and software-pipelined:
//   phase 1: the 2*KS score products of step j+1 (K operand read two products ahead)
//            with the exponentials of step j spread between them;
//   phase 2: the 4*DB products P_j V_j (V^T operand read two products ahead) with the
//            bf16 weight sums and the raw (unmasked) row max of step j+1 between them.
// The four LDS tiles are separate restrict pointers: the direct loads into k_dst/v_dst
// never overlap the reads of k_src/v_src, so no read waits for the loads in flight.
template <int D>
__device__ __forceinline__ void step_body(char *__restrict__ k_dst, char *__restrict__ v_dst,
                                          const char *__restrict__ k_src, const char *__restrict__ v_src,
                                          const TileSrc &kld, bool do_k, const TileSrc &vld, bool do_v,
                                          const Lane<D> &ln, int wave, const bf16x8 (&qf)[Cfg<D>::KS],
                                          const f32x16 (&cur)[2], float c, Acc<D> &acc, f32x16 (&nxt)[2],
                                          float &mx_raw)
{
    using C = Cfg<D>;
    constexpr int NS = 2 * C::KS;   // score products
    constexpr int NP = 4 * C::DB;   // PV products
    constexpr int EPG = 32 / NS;    // exponentials per score product
    constexpr int DPG = 16 / NP;    // dot2 sums per PV product
    static_assert(EPG * NS == 32 && DPG * NP == 16 && EPG % 2 == 0, "even split of the vector work");

    // The 2*NLD direct loads of K_{j+2} and V_{j+1} go one per score product below (a
    // burst of them right after the barrier stalls the issue of the products); a tile
    // that is not needed gets an empty resource.
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kld.base, kld.st, do_k ? kld.n : 0);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vld.base, vld.st, do_v ? vld.n : 0);
    static_assert(2 * C::NLD <= NS, "one load per score product");

    const float nm = -acc.m;
    bf16x8 pb[4];
    f32x8 pf;
    float e0, e1;
    bf16x8 kop[3], vop[3];
    kop[0] = k_operand<D>(k_src, ln, 0);
    kop[1] = k_operand<D>(k_src, ln, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        if (i + 2 < NS) kop[(i + 2) % 3] = k_operand<D>(k_src, ln, i + 2);
        else vop[i + 2 - NS] = v_operand<D>(v_src, ln, i + 2 - NS);
        if (i < C::NLD)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(k_dst + (wave * C::NLD + i) * 1024), 16,
                                                     (int)ln.kg[i], 0, 0, 0);
        else if (i < 2 * C::NLD)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(v_dst + (wave * C::NLD + i - C::NLD) * 1024), 16,
                                                     (int)ln.vg[i - C::NLD], 0, 0, 0);
        const int kb = i & 1;
        nxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i % 3], qf[i >> 1], i < 2 ? f32x16{} : nxt[kb],
                                                          0, 0, 0);
#pragma unroll
        for (int u = 0; u < EPG; ++u) {
            const int v = EPG * i + u, j = v >> 3, r = v & 7;   // weight v -> pb[j][r]
            pf[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[j >> 1][(j & 1) * 8 + r], c, nm));
            float &ex = (r & 1) ? e1 : e0;
            ex = v < 2 ? pf[r] : ex + pf[r];
            if (r == 7) pb[j] = __builtin_convertvector(pf, bf16x8);   // v_cvt_pk_bf16_f32 x 4
        }
        // keep the sums in this group (left alone they sink past the matrix products)
        asm volatile("" : "+v"(e0), "+v"(e1));
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kLazyMax<D>) {
        // Conditional rescale after the fact (FlashAttention-4 article: rescale only when
        // needed): the weights were taken against the running max; only when one of them
        // (conservatively: their sum over this lane's keys) exceeds 2^tau, or overflowed,
        // does the step take its true max, rescale the rows whose max moved by more than
        // tau and take its weights again.  Both halves of a query row see the same max.
        if (__builtin_amdgcn_ballot_w64(!(e0 + e1 <= acc.rsum)) != 0) {
            rescale_for<D>(tile_max(cur, c), acc);
            const float nm2 = -acc.m;
#pragma unroll
            for (int v = 0; v < 32; ++v) {
                const int j = v >> 3, r = v & 7;
                pf[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[j >> 1][(j & 1) * 8 + r], c, nm2));
                float &ex = (r & 1) ? e1 : e0;
                ex = v < 2 ? pf[r] : ex + pf[r];
                if (r == 7) pb[j] = __builtin_convertvector(pf, bf16x8);
            }
        }
    }
    acc.l += e0 + e1;

    // Phase 2 also takes the unmasked tile max of the new scores (block 0 once its
    // chain has finished, block 1 later).
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float s0 = 0.f, s1 = 0.f, mx0 = 0.f, mx1 = 0.f;
    constexpr int MG = 5, B0 = 2, B1 = NP >= 8 + MG ? 8 : NP;   // B1 == NP: after the loop
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        if (i + 2 < NP) vop[(i + 2) % 3] = v_operand<D>(v_src, ln, i + 2);
        acc.o[i % C::DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[i % 3], pb[i / C::DB], acc.o[i % C::DB],
                                                                   0, 0, 0);
#pragma unroll
        for (int u = 0; u < DPG; ++u) {
            const int t = DPG * i + u, j = t >> 2, e = 2 * (t & 3);   // pair t -> pb[j][e, e+1]
            float &sx = (t & 1) ? s1 : s0;
            sx = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[j][e], pb[j][e + 1]}, ones, sx, false);
        }
        // max over 16 scores of one block: a 3-way max per group on groups B0.. (block 0)
        // and B1.. (block 1), the last element folded in at the end
        if constexpr (!kLazyMax<D>) {
            if (i >= B0 && i < B0 + MG) mx0 = max3_step(nxt[0], i - B0, mx0);
            if (i >= B1 && i < B1 + MG) mx1 = max3_step(nxt[1], i - B1, mx1);
        }
        asm volatile("" : "+v"(s0), "+v"(s1), "+v"(mx0), "+v"(mx1));
        __builtin_amdgcn_sched_barrier(0);
    }
    acc.lb += s0 + s1;
    if constexpr (kLazyMax<D>) {
        mx_raw = 0.f;   // not used
    } else {
        if (B1 == NP)
#pragma unroll
            for (int q = 0; q < MG; ++q) mx1 = max3_step(nxt[1], q, mx1);
        mx_raw = vmax(vmax(mx0, nxt[0][15]), vmax(mx1, nxt[1][15]));
    }
}

// The kernel body; OUT_F32 selects the type of O (bf16, or the fp32 value it is rounded
// from).
template <int D, bool OUT_F32>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs &a)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_B];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform within a wave
    const int l32 = lane & 31, hh = lane >> 5;
    const int i0 = cload(a.meta.bin_ptr, (int)blockIdx.x), i1 = cload(a.meta.bin_ptr, (int)blockIdx.x + 1);
    const int group = a.hq / a.hkv;
    const float c = a.c;
    const __amdgpu_buffer_rsrc_t r_ent = rsrc(a.meta.entries, (uint32_t)a.n_entries * 16u);
    const __amdgpu_buffer_rsrc_t r_pc = rsrc(a.meta.pieces, (uint32_t)a.n_pieces * 32u);

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
        // unit: (item, entry range of its row, partial slot or -1)
        const i32x4 un = ((cptr_i32x4)a.meta.units)[cload(a.meta.bin_items, it)];
        const int item = un[0], slot = un[3];
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
            const uint32_t qbytes = __builtin_amdgcn_readfirstlane((uint32_t)rows * (uint32_t)a.q_st * 2u);
            const __amdgpu_buffer_rsrc_t rq = rsrc(qb, qbytes);
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
        acc.tau = a.tau;
        acc.rsum = a.rsum;

        const int e0 = un[1], e1 = un[2];
        const int spe = a.bk_plan / kBkS;     // steps per CSR entry
        const int n = (e1 - e0) * spe;        // steps of this item
        if (n > 0) {
            // Step cursor (entry ce, sub-step cs) of the next step to create, and that
            // entry prefetched into registers.
            int ce = e0, cs = 0;
            auto advance = [&]() {
                if (++cs == spe) {
                    cs = 0;
                    ++ce;
                }
            };
            const Step st0 = make_step(a, cload(a.meta.entries, ce), cs);
            advance();
            const Step st1 = n > 1 ? make_step(a, cload(a.meta.entries, ce), cs) : st0;
            if (n > 1) advance();
            i32x4 en_pf = vload16(r_ent, ce * 16);   // out of range reads as zeros
            // pieces of the step whose mask is built next (st1 first)
            PiecePair pp;
            auto fetch_pieces = [&](const Step &st) {
                if (st.partial && st.pcnt <= kPfPieces) {
                    pp.r0 = vload16(r_pc, st.pbeg * 32);
                    pp.d0 = vload16(r_pc, st.pbeg * 32 + 16)[0];
                    if (st.pcnt > 1) {
                        pp.r1 = vload16(r_pc, st.pbeg * 32 + 32);
                        pp.d1 = vload16(r_pc, st.pbeg * 32 + 48)[0];
                    }
                }
            };
            fetch_pieces(st1);
            // prologue: K0, V0 and K1 into LDS; S0 and its max
            load_k<D>(a, st0, g, ln, smem + C::K_OFF0, wave);
            load_v<D>(a, st0, g, ln, smem + C::V_OFF0, wave);
            if (n > 1) load_k<D>(a, st1, g, ln, smem + C::K_OFF1, wave);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            f32x16 sA[2], sB[2];
            scores<D>(smem + C::K_OFF0, ln, qf, sA);
            if (needs_mask(st0)) apply_bits<D>(mask_bits(a, st0, qrow, hh), sA);
            float mxA = tile_max(sA, c), mxB = 0.f;
            acc.m = fmaxf(acc.m, mxA);   // O, l are still zero: start at the first tile's max

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
                // step j+1's mask from the pieces fetched last step, before they are replaced
                const bool m1 = has1 && needs_mask(sj1);
                uint64_t bits = 0;
                if (m1) bits = sj1.pcnt <= kPfPieces ? mask_bits_pf(sj1, pp, qrow, hh) : mask_bits(a, sj1, qrow, hh);
                Step sj2 = sj1;
                if (has2) {
                    sj2 = make_step(a, uniform_entry(en_pf), cs);
                    advance();
                    if (cs == 0 && ce < e1) en_pf = vload16(r_ent, ce * 16);
                    fetch_pieces(sj2);
                }
                const TileSrc kld{(const __bf16 *)a.k + (int64_t)g * a.k_sh + (int64_t)sj2.kv0 * a.k_st, a.k_st,
                                  min(kBkS, sj2.kv_end - sj2.kv0)};
                const TileSrc vld{(const __bf16 *)a.v + (int64_t)g * a.v_sh + (int64_t)sj1.kv0 * a.v_st, a.v_st,
                                  min(kBkS, sj1.kv_end - sj1.kv0)};
                if constexpr (!kLazyMax<D>) rescale_for<D>(mx_cur, acc);   // needs only step j's tile max
                __builtin_amdgcn_sched_barrier(0);
                // The score products run unconditionally so the block stays straight-line;
                // on the last step they read a stale (valid) tile and are discarded.
                // One body for every step (two variants of it would not fit the register
                // budget): a masked step applies its mask after the body and takes the
                // max again.
                float mx_raw;
                step_body<D>(smem + K_FREE, smem + V_NEXT, smem + K_NEXT, smem + V_CUR, kld, has2, vld, has1, ln,
                             wave, qf, cur, c, acc, nxt, mx_raw);
                if constexpr (kLazyMax<D>) {
                    if (m1) apply_bits<D>(bits, nxt);   // the maxima are taken only when needed
                } else if (m1) {
                    apply_bits<D>(bits, nxt);
                    mx_nxt = tile_max(nxt, c);
                } else if (has1) {
                    mx_nxt = wave_cross_half_max(mx_raw) * c;
                }
                return sj2;
            };

            Step sj1 = st1;
            for (int j = 0; j < n; j += 2) {
                sj1 = step(std::integral_constant<int, 0>{}, sA, mxA, sB, mxB, sj1, j);
                if (j + 1 >= n) break;
                sj1 = step(std::integral_constant<int, 1>{}, sB, mxB, sA, mxA, sj1, j + 1);
            }
            // the last steps' direct loads (zero fills of unused tiles included) have landed
            // and every wave is done with the LDS tiles before they are reused
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }

        // ---- epilogue: O = O^T columns / (sum of bf16 weights), LSE = ln2 * (m + log2 l).
        // A lane holds 4-value pieces of its query's row; the wave stages its 32 rows in
        // LDS (the K tiles' space, free after the last step) and writes whole rows, 16 B
        // per lane.  Staging swizzle (conflict-free writes and reads): 16-byte chunk c of
        // row q at c ^ ((q >> ESH) mod NCH), its 8-byte halves swapped on rows 16..31.
        const float l_tot = wave_cross_half_sum(acc.l);
        const float lb_tot = wave_cross_half_sum(acc.lb);
        const bool any = l_tot > 0.f;
        const float inv = any ? 1.0f / lb_tot : 0.f;
        const float lse_v = any ? (acc.m + __log2f(l_tot)) * kLn2 : -INFINITY;
        if (slot >= 0) {
            // one part of a split row: normalised fp32 O and its LSE into the workspace
            // slot (rows past the end included; the merge skips them)
            float *ws = a.ws + (size_t)slot * (kKernelBq * (D + 1));
            const int r = wave * 32 + l32;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    f32x4 w;
#pragma unroll
                    for (int t = 0; t < 4; ++t) w[t] = acc.o[db][g4 * 4 + t] * inv;
                    *(f32x4 *)(ws + (size_t)r * D + db * 32 + 8 * g4 + 4 * hh) = w;
                }
            if (hh == 0) ws[kKernelBq * D + r] = lse_v;
            continue;
        }
        if constexpr (OUT_F32) {
            // fp32 O: the same products the bf16 output is rounded from, stored straight
            // from the lane's registers (4 head dims of its query row per store)
            if (qvalid) {
                float *orow = (float *)a.o + (int64_t)qrow * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        f32x4 w;
#pragma unroll
                        for (int t = 0; t < 4; ++t) w[t] = acc.o[db][g4 * 4 + t] * inv;
                        *(f32x4 *)(orow + db * 32 + 8 * g4 + 4 * hh) = w;
                    }
            }
        } else {
            constexpr int ESH = D == 128 ? 0 : 1;
            constexpr int RPI = 1024 / C::ROWB;   // rows per 16-byte-per-lane read
            char *stage = smem + wave * 32 * C::ROWB;
            const int qsw = (l32 >> ESH) & (C::NCH - 1), hsw = hh ^ ((l32 >> 4) & 1);
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    bf16x4 w;
#pragma unroll
                    for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc.o[db][g4 * 4 + r] * inv);
                    *(bf16x4 *)(stage + l32 * C::ROWB + ((4 * db + g4) ^ qsw) * 16 + hsw * 8) = w;
                }
            const int cc = lane % C::NCH;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int row = RPI * k + lane / C::NCH;
                const u32x4 v = *(const u32x4 *)(stage + row * C::ROWB + (cc ^ ((row >> ESH) & (C::NCH - 1))) * 16);
                if (qrow0 + row < a.sq)
                    *(u32x4 *)((__bf16 *)a.o + (int64_t)(qrow0 + row) * a.o_st + (int64_t)h * a.o_sh + cc * 8) =
                        ((RPI * k) >> 4) & 1 ? u32x4{v[2], v[3], v[0], v[1]} : v;
            }
            __syncthreads();   // every wave has read its rows before the next item's loads
        }
        if (qvalid && hh == 0) a.lse[(int64_t)h * a.lse_sh + qrow] = lse_v;
    }
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(const FwdArgs a)
{
    attn_fwd_body<D, false>(a);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_o32_kernel(const FwdArgs a)
{
    attn_fwd_body<D, true>(a);
}

}  // namespace

// Static workspace for the split rows' partial results of bsfa_attn_fwd_noalloc (callers
// that cannot allocate device memory).  One copy per GPU, held until the process ends;
// every call on a GPU shares it (overlapping calls on one GPU race), and it keeps the
// last call's contents: each part writes all of its slot before the merge reads it, so
// nothing needs clearing.  Host code uses the per-device address from
// hipGetSymbolAddress, never the array's name (a host-side stand-in).
static __device__ __align__(256) float scratch[kStaticWorkspaceBytes / sizeof(float)];

hipError_t static_workspace(float **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        // once per device, with that device current (it is: the caller's)
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = (float *)p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_attn_fwd(const FwdArgs &a, int d, hipStream_t stream)
{
    if (a.n_bins <= 0) return hipSuccess;
    if (a.o_f32) {
        if (d == 128)
            hipLaunchKernelGGL(attn_fwd_o32_kernel<128>, dim3(a.n_bins), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(attn_fwd_o32_kernel<64>, dim3(a.n_bins), dim3(kThreads), 0, stream, a);
    } else if (d == 128) {
        hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(a.n_bins), dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(a.n_bins), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace bsfa
