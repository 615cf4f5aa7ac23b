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
//     the accumulator layout then gives every lane one query column and 16 keys,
//     so row statistics and the O^T accumulator columns live in the same lane, the
//     max needs one cross-half exchange (v_permlane32_swap) and the exponentials
//     feed the P.V product as its B operand without any shuffle.
//   * O^T = V^T P^T: V is staged into LDS transposed, each head-dim row holding
//     its 64 keys in the order the B operand uses them, so one 16-byte LDS read
//     is one A operand; 16-byte units are XOR-swizzled by ((d>>1)^(d>>2))&7, which
//     keeps both the transposing writes and the reads free of bank conflicts.  K
//     is staged row-major with a 16-byte pad per row.  Two buffers: the next
//     step's K/V loads are in flight while the current step is computed
//     (FlashAttention-T: double-buffered on-chip staging).
//   * K/V/Q are read with buffer loads: the per-step base and row count live in a
//     scalar resource, per-lane offsets are fixed for the whole kernel, and rows
//     past the end of the keys read as zero without a branch.
//   * Softmax in base 2 with a single FMA for scale and shift, and conditional
//     rescaling (FlashAttention-4 article: rescale only when needed): a row's
//     running max moves only when its tile max exceeds it by more than tau = 8.
//   * The per-element mask runs only on partial tiles and on the key tail
//     (MagiAttention news: flexible masks at small cost; cheap boundary
//     predicates): each lane turns the tile's slice pieces into key intervals for
//     its query row; one compare per score when the interval's start is behind
//     the step for every lane, two otherwise, a bit mask for several pieces.
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

constexpr int kThreads = 256;
constexpr int kBkS = kKernelBk;          // keys per inner step
constexpr float kTau = 8.0f;             // rescale threshold, log2 units
constexpr float kMFloor = -1.0e30f;      // finite start of the running max
constexpr float kLn2 = 0.693147180559945309f;
constexpr int32_t kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

template <int D>
struct Cfg {
    static constexpr int KP = D + 8;                  // K row pitch in LDS (bf16)
    static constexpr int VP = kBkS;                   // V^T row pitch (bf16): 8 units of 16 B
    static constexpr int NKC = D / 8;                 // 16-byte chunks per key row
    static constexpr int KCH = kBkS * NKC / kThreads; // K chunks per thread
    static constexpr int KS = D / 16;                 // k-steps of the score product
    static constexpr int DB = D / 32;                 // 32-row blocks of O^T
    static constexpr int VGROUPS = (kBkS / 4) * NKC;  // (4 keys x 8 dims) groups of V
    static constexpr int K_BYTES = kBkS * KP * 2;
    static constexpr int V_BYTES = D * VP * 2;
    static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    static_assert(KCH * kThreads == kBkS * NKC, "K staging must tile the threads");
    static_assert(VGROUPS <= kThreads, "one V group per thread at most");
    static_assert(BUF_BYTES % 16 == 0, "16-byte aligned buffers");
};

// 16-byte unit swizzle of V^T row d; f(d + 32) == f(d).
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 2)) & 7; }

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
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t *cptr_i32;
typedef const __attribute__((address_space(4))) i32x4 *cptr_i32x4;

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

template <int D>
struct Stage {
    u32x4 k[Cfg<D>::KCH];
    u32x4 v[4];
};

// Per-thread offsets, fixed for the whole kernel.
template <int D>
struct Lane {
    uint32_t koff[Cfg<D>::KCH];  // global byte offsets of this thread's K chunks (step-relative)
    uint32_t voff[4];            // global byte offsets of its 4 V rows (step-relative)
    uint32_t k_w;                // LDS byte address of its first K chunk
    uint32_t v_w[4];             // LDS byte addresses of its V^T writes, by swizzle class
    uint32_t k_r;                // LDS byte address of its K operand reads
    uint32_t v_r[4];             // LDS byte addresses of its V^T operand reads, by k-step
    bool vgroup;
};

template <int D>
__device__ __forceinline__ void load_step(const FwdArgs &a, const Step &st, int g,
                                          const Lane<D> &ln, Stage<D> &r)
{
    using C = Cfg<D>;
    const int n = max(0, min(kBkS, st.kv_end - st.kv0));
    const __bf16 *kb = (const __bf16 *)a.k + (int64_t)g * a.k_sh + (int64_t)st.kv0 * a.k_st;
    const __bf16 *vb = (const __bf16 *)a.v + (int64_t)g * a.v_sh + (int64_t)st.kv0 * a.v_st;
    // rows >= n are outside the resource and read as zero (they are masked anyway)
    const __amdgpu_buffer_rsrc_t rk = rsrc(kb, (uint32_t)n * (uint32_t)a.k_st * 2u);
    const __amdgpu_buffer_rsrc_t rv = rsrc(vb, (uint32_t)n * (uint32_t)a.v_st * 2u);
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) r.k[i] = ld16(rk, ln.koff[i]);
    if (ln.vgroup) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i] = ld16(rv, ln.voff[i]);
    }
}

template <int D, int BUF>
__device__ __forceinline__ void store_step(char *smem, const Lane<D> &ln, const Stage<D> &r)
{
    using C = Cfg<D>;
    char *base = smem + BUF * C::BUF_BYTES;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i)
        *(u32x4 *)(base + ln.k_w + i * (kThreads / C::NKC) * C::KP * 2) = r.k[i];
    if (ln.vgroup) {
        // transpose 4 keys x 8 dims into 8 head-dim rows of 4 keys; the swizzle class
        // of row 8*dc + e is ((e>>1) ^ (e>>2)) & 3 on top of the lane's own part
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t lo = __builtin_amdgcn_perm(r.v[1][e >> 1], r.v[0][e >> 1], sel);
            const uint32_t hi = __builtin_amdgcn_perm(r.v[3][e >> 1], r.v[2][e >> 1], sel);
            const int cls = ((e >> 1) ^ (e >> 2)) & 3;
            *(u32x2 *)(base + C::K_BYTES + ln.v_w[cls] + e * C::VP * 2) = u32x2{lo, hi};
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

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(const FwdArgs a)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int i0 = cload(a.meta.bin_ptr, (int)blockIdx.x), i1 = cload(a.meta.bin_ptr, (int)blockIdx.x + 1);
    const int group = a.hq / a.hkv;

    Lane<D> ln;
    {
        const int key0 = tid / C::NKC, dc = tid % C::NKC;
#pragma unroll
        for (int i = 0; i < C::KCH; ++i)
            ln.koff[i] = (uint32_t)((key0 + i * (kThreads / C::NKC)) * a.k_st * 2 + dc * 16);
        ln.k_w = (uint32_t)(key0 * C::KP * 2 + dc * 16);
        // V staging: key quads fastest in groups of 4 lanes, then head-dim chunks
        ln.vgroup = tid < C::VGROUPS;
        const int kq = (tid % 4) + 4 * (tid / (4 * C::NKC));
        const int vdc = (tid / 4) % C::NKC;
#pragma unroll
        for (int i = 0; i < 4; ++i) ln.voff[i] = (uint32_t)((kq * 4 + i) * a.v_st * 2 + vdc * 16);
        const int qi = kq % 4;
        const int unit = 2 * (kq / 4) + (qi & 1), half = qi >> 1;
        const int gdc = ((4 * vdc) ^ (2 * vdc)) & 7;
#pragma unroll
        for (int x = 0; x < 4; ++x)
            ln.v_w[x] = (uint32_t)(8 * vdc * C::VP * 2 + ((unit ^ gdc ^ x) * 16) + half * 8);
        ln.k_r = (uint32_t)(l32 * C::KP * 2 + 16 * hh);
        const int sw = vt_swz(l32);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            ln.v_r[ks] = (uint32_t)(C::K_BYTES + l32 * C::VP * 2 + (((2 * ks + hh) ^ sw) * 16));
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
        f32x16 oacc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
        float m_run = kMFloor, l_run = 0.f, lb_run = 0.f;  // max, fp32 sum, bf16-weight sum

        const int e0 = cload(a.meta.row_ptr, qt), e1 = cload(a.meta.row_ptr, qt + 1);
        if (e0 < e1) {
            const int spe = a.bk_plan / kBkS;   // steps per CSR entry
            Stage<D> stage;
            int e = e0, s = 0;                  // cursor: entry, step within it
            Step cur = make_step(a, e, 0);
            load_step<D>(a, cur, g, ln, stage);
            store_step<D, 0>(smem, ln, stage);
            __syncthreads();

            // One step on buffer BUF; returns false after the last step.
            auto run_step = [&](auto buf_tag) -> bool {
                constexpr int BUF = decltype(buf_tag)::value;
                // advance the cursor and put the next step's loads in flight
                int en = e, sn = s + 1;
                if (sn == spe) {
                    en = e + 1;
                    sn = 0;
                }
                const bool has_next = en < e1;
                Step nxt = cur;
                if (has_next) {
                    nxt = make_step(a, en, sn);
                    load_step<D>(a, nxt, g, ln, stage);
                }

                const char *sb = smem + BUF * C::BUF_BYTES;
                // ---- S^T = K Q^T: 64 keys x 32 queries as two interleaved 32x32 chains
                f32x16 sacc[2];
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const bf16x8 ka = *(const bf16x8 *)(sb + ln.k_r + kb * 32 * C::KP * 2 + ks * 32);
                        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            ka, qf[ks], ks == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
                    }
                }

                // ---- mask: partial tiles and the key tail only
                if (cur.partial || cur.kv_end - cur.kv0 < kBkS) apply_mask(a, cur, qrow, hh, sacc);

                // ---- online softmax, base 2, conditional rescale
                float mx = sacc[0][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
                mx = wave_cross_half_max(mx) * a.c;   // tile max of t = c * s (c > 0)
                // Each row moves its max only when its own tile max exceeds it by more
                // than tau; other rows keep m and get alpha = 2^0 = 1 exactly, so a row's
                // result never depends on the scores of another row.
                const bool need = mx > m_run + kTau;
                if (__builtin_amdgcn_ballot_w64(need) != 0) {
                    const float m_new = need ? fmaxf(m_run, mx) : m_run;
                    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                    l_run *= alpha;
                    lb_run *= alpha;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
                    m_run = m_new;
                }
                bf16x8 pb[4];
                float e0s = 0.f, e1s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x8 pf;
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const float p = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(sacc[j >> 1][(j & 1) * 8 + r], a.c, -m_run));
                        if (r & 1) e1s += p; else e0s += p;
                        pf[r] = p;
                    }
                    pb[j] = __builtin_convertvector(pf, bf16x8);   // v_cvt_pk_bf16_f32 x 4
                }
                l_run += e0s + e1s;
                // O's normaliser sums the same bf16 weights that multiply V, so O is an
                // exact weighted average of the rounded weights (in a peaked row the
                // dominant weight's rounding cancels); v_dot2 adds two weights at once.
                // The LSE keeps the fp32 sum above.
                {
                    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int t = 0; t < 4; t += 2) {
                            s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[j][2 * t], pb[j][2 * t + 1]}, ones, s0, false);
                            s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[j][2 * t + 2], pb[j][2 * t + 3]}, ones, s1, false);
                        }
                    lb_run += s0 + s1;
                }

                // ---- O^T += V^T P^T: A = V^T rows (head dims, one 16-byte read), B = P^T
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const bf16x8 va = *(const bf16x8 *)(sb + ln.v_r[ks] + db * 32 * C::VP * 2);
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], oacc[db], 0, 0, 0);
                    }

                if (has_next) store_step<D, BUF ^ 1>(smem, ln, stage);
                __syncthreads();
                e = en;
                s = sn;
                cur = nxt;
                return has_next;
            };
            while (run_step(std::integral_constant<int, 0>{}) &&
                   run_step(std::integral_constant<int, 1>{})) {
            }
        }

        // ---- epilogue: O = O^T columns / (sum of bf16 weights), LSE = ln2 * (m + log2 l)
        const float l_tot = wave_cross_half_sum(l_run);
        const float lb_tot = wave_cross_half_sum(lb_run);
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
                    for (int r = 0; r < 4; ++r) w[r] = (__bf16)(oacc[db][g4 * 4 + r] * inv);
                    *(bf16x4 *)(op + db * 32 + 8 * g4 + 4 * hh) = w;
                }
            if (hh == 0)
                a.lse[(int64_t)h * a.lse_sh + qrow] = any ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
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
