// Masked flash-attention forward for gfx950 (MI355X), driven by a tile CSR and a
// persistent schedule.
//
// What is computed (FlashAttention-T blog, FlashAttention lineage paragraph: tiles
// plus an incremental softmax kept on chip give the exact softmax; UltraAttn blog
// 3.2: the running (max, normaliser, rescaled sum) summary):
//   for every query row i of a work item and every admitted key j,
//   O_i = sum_j 2^(t_ij - m_i) v_j / l_i with t_ij = scale*log2(e) * q_i.k_j,
//   m_i = max_j t_ij, l_i = sum_j 2^(t_ij - m_i), LSE_i = ln2 * (m_i + log2 l_i).
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
//   * O^T = V^T P^T: V is staged into LDS transposed (key-quads of each head-dim
//     row, 8-byte reads), K row-major; both tiles are padded against bank
//     conflicts and double-buffered, with the next tile's global loads in flight
//     while the current tile is computed (FlashAttention-T: double-buffered
//     on-chip staging).
//   * Softmax in base 2 with a single FMA for scale and shift, and conditional
//     rescaling (FlashAttention-4 article: rescale only when needed): the running
//     max moves only when some row's tile max exceeds it by more than tau = 8
//     (a factor 256 of headroom in fp32).
//   * The per-element mask runs only on partial tiles and on the key tail
//     (MagiAttention news: flexible masks at small cost; cheap boundary
//     predicates): each lane turns the tile's slice pieces into key intervals for
//     its query row and compares.
//   * A row with no admitted key ends with l = 0 and gets O = 0, LSE = -inf; the
//     running max starts at a finite floor so 2^(-inf - m) is exactly 0 and no NaN
//     can form (FlashAttention-T: a floor on the exponent).
#include "bsfa_internal.h"

namespace bsfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBkS = kKernelBk;          // keys per inner step
constexpr float kTau = 8.0f;             // rescale threshold, log2 units
constexpr float kMFloor = -1.0e30f;      // finite start of the running max
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
struct Cfg {
    static constexpr int KP = D + 8;            // K row pitch in LDS (bf16): +16 B per row
    static constexpr int VP = kBkS + 4;         // V^T row pitch (bf16): 34 dwords per head-dim row
    static constexpr int NKC = D / 8;           // 16-byte chunks per key row
    static constexpr int KCH = kBkS * NKC / kThreads;  // K chunks per thread
    static constexpr int KS = D / 16;           // k-steps of the score product
    static constexpr int DB = D / 32;           // 32-row blocks of O^T
    static constexpr int VGROUPS = (kBkS / 4) * NKC;  // (4 keys x 8 dims) groups of V
    static_assert(KCH * kThreads == kBkS * NKC, "K staging must tile the threads");
    static_assert(VGROUPS <= kThreads, "one V group per thread at most");
};

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

// One 64-key step: its key range and how to mask it.
struct Step {
    int32_t kv0, kv_end;       // keys [kv0, min(kv0 + 64, kv_end)) exist
    int32_t piece_begin, piece_count;
    bool partial;
};

__device__ __forceinline__ Step make_step(const FwdArgs &a, int e, int s)
{
    const Entry en = a.meta.entries[e];
    Step st;
    const int32_t c0 = en.col * a.bk_plan;
    st.kv0 = c0 + s * kBkS;
    st.kv_end = min(c0 + a.bk_plan, a.sk);
    st.piece_begin = en.piece_begin;
    st.piece_count = en.piece_count;
    st.partial = en.tag == BSFA_TILE_PARTIAL;
    return st;
}

__device__ __forceinline__ int steps_of(const FwdArgs &a, int e)
{
    const int32_t c0 = a.meta.entries[e].col * a.bk_plan;
    const int32_t keys = min(c0 + a.bk_plan, a.sk) - c0;
    return (keys + kBkS - 1) / kBkS;
}

template <int D>
struct Stage {
    u32x4 k[Cfg<D>::KCH];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_step(const FwdArgs &a, const Step &st, int g, int tid,
                                          Stage<D> &r)
{
    using C = Cfg<D>;
    const int n = min(kBkS, st.kv_end - st.kv0);
    const __bf16 *kb = (const __bf16 *)a.k + (int64_t)g * a.k_sh;
    const __bf16 *vb = (const __bf16 *)a.v + (int64_t)g * a.v_sh;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
        const int c = tid + kThreads * i;
        const int key = c / C::NKC, dc = c % C::NKC;
        r.k[i] = key < n ? *(const u32x4 *)(kb + (int64_t)(st.kv0 + key) * a.k_st + dc * 8)
                         : u32x4{0, 0, 0, 0};
    }
    if (tid < C::VGROUPS) {
        const int dc = tid % C::NKC, kq = tid / C::NKC;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kq * 4 + i;
            r.v[i] = key < n ? *(const u32x4 *)(vb + (int64_t)(st.kv0 + key) * a.v_st + dc * 8)
                             : u32x4{0, 0, 0, 0};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_step(__bf16 *sk, __bf16 *sv, int tid, const Stage<D> &r)
{
    using C = Cfg<D>;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
        const int c = tid + kThreads * i;
        const int key = c / C::NKC, dc = c % C::NKC;
        *(u32x4 *)(sk + key * C::KP + dc * 8) = r.k[i];
    }
    if (tid < C::VGROUPS) {
        const int dc = tid % C::NKC, kq = tid / C::NKC;
        // transpose 4 keys x 8 dims into 8 rows of 4 keys; quad index swizzled by
        // (row / 32) so the 16 lanes of a write phase hit distinct banks
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t lo = __builtin_amdgcn_perm(r.v[1][e >> 1], r.v[0][e >> 1], sel);
            const uint32_t hi = __builtin_amdgcn_perm(r.v[3][e >> 1], r.v[2][e >> 1], sel);
            const int d = dc * 8 + e;
            const int quad = kq ^ ((d >> 5) & 3);
            *(u32x2 *)(sv + d * C::VP + quad * 4) = u32x2{lo, hi};
        }
    }
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(const FwdArgs a)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) __bf16 s_k[2][kBkS * C::KP];
    __shared__ __attribute__((aligned(16))) __bf16 s_v[2][D * C::VP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int i0 = a.meta.bin_ptr[blockIdx.x], i1 = a.meta.bin_ptr[blockIdx.x + 1];
    const int group = a.hq / a.hkv;

    for (int it = i0; it < i1; ++it) {
        const int item = a.meta.bin_items[it];
        const int h = item / a.n_qt, qt = item - h * a.n_qt;
        const int g = h / group;
        const int qrow = qt * kKernelBq + wave * 32 + l32;
        const bool qvalid = qrow < a.sq;

        // Q operand (B of S^T = K Q^T): query qrow, dims 16*ks + 8*hh .. +7
        bf16x8 qf[C::KS];
        {
            const __bf16 *qp = (const __bf16 *)a.q + (int64_t)qrow * a.q_st + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                u32x4 w = qvalid ? *(const u32x4 *)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
                qf[ks] = __builtin_bit_cast(bf16x8, w);
            }
        }
        f32x16 oacc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
        float m_run = kMFloor, l_run = 0.f, lb_run = 0.f;  // max, fp32 sum, bf16-weight sum

        const int e0 = a.meta.row_ptr[qt], e1 = a.meta.row_ptr[qt + 1];
        if (e0 < e1) {
            Stage<D> stage;
            int e = e0, s = 0, buf = 0;
            int ns = steps_of(a, e);
            Step cur = make_step(a, e, 0);
            load_step<D>(a, cur, g, tid, stage);
            store_step<D>(s_k[0], s_v[0], tid, stage);
            __syncthreads();
            while (true) {
                // advance the cursor and put the next step's loads in flight
                int en = e, sn = s + 1, nsn = ns;
                if (sn >= ns) {
                    en = e + 1;
                    sn = 0;
                    if (en < e1) nsn = steps_of(a, en);
                }
                const bool has_next = en < e1;
                Step nxt;
                if (has_next) {
                    nxt = make_step(a, en, sn);
                    load_step<D>(a, nxt, g, tid, stage);
                }

                // ---- S^T = K Q^T for 64 keys x 32 queries (two 32x32 blocks)
                const __bf16 *sk = s_k[buf];
                const __bf16 *sv = s_v[buf];
                f32x16 sacc[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    sacc[kb] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < C::KS; ++ks) {
                        const bf16x8 ka = *(const bf16x8 *)(sk + (kb * 32 + l32) * C::KP + ks * 16 + 8 * hh);
                        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sacc[kb], 0, 0, 0);
                    }
                }

                // ---- mask: partial tiles and the key tail only
                const int kv_hi = min(cur.kv0 + kBkS, cur.kv_end);
                if (cur.partial || kv_hi - cur.kv0 < kBkS) {
                    const int base = cur.kv0 + 4 * hh;  // key of register r in block kb: base + kb*32 + 8*(r>>2) + (r&3)
                    uint32_t ok = 0;
                    if (!cur.partial) {
                        ok = 0xffffffffu;
                    } else {
                        for (int pi = 0; pi < cur.piece_count; ++pi) {
                            const Piece pc = a.meta.pieces[cur.piece_begin + pi];
                            const bool inq = qrow >= pc.q_lo && qrow < pc.q_hi;
                            const int lo = pc.k_lo - base;
                            const int hi = inq ? min(pc.k_hi, qrow + pc.diag + 1) - base : -1000000;
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                                    if (off >= lo && off < hi) ok |= 1u << (kb * 16 + r);
                                }
                        }
                    }
                    const int tail = kv_hi - base;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                            const bool keep = ((ok >> (kb * 16 + r)) & 1u) && off < tail;
                            sacc[kb][r] = keep ? sacc[kb][r] : -INFINITY;
                        }
                }

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
                float e0 = 0.f, e1 = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], a.c, -m_run));
                        if (r & 1) e1 += p; else e0 += p;
                        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
                    }
                l_run += e0 + e1;
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

                // ---- O^T += V^T P^T: A = V^T rows (head dims), B = P^T (from the score layout)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int quad = kb * 8 + half * 4 + hh;   // keys 4*quad .. +3, then +8 keys
#pragma unroll
                        for (int db = 0; db < C::DB; ++db) {
                            const int d = db * 32 + l32;
                            const int sw = (d >> 5) & 3;
                            const u32x2 lo = *(const u32x2 *)(sv + d * C::VP + ((quad) ^ sw) * 4);
                            const u32x2 hi = *(const u32x2 *)(sv + d * C::VP + ((quad + 2) ^ sw) * 4);
                            const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb * 2 + half], oacc[db], 0, 0, 0);
                        }
                    }

                if (has_next) store_step<D>(s_k[buf ^ 1], s_v[buf ^ 1], tid, stage);
                __syncthreads();
                if (!has_next) break;
                buf ^= 1;
                e = en;
                s = sn;
                ns = nsn;
                cur = nxt;
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
