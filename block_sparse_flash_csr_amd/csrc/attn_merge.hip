// Merge of KV-split partial attention results (UltraAttn blog, 3.2: each key/value
// shard keeps a mergeable summary; to combine, take the common maximum, rescale
// every summary to it and add).  With the partial outputs stored normalised, as
// (O_t, LSE_t):
//   M = max_t LSE_t,  w_t = exp(LSE_t - M),  LSE = M + ln sum_t w_t,
//   O = sum_t (w_t / sum_t w_t) O_t;  every LSE_t = -inf  ->  O = 0, LSE = -inf.
//
// The kernel is a pure stream: every (token, head) row of every partial is read
// once and the result written once, so HBM bandwidth bounds it.  A workgroup
// owns rows (t0 .. t0+R-1, head h): the LSE reads of one partial are then one
// contiguous run, and each row of O is read as 16-byte pieces by D/8 adjacent
// lanes.  All n loads of a lane are issued before any arithmetic; the partials and
// the result are touched once, so they are read and written non-temporally (measured
// +16 % at 8 partials x 8192 tokens x 32 heads, to 5.9 TB/s).
#include "bsfa_internal.h"

namespace bsfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One lane: EPL head dims (16 bytes of a partial row) of one (token, head) row.
// IN32 / OUT32: the partials / the result are fp32 (else bf16).
template <int D, bool IN32, bool OUT32>
__device__ __forceinline__ void merge_body(const MergeArgs &a)
{
    constexpr int EPL = IN32 ? 4 : 8;        // head dims per lane (16-byte loads)
    constexpr int TPR = D / EPL;             // lanes per row
    constexpr int RPB = kThreads / TPR;      // rows per workgroup
    const int tid = threadIdx.x;
    // heads vary fastest across workgroups: the workgroups running together read whole
    // [heads, d] token rows of each partial, which are contiguous
    const int h = (int)(blockIdx.x % (unsigned)a.n_head);
    const int t = (int)(blockIdx.x / (unsigned)a.n_head) * RPB + tid / TPR;
    const int chunk = tid % TPR;
    if (t >= a.n_tok) return;

    float lse[BSFA_MERGE_MAX_PARTS];
    u32x4 ov[BSFA_MERGE_MAX_PARTS];
    const int64_t lse_off = (int64_t)h * a.lse_sh + t;
    const int64_t o_off = (int64_t)t * a.p_st + (int64_t)h * a.p_sh + chunk * EPL;
#pragma unroll
    for (int i = 0; i < BSFA_MERGE_MAX_PARTS; ++i) {
        if (i < a.n) {
            lse[i] = a.lse_parts[i][lse_off];
            const u32x4 *src = IN32 ? (const u32x4 *)((const float *)a.o_parts[i] + o_off)
                                    : (const u32x4 *)((const __bf16 *)a.o_parts[i] + o_off);
            ov[i] = __builtin_nontemporal_load(src);
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < BSFA_MERGE_MAX_PARTS; ++i)
        if (i < a.n) m = fmaxf(m, lse[i]);

    float acc[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
    float out_lse = -INFINITY;
    if (m != -INFINITY) {
        float w[BSFA_MERGE_MAX_PARTS];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < BSFA_MERGE_MAX_PARTS; ++i) {
            if (i < a.n) {
                w[i] = __builtin_amdgcn_exp2f((lse[i] - m) * kLog2e);
                sum += w[i];
            }
        }
        const float inv = 1.0f / sum;
#pragma unroll
        for (int i = 0; i < BSFA_MERGE_MAX_PARTS; ++i) {
            if (i < a.n) {
                const float wi = w[i] * inv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (IN32) {
                        acc[j] += wi * __uint_as_float(ov[i][j]);
                    } else {
                        acc[2 * j] += wi * bf16_lo(ov[i][j]);
                        acc[2 * j + 1] += wi * bf16_hi(ov[i][j]);
                    }
                }
            }
        }
        out_lse = m + __log2f(sum) * kLn2;
    }
    const int64_t r_off = (int64_t)t * a.o_st + (int64_t)h * a.o_sh + chunk * EPL;
    if constexpr (OUT32) {
#pragma unroll
        for (int j = 0; j < EPL; j += 4)
            __builtin_nontemporal_store(f32x4{acc[j], acc[j + 1], acc[j + 2], acc[j + 3]},
                                        (f32x4 *)((float *)a.o + r_off + j));
    } else {
        uint32_t res[EPL / 2];
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) {
            const __bf16 lo = (__bf16)acc[2 * j], hi = (__bf16)acc[2 * j + 1];
            res[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        if constexpr (EPL == 8)
            __builtin_nontemporal_store(u32x4{res[0], res[1], res[2], res[3]}, (u32x4 *)((__bf16 *)a.o + r_off));
        else
            __builtin_nontemporal_store(u32x2{res[0], res[1]}, (u32x2 *)((__bf16 *)a.o + r_off));
    }
    if (chunk == 0) a.lse[lse_off] = out_lse;
}

template <int D>
__global__ void __launch_bounds__(kThreads) attn_merge_kernel(const MergeArgs a)
{
    merge_body<D, false, false>(a);
}

template <int D, bool IN32, bool OUT32>
__global__ void __launch_bounds__(kThreads) attn_merge_typed_kernel(const MergeArgs a)
{
    merge_body<D, IN32, OUT32>(a);
}

}  // namespace

// Rows of the forward launch that were split into parts: the parts' normalised fp32
// (O_t, LSE_t) in the workspace merge the same way into the caller's O and LSE.  A
// workgroup takes RPB rows of one split row; a lane owns 4 head dims.
template <int D, bool OUT32>
__device__ __forceinline__ void split_merge_body(const SplitMergeArgs &a)
{
    constexpr int TPR = D / 4;               // lanes per row (4 floats each)
    constexpr int RPB = kThreads / TPR;      // rows per workgroup
    constexpr size_t kSlot = (size_t)kKernelBq * (D + 1);
    const int r = (int)blockIdx.y * RPB + (int)threadIdx.x / TPR;   // row within the tile
    const int c = ((int)threadIdx.x % TPR) * 4;
    const Split sp = a.splits[blockIdx.x];
    const int h = sp.item / a.n_qt, qt = sp.item - h * a.n_qt;
    const int row = qt * kKernelBq + r;
    if (r >= kKernelBq || row >= a.sq) return;
    const float *ws = a.ws + (size_t)sp.first * kSlot;
    float m = -INFINITY;
    for (int t = 0; t < sp.parts; ++t) m = fmaxf(m, ws[t * kSlot + kKernelBq * D + r]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse = -INFINITY;
    if (m != -INFINITY) {
        float sum = 0.f;
        for (int t = 0; t < sp.parts; ++t) {
            const float w = exp2f((ws[t * kSlot + kKernelBq * D + r] - m) * kLog2e);
            sum += w;
            o += w * *(const f32x4 *)(ws + t * kSlot + (size_t)r * D + c);
        }
        o *= 1.0f / sum;
        lse = m + __log2f(sum) * kLn2;
    }
    const int64_t r_off = (int64_t)row * a.o_st + (int64_t)h * a.o_sh + c;
    if constexpr (OUT32) {
        *(f32x4 *)((float *)a.o + r_off) = o;
    } else {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (__bf16)o[e];
        *(bf16x4 *)((__bf16 *)a.o + r_off) = ob;
    }
    if (c == 0) a.lse[(int64_t)h * a.lse_sh + row] = lse;
}

template <int D>
__global__ void __launch_bounds__(kThreads) split_merge_kernel(const SplitMergeArgs a)
{
    split_merge_body<D, false>(a);
}

template <int D>
__global__ void __launch_bounds__(kThreads) split_merge_o32_kernel(const SplitMergeArgs a)
{
    split_merge_body<D, true>(a);
}

hipError_t launch_split_merge(const SplitMergeArgs &a, int d, hipStream_t stream)
{
    if (a.n_splits <= 0) return hipSuccess;
    const int rpb = kThreads / (d / 4);
    dim3 grid(a.n_splits, (kKernelBq + rpb - 1) / rpb);
    if (a.o_f32) {
        if (d == 128)
            hipLaunchKernelGGL(split_merge_o32_kernel<128>, grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(split_merge_o32_kernel<64>, grid, dim3(kThreads), 0, stream, a);
    } else if (d == 128) {
        hipLaunchKernelGGL(split_merge_kernel<128>, grid, dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(split_merge_kernel<64>, grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeArgs &a, int d, hipStream_t stream)
{
    if (a.n_tok <= 0 || a.n_head <= 0) return hipSuccess;
    const int rpb = kThreads / (d / (a.parts_f32 ? 4 : 8));
    dim3 grid((unsigned)(((int64_t)a.n_tok + rpb - 1) / rpb * a.n_head));
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, a); };
    const int sel = (a.parts_f32 ? 2 : 0) + (a.o_f32 ? 1 : 0);
    if (d == 128) {
        if (sel == 0) go(attn_merge_kernel<128>);
        else if (sel == 1) go(attn_merge_typed_kernel<128, false, true>);
        else if (sel == 2) go(attn_merge_typed_kernel<128, true, false>);
        else go(attn_merge_typed_kernel<128, true, true>);
    } else {
        if (sel == 0) go(attn_merge_kernel<64>);
        else if (sel == 1) go(attn_merge_typed_kernel<64, false, true>);
        else if (sel == 2) go(attn_merge_typed_kernel<64, true, false>);
        else go(attn_merge_typed_kernel<64, true, true>);
    }
    return hipGetLastError();
}

}  // namespace bsfa
