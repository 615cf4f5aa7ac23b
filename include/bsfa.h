/*
 * bsfa.h -- C ABI of libbsfa.so: masked flash-attention forward over a tile CSR
 * and the merge of KV-split partials, for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as published):
 *   [MA] "Sand.ai releases MagiAttention v1.1.0" (news), list "Blackwell adaptation":
 *        flexible masks, block-sparse mask generation without a dense mask,
 *        CSR-compressed mask metadata, cheap kernel launches; list "system-level
 *        co-optimisation": Dispatch Solver, a min-heap greedy balancer.
 *   [UA] "UltraAttn: hierarchical context tiling" (blog), 3 (Full / Causal / Empty
 *        blocks), 3.1 (Q split), 3.2 (KV split and the mergeable summary),
 *        3.3 (2-D block view), 4.1 (block weights 1 / 0.5 / 0 and the imbalance
 *        bound), 8 (strided block-sparse pattern).
 *   [F4] QbitAI article on FlashAttention-4, "three techniques" part
 *        (conditional softmax rescaling; softmax overlapped with matrix products).
 *   [FT] "FlashAttention-T: tensor-vector parallel optimisation" (blog),
 *        FlashAttention lineage (tiling + incremental softmax), double-buffered
 *        on-chip staging, numerical-stability parameters.
 *
 * Conventions for every call:
 *   - Status codes only; nothing throws across this boundary.  Arguments are
 *     validated before any device work is enqueued; a rejected call writes nothing.
 *   - Device pointers are HIP device memory of the current device, owned by the
 *     caller.  The library does not inspect where an address points (a host address
 *     would reach the kernels as it is); the Python binding checks its tensors.  "stream" is a
 *     hipStream_t passed as void* (NULL = the default stream).  Device work is
 *     enqueued on that stream and the call returns without synchronising.
 *   - Tensors are bf16 with the head dimension contiguous; token and head strides
 *     are given in elements, must be multiples of 8, and base pointers must be
 *     16-byte aligned.
 */
#ifndef BSFA_H
#define BSFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSFA_OK = 0,
    BSFA_ERR_ARG = 1,         /* null pointer, bad count, value out of range */
    BSFA_ERR_SHAPE = 2,       /* shapes disagree with the plan, Hq % Hkv != 0, ... */
    BSFA_ERR_ALIGN = 3,       /* base pointer not 16-byte aligned or stride not a multiple of 8 */
    BSFA_ERR_UNSUPPORTED = 4, /* head dim / tile size the kernels do not implement */
    BSFA_ERR_MASK = 5,        /* slice outside [0, S), q1 < q0, k1 < k0, unknown type or code */
    BSFA_ERR_OOM = 6,         /* host or device allocation failed */
    BSFA_ERR_HIP = 7,         /* a HIP runtime call failed (including a sticky earlier fault) */
    BSFA_ERR_STATE = 8,       /* plan not uploaded to the current device */
    BSFA_ERR_PLAN = 9         /* plan metadata failed its consistency check (internal error) */
} bsfa_status;

/* One mask slice ([MA] flexible masks; [UA] 3): the pairs (i, j) with q0 <= i < q1 and
 * k0 <= j < k1; type BSFA_FULL admits all of them, BSFA_CAUSAL only those with
 * j - k1 <= i - q1 (causal aligned at the slice's bottom-right corner, which is
 * plain j <= i when k1 == q1).  A mask is the union of its slices' pair sets. */
typedef struct {
    int32_t q0, q1, k0, k1, type;
} bsfa_slice;

enum { BSFA_FULL = 0, BSFA_CAUSAL = 1 };
enum { BSFA_TILE_FULL = 1, BSFA_TILE_PARTIAL = 2 };

/* A bf16 [tokens, heads, head_dim] tensor view: element (t, h, e) lives at
 * ptr + t * stride_tok + h * stride_head + e  (strides in elements). */
typedef struct {
    void *ptr;
    int64_t stride_tok;
    int64_t stride_head;
} bsfa_tensor;

typedef struct bsfa_plan bsfa_plan;

typedef struct {
    int32_t sq, sk, hq, hkv, d, bq, bk;
    int32_t n_qtiles, n_ktiles;
    int64_t nnz;          /* non-empty (bq x bk) tiles in the CSR */
    int64_t n_full;       /* tiles tagged BSFA_TILE_FULL */
    int64_t n_partial;    /* tiles tagged BSFA_TILE_PARTIAL */
    int64_t n_pieces;     /* clipped slice pieces stored for partial tiles */
    int64_t pairs;        /* admitted (query, key) pairs of one head */
    int32_t n_items;      /* work items = (query head, query tile) */
    int32_t n_bins;       /* persistent workgroups of the forward launch */
    double makespan;      /* largest bin cost of the schedule (cost units) */
    double total_cost;    /* sum of unit costs */
    int32_t uploaded;     /* 1 once bsfa_plan_upload has run */
    int32_t n_units;      /* scheduled units: n_items plus one per extra part of a split row */
    int32_t n_splits;     /* (query head, query tile) rows split into parts */
    int64_t workspace_bytes;  /* device bytes for the parts' partial results (0 if no split) */
} bsfa_plan_info;

/* ---- plans: mask compiler + scheduler (host) --------------------------------
 * A plan is the compiled form of one mask for fixed shapes: a CSR of the non-empty
 * (bq x bk) tiles of every query tile ([MA] CSR metadata; [UA] 3.3 skip Empty
 * blocks), each tagged full or partial ([UA] 3 block classes), the slice pieces of
 * each partial tile, and a schedule of (query head, query tile) items over the
 * persistent workgroups built by a min-heap greedy on a tile-count cost ([MA]
 * Dispatch Solver; [UA] 4.1 weights).  Creation is host-only and never touches
 * the GPU.  The kernels need bq == 128 and bk a multiple of 64; other tile sizes
 * build a plan whose CSR can be exported but which bsfa_attn_fwd rejects.
 * A plan is immutable after creation and may be shared by launches on several streams
 * at once; the caller frees it with bsfa_plan_destroy.
 * Limits: fewer than 2^27 non-empty tiles and 2^26 pieces (the kernels address both
 * arrays with 32-bit byte offsets), e.g. a single causal sequence of up to about 2.9M
 * tokens at 128 x 128 tiles; larger plans are refused with BSFA_ERR_UNSUPPORTED.
 * Errors: BSFA_ERR_ARG (null out, n_slices < 0, bad sizes), BSFA_ERR_SHAPE
 * (hq % hkv), BSFA_ERR_MASK (slice outside [0,sq) x [0,sk], q1 < q0, k1 < k0, unknown
 * type), BSFA_ERR_UNSUPPORTED (the limits above), BSFA_ERR_OOM. */
bsfa_status bsfa_plan_create(const bsfa_slice *slices, int32_t n_slices, int32_t sq, int32_t sk,
                             int32_t hq, int32_t hkv, int32_t d, int32_t bq, int32_t bk,
                             bsfa_plan **out);

/* Packed variable-length documents ([MA] varlen masks): document t covers tokens
 * [cu_seqlens[t], cu_seqlens[t+1]) on both axes, causal when causal != 0, full
 * otherwise; no pair crosses documents.  cu_seqlens has n_docs + 1 nondecreasing
 * host int32 entries starting at 0; the total length is cu_seqlens[n_docs]. */
bsfa_status bsfa_plan_from_varlen(const int32_t *cu_seqlens, int32_t n_docs, int32_t causal,
                                  int32_t hq, int32_t hkv, int32_t d, int32_t bq, int32_t bk,
                                  bsfa_plan **out);

/* Block pattern ([MA] block-sparse masks; [UA] 8 strided pattern): codes is a host
 * uint8 [nbq, nbk] row-major map over (block_q x block_k) blocks, 0 = empty,
 * 1 = full, 2 = causal inside the block; blocks are clipped to [0, sq) x [0, sk). */
bsfa_status bsfa_plan_from_blocks(const uint8_t *codes, int32_t nbq, int32_t nbk,
                                  int32_t block_q, int32_t block_k, int32_t sq, int32_t sk,
                                  int32_t hq, int32_t hkv, int32_t d, int32_t bq, int32_t bk,
                                  bsfa_plan **out);

/* Copy the plan's metadata to the current HIP device.  The copy runs on an internal
 * per-device copy stream (so it overlaps kernels already enqueued on stream); every
 * library launch that reads the metadata (bsfa_attn_fwd, bsfa_attn_bwd), on any
 * stream, is ordered after it: once the copy is seen complete nothing is enqueued,
 * before that the launch stream waits for it, so a plan uploaded ahead of its launch
 * adds no cross-stream dependency.  stream is the stream the device buffer is also
 * released behind (with every launch stream) at bsfa_plan_destroy.  The device buffer comes from a
 * per-device pool the library owns: buffers are
 * allocated on first need, reused by later plans and held until process exit, so a
 * steady stream of plans allocates nothing and never synchronises.  Must precede
 * bsfa_attn_fwd.  Before any device work the plan's metadata is checked on the host
 * (offsets monotone and in range, every scheduled unit in exactly one bin, ...), since
 * the kernels trust it.  Errors: BSFA_ERR_ARG, BSFA_ERR_STATE (already uploaded),
 * BSFA_ERR_PLAN (metadata inconsistent: an internal error), BSFA_ERR_OOM, BSFA_ERR_HIP. */
bsfa_status bsfa_plan_upload(bsfa_plan *plan, void *stream);

/* Releases host memory and, if uploaded, hands the device buffer back to the pool
 * behind the work enqueued so far on the upload stream and on every stream the plan
 * was launched on (an event is recorded on each; the buffer is reused only after all
 * of them have completed).  Never waits.  NULL is accepted. */
void bsfa_plan_destroy(bsfa_plan *plan);

bsfa_status bsfa_plan_get_info(const bsfa_plan *plan, bsfa_plan_info *info);

/* Copy out the tile CSR (for bit-exact checks): row_ptr [n_qtiles + 1], col [nnz]
 * (ascending within a row), tag [nnz] (BSFA_TILE_FULL / BSFA_TILE_PARTIAL), all host
 * memory.  cap is the capacity of col and tag; *nnz is always set.  Returns
 * BSFA_ERR_ARG if cap < nnz (nothing but *nnz written). */
bsfa_status bsfa_plan_export_csr(const bsfa_plan *plan, int32_t *row_ptr, int32_t *col,
                                 uint8_t *tag, int64_t cap, int64_t *nnz);

/* Copy out the schedule: bin_ptr [n_bins + 1], units [n_units] (unit ids in execution
 * order within a bin) and unit_cost [n_units] (indexed by unit id), host memory.  Any
 * pointer may be NULL to skip it.  When no row is split, unit id == item id =
 * h * n_qtiles + qtile and the unit costs are the item costs. */
bsfa_status bsfa_plan_export_schedule(const bsfa_plan *plan, int32_t *bin_ptr, int32_t *units,
                                      float *unit_cost);

/* Copy out the units ([UA] 3.2: a query tile's key range split into parts whose
 * summaries merge exactly): units [n_units][4] = {item, entry_begin, entry_end, slot}
 * where [entry_begin, entry_end) indexes the tile CSR's col/tag arrays and slot is -1
 * for a whole row or the partial-result slot of a part.  A row is split when its cost
 * exceeds both the per-bin target (total cost / resident workgroups) and 16 steps: into
 * at most 16 parts of contiguous entries with about equal cost. */
bsfa_status bsfa_plan_export_units(const bsfa_plan *plan, int32_t *units);

/* Copy out the pieces of the partial tiles: piece_ptr [nnz + 1] (pieces of entry e are
 * piece_ptr[e] .. piece_ptr[e + 1] - 1; a full tile has none) and pieces
 * [n_pieces][5] = {q_lo, q_hi, k_lo, k_hi, diag}: the piece admits (i, j) iff
 * q_lo <= i < q_hi, k_lo <= j < k_hi and j <= i + diag (a full slice stores
 * diag = 2^30).  Host memory; cap is the capacity of pieces in pieces.  Returns
 * BSFA_ERR_ARG if cap < n_pieces or a pointer is NULL. */
bsfa_status bsfa_plan_export_pieces(const bsfa_plan *plan, int32_t *piece_ptr, int32_t *pieces,
                                    int64_t cap);

/* Cost of one tile under the scheduler's model ([UA] 4.1: full = 1, causal/partial =
 * w_partial, empty = 0) and the page's imbalance bound ceil(avg)/avg - 1 for a total
 * cost split over n_bins units of integral capacity. */
double bsfa_tile_cost(int32_t tag, double w_partial);
double bsfa_imbalance_bound(double total_cost, int32_t n_bins);

/* The scheduler's core, usable on any list of costs ([MA] Dispatch Solver, a
 * min-heap greedy): items in order of decreasing cost (ties: lower index first) go
 * one by one to the least-loaded bin (ties: lower bin index).  bin_of[n_items]
 * receives each item's bin, bin_load[n_bins] (may be NULL) the final loads.
 * Returns the makespan (largest load), or -1 on bad arguments (n_items < 0,
 * n_bins < 1, null cost/bin_of with n_items > 0, a negative or non-finite cost). */
double bsfa_lpt_assign(const float *cost, int32_t n_items, int32_t n_bins, int32_t *bin_of,
                       double *bin_load);

/* ---- forward ([FT] tiling + incremental softmax; [UA] 3.1-3.3; [F4]) --------
 * O[i, h, :] = sum_j softmax_j(scale * q_i . k_j) v_j over the plan's admitted keys of
 * row i, for every query row i < sq and query head h; LSE[h * lse_stride_head + i] =
 * natural log-sum-exp of the scaled scores.  A row with no admitted key gets O = 0
 * and LSE = -inf.  Query head h reads key/value head h / (hq / hkv).
 * q, o: [sq, hq, d]; k, v: [sk, hkv, d]; lse: fp32, lse_stride_head >= sq.  Pointers of
 * empty extents may be NULL (sq == 0: q, o, lse; sk == 0: k, v).
 * Shapes come from the plan, which must be uploaded to the current device.
 * No allocation, no synchronisation; deterministic (no atomics).  The stream is
 * remembered so that bsfa_plan_destroy releases the plan's buffer behind it.
 * A plan with split rows (info.n_splits > 0; [UA] 3.2: a key range cut into parts whose
 * summaries merge exactly) runs a second kernel on the same stream that merges the
 * parts.  Their partial results go to `workspace`: caller device memory of at least
 * info.workspace_bytes bytes (16-byte aligned), read and written only by this call's
 * kernels; NULL (with workspace_bytes 0) is accepted when the plan has no split row.
 * The plan itself is never written, so launches of one plan may overlap on several
 * streams as long as each has its own workspace.
 * Errors: BSFA_ERR_ARG (also a missing or too small workspace), BSFA_ERR_ALIGN,
 * BSFA_ERR_SHAPE (stride_tok < d for a tensor with a token), BSFA_ERR_UNSUPPORTED (d not
 * 64/128, bq != 128, bk % 64 != 0), BSFA_ERR_STATE (plan not on this device),
 * BSFA_ERR_HIP. */
bsfa_status bsfa_attn_fwd(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                          const bsfa_plan *plan, float scale, bsfa_tensor *o, float *lse,
                          int64_t lse_stride_head, void *workspace, int64_t workspace_bytes,
                          void *stream);

/* ---- fp32 outputs ([UA] 3.2: a partial result is its normalised output and LSE) ----
 * bsfa_attn_fwd and bsfa_attn_merge write bf16 outputs.  The _typed forms take the
 * element type of O (and of the merge's partials): BSFA_DTYPE_BF16 or BSFA_DTYPE_F32.
 * An fp32 O holds the normalised fp32 value that the bf16 output is rounded from (round
 * to nearest even), so a bf16 call and an fp32 call on the same inputs and plan give
 * bf16(O_f32) == O_bf16 bit for bit and the same LSE; it keeps the half-ulp rounding of
 * a bf16 output (up to 2^-9 |O|) out of KV-split partials that are merged afterwards.
 * An fp32 O is a [tokens, heads, d] fp32 tensor view (bsfa_tensor, element strides)
 * with 16-byte aligned base and strides that are multiples of 4 elements; everything
 * else is as for bsfa_attn_fwd.  Errors as bsfa_attn_fwd, plus BSFA_ERR_ARG for an
 * unknown o_dtype. */
enum { BSFA_DTYPE_BF16 = 0, BSFA_DTYPE_F32 = 1 };
bsfa_status bsfa_attn_fwd_typed(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                                const bsfa_plan *plan, float scale, bsfa_tensor *o, int32_t o_dtype,
                                float *lse, int64_t lse_stride_head, void *workspace,
                                int64_t workspace_bytes, void *stream);

/* ---- forward without allocation ------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): bsfa_attn_fwd with the split rows'
 * partial results in a static device workspace of the library instead of a caller
 * buffer.  The workspace is BSFA_STATIC_WORKSPACE_BYTES (32 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends, and shared by every call on
 * that GPU: calls that overlap on one GPU (on different streams, or from several host
 * threads) race on it and must be ordered by the caller.  Plans whose
 * info.workspace_bytes exceeds it are refused with BSFA_ERR_UNSUPPORTED (about 500
 * split-row parts at d = 128); plans without split rows never touch it.  Arguments,
 * results and every other error as bsfa_attn_fwd; no allocation, no synchronisation.
 * The workspace's address is looked up once per GPU, on the first call with that GPU
 * current. */
enum { BSFA_STATIC_WORKSPACE_BYTES = 32 << 20 };
bsfa_status bsfa_attn_fwd_noalloc(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                                  const bsfa_plan *plan, float scale, bsfa_tensor *o, float *lse,
                                  int64_t lse_stride_head, void *stream);

/* ---- backward ([MA] the same masked attention, forward and backward) ----------
 * Gradients of the forward above for an upstream gradient dO:
 *   P_ij = exp(scale q_i.k_j - LSE_i) on the plan's admitted pairs (0 elsewhere),
 *   dP_ij = dO_i.v_j,  D_i = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - D_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_(h,i) dS_ij q_i,
 *   dV_j = sum_(h,i) P_ij dO_i  (h over the query heads of j's key/value head).
 * D_i is formed from the recomputed P and dP (it equals dO_i.O_i for the exact O), so
 * the forward's output is not an input and its bf16 rounding does not enter the
 * gradients.
 * q, dout: bf16 [sq, hq, d]; k, v: bf16 [sk, hkv, d] (strides as bsfa_attn_fwd);
 * lse: the forward's fp32 LSE [hq, lse_stride_head].  dq [sq, hq, d], dk and dv
 * [sk, hkv, d]: fp32, contiguous, 16-byte aligned, fully written (rows no key reaches
 * get zeros).  delta: caller scratch of LSE's shape (fp32 [hq, lse_stride_head]),
 * overwritten with D.  With sq == 0, q, dout, lse, delta and dq may be NULL; with
 * sk == 0, k, v, dk and dv.  The plan must have bq = 128 and bk = 128 and be uploaded to the
 * current device.  Three kernels on stream: D by query tile over its CSR row, dQ by
 * query tile, then dK/dV by key tile over the query heads of its key/value head (no
 * atomics, deterministic).  No allocation, no synchronisation.
 * Errors: BSFA_ERR_ARG, BSFA_ERR_ALIGN, BSFA_ERR_SHAPE (stride_tok < d for a tensor with
 * a token), BSFA_ERR_UNSUPPORTED (d not 64/128, tiles not 128 x 128), BSFA_ERR_STATE,
 * BSFA_ERR_HIP. */
bsfa_status bsfa_attn_bwd(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                          const bsfa_tensor *dout, const float *lse, int64_t lse_stride_head,
                          const bsfa_plan *plan, float scale, float *dq, float *dk, float *dv,
                          float *delta, void *stream);

/* bsfa_attn_bwd given the forward's fp32 output o (bsfa_attn_fwd_typed with
 * BSFA_DTYPE_F32, same inputs and plan): D_i = dO_i . O_i is formed from it (the fp32
 * value the bf16 output is rounded from, so the bf16 rounding stays out of D) inside
 * the dQ kernel, and the separate D pass is skipped (two kernels instead of three).
 * o: fp32 [sq, hq, d], 16-byte aligned, strides multiples of 4 elements, stride_tok >= d;
 * may be NULL's ptr only when sq == 0.  delta still receives D.  Everything else, errors
 * included, as bsfa_attn_bwd; BSFA_ERR_ARG for a NULL o. */
bsfa_status bsfa_attn_bwd_o32(const bsfa_tensor *q, const bsfa_tensor *k, const bsfa_tensor *v,
                              const bsfa_tensor *dout, const bsfa_tensor *o, const float *lse,
                              int64_t lse_stride_head, const bsfa_plan *plan, float scale, float *dq,
                              float *dk, float *dv, float *delta, void *stream);

/* ---- merge of KV-split partials ([UA] 3.2) -----------------------------------
 * For n partial results (O_t, LSE_t) of the same queries over disjoint key sets:
 *   M = max_t LSE_t, LSE = M + ln sum_t exp(LSE_t - M), O = sum_t exp(LSE_t - LSE) O_t;
 * rows where every LSE_t is -inf get O = 0, LSE = -inf.
 * o_parts / lse_parts: host arrays of n device pointers; every O_t is a bf16
 * [n_tok, n_head, d] tensor with element strides part_stride_tok and part_stride_head
 * (multiples of 8, head dim contiguous), every LSE_t an fp32 [n_head, lse_stride_head]
 * array.  o (bf16, strides from o->stride_*) and lse receive
 * the result and must not overlap any partial.  1 <= n <= BSFA_MERGE_MAX_PARTS,
 * d in {64, 128}, ceil(n_tok / 16) * n_head < 2^31.  With n_tok == 0 or n_head == 0 the
 * call does nothing and returns BSFA_OK (its pointers may then be NULL).  Partials and result are streamed
 * with non-temporal accesses (they bypass the caches' retention).
 * Errors: BSFA_ERR_ARG, BSFA_ERR_ALIGN, BSFA_ERR_UNSUPPORTED, BSFA_ERR_HIP. */
enum { BSFA_MERGE_MAX_PARTS = 16 };
bsfa_status bsfa_attn_merge(const void *const *o_parts, const float *const *lse_parts, int32_t n,
                            int64_t part_stride_tok, int64_t part_stride_head,
                            int64_t lse_stride_head, int32_t n_tok, int32_t n_head, int32_t d,
                            bsfa_tensor *o, float *lse, void *stream);

/* bsfa_attn_merge with the partials' and the result's element types given
 * (BSFA_DTYPE_BF16 / BSFA_DTYPE_F32, independently).  fp32 tensors need strides that are
 * multiples of 4 elements; with fp32 partials the limit is ceil(n_tok / 8) * n_head < 2^31.
 * Errors as bsfa_attn_merge, plus BSFA_ERR_ARG for an unknown type. */
bsfa_status bsfa_attn_merge_typed(const void *const *o_parts, int32_t parts_dtype,
                                  const float *const *lse_parts, int32_t n, int64_t part_stride_tok,
                                  int64_t part_stride_head, int64_t lse_stride_head, int32_t n_tok,
                                  int32_t n_head, int32_t d, bsfa_tensor *o, int32_t o_dtype, float *lse,
                                  void *stream);

/* ---- device mask compiler ------------------------------------------------------
 * The tile CSR of a slice mask built on the GPU ([MA] "Blackwell adaptation": block-
 * sparse mask generation without instantiating a dense mask, CSR mask metadata; [UA] 3
 * block classes, 3.3 skip Empty blocks).  Its arrays equal, entry for entry, those of a
 * plan made from the same slices and tile sizes (bsfa_plan_export_csr /
 * bsfa_plan_export_pieces): per query tile the non-empty key tiles in ascending order,
 * tagged full when one slice or the union of the slices admits every in-range pair of
 * the tile, else partial with the tile's clipped slices in ascending slice order.
 *
 * bsfa_dcsr_build validates the slices on the host (as bsfa_plan_create), lists every
 * (slice, query tile) pair with the key tiles it reaches (host work proportional to the
 * number of such pairs), allocates one device buffer on the current device and enqueues
 * the compile on `stream` (a hipStream_t, NULL = the default stream); it does not wait
 * for the GPU.  The work is proportional to the (tile, slice) incidences ("touches").
 * Limits: bk <= 256, n_slices < 2^24, touches < 2^31, and the key
 * (query tile * n_ktiles + key tile) * 2^ceil(log2 n_slices) must fit in 64 bits
 * (else BSFA_ERR_UNSUPPORTED).  Errors: BSFA_ERR_ARG, BSFA_ERR_MASK as
 * bsfa_plan_create; BSFA_ERR_OOM; BSFA_ERR_HIP for a failed allocation, copy or launch.
 *
 * bsfa_dcsr_view_get waits for the compile and fills `view` with device pointers into
 * the object's buffer and the totals (one small device-to-host copy the first time).
 * bsfa_dcsr_destroy waits for the compile and frees the buffer; views die with it. */
typedef struct bsfa_dcsr bsfa_dcsr;

typedef struct {
    const int32_t *row_ptr;    /* [n_qtiles + 1], device */
    const int32_t *col;        /* [nnz], device */
    const uint8_t *tag;        /* [nnz], device: BSFA_TILE_FULL / BSFA_TILE_PARTIAL */
    const int32_t *piece_ptr;  /* [nnz + 1], device */
    const int32_t *pieces;     /* [n_pieces][8], device: q_lo, q_hi, k_lo, k_hi, diag, 0, 0, 0 */
    int32_t n_qtiles, n_ktiles;
    int64_t nnz, n_full, n_partial, n_pieces;
    int64_t pairs;             /* admitted (query, key) pairs of one head */
    int64_t touches;           /* (tile, slice) incidences the compile expanded */
} bsfa_dcsr_view;

bsfa_status bsfa_dcsr_build(const bsfa_slice *slices, int32_t n_slices, int32_t sq, int32_t sk,
                            int32_t bq, int32_t bk, void *stream, bsfa_dcsr **out);
/* The same device CSR from a block-code map whose blocks are the tiles ([MA] "Blackwell
 * adaptation": block-sparse mask generation on the device; [UA] 3 Full / Causal / Empty
 * blocks): codes is a host uint8 [nbq, nbk] row-major map over (bq x bk) blocks, 0 =
 * empty, 1 = full, 2 = causal inside the block, blocks clipped to [0, sq) x [0, sk) --
 * the mask bsfa_plan_from_blocks builds with block_q = bq, block_k = bk.  The arrays
 * equal, entry for entry, those of that plan: each non-empty block in range is one
 * entry, full for code 1 (and for a causal block of one row), else partial with the
 * block itself as its one piece (diag = k1 - q1 of the clipped block).  The host checks
 * the codes and counts the entries (one pass over the map), copies the map to the
 * device and enqueues the compile on stream (no wait); touches = nnz.  Errors:
 * BSFA_ERR_ARG, BSFA_ERR_MASK (a code above 2), BSFA_ERR_UNSUPPORTED (2^31 entries or
 * pieces or more), BSFA_ERR_OOM, BSFA_ERR_HIP. */
bsfa_status bsfa_dcsr_build_blocks(const uint8_t *codes, int32_t nbq, int32_t nbk, int32_t sq, int32_t sk,
                                   int32_t bq, int32_t bk, void *stream, bsfa_dcsr **out);
bsfa_status bsfa_dcsr_view_get(bsfa_dcsr *csr, bsfa_dcsr_view *view);
/* Waits for the compile and copies its arrays to host memory in the layouts of
 * bsfa_plan_export_csr and bsfa_plan_export_pieces: row_ptr [n_qtiles + 1], col and tag
 * [nnz], piece_ptr [nnz + 1], pieces [n_pieces][5].  cap_nnz / cap_pieces are the
 * capacities of col, tag / pieces; BSFA_ERR_ARG if too small or a pointer is NULL
 * (pieces may be NULL when n_pieces is 0). */
bsfa_status bsfa_dcsr_export(bsfa_dcsr *csr, int32_t *row_ptr, int32_t *col, uint8_t *tag,
                             int32_t *piece_ptr, int32_t *pieces, int64_t cap_nnz, int64_t cap_pieces);
void bsfa_dcsr_destroy(bsfa_dcsr *csr);

/* A plan over a device-compiled tile CSR ([MA]: block-sparse mask generation without a
 * dense mask, CSR mask metadata driving the kernels), built where the CSR is: the GPU
 * counts each query tile's full and partial steps and each key tile's entries, the host
 * receives only those n_qtiles + n_ktiles counts (and row_ptr) and builds the min-heap
 * schedule and the gradient launch orders from them (a row split into parts also has its
 * own entries copied back), and the plan's device image (entry records, pieces, the
 * column view by a stable sort of the entries' key tiles) is assembled on the GPU.  The
 * plan equals the one bsfa_plan_create builds from the same slices and tile sizes field
 * for field (CSR, pieces, schedule, units, launch orders), so the forward and backward
 * outputs are bit-identical.  It is resident on the current device from the start:
 * bsfa_plan_upload on it copies nothing and only records its stream as one to release the
 * buffer behind; launches are ordered after the image's assembly (an internal stream) as
 * after an upload.  The exports copy its CSR back from the device image.  hq, hkv, d as
 * for bsfa_plan_create; the extents and tile sizes are those csr was compiled with.  csr
 * stays owned by the caller and may be destroyed afterwards.  The current device must be
 * the one csr was built on.  Errors: BSFA_ERR_ARG, BSFA_ERR_SHAPE (hq % hkv),
 * BSFA_ERR_STATE (another current device), BSFA_ERR_UNSUPPORTED (plan limits),
 * BSFA_ERR_OOM, BSFA_ERR_HIP, BSFA_ERR_PLAN (internal inconsistency). */
bsfa_status bsfa_plan_from_dcsr(bsfa_dcsr *csr, int32_t hq, int32_t hkv, int32_t d, bsfa_plan **out);

/* Threshold of the forward's conditional rescaling ([F4] "three techniques": rescale the
 * running sums only when needed): a row's running max moves only when a tile's maximum
 * scaled score exceeds it by more than tau_log2 (log2 units); until then the tile's
 * weights are taken against the old max and may reach 2^tau.  Results equal those of any
 * other threshold up to rounding; 0 moves the max whenever it grows.  Default 8.
 * Process-wide, read when a forward launch is enqueued (launches already enqueued keep
 * theirs).  Errors: BSFA_ERR_ARG unless 0 <= tau_log2 <= 64 (weights up to 2^64 keep the
 * fp32 sums finite). */
bsfa_status bsfa_set_rescale_threshold(float tau_log2);
float bsfa_get_rescale_threshold(void);

const char *bsfa_status_str(bsfa_status status);

#ifdef __cplusplus
}
#endif

#endif /* BSFA_H */
