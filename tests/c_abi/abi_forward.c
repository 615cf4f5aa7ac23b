/* A C99 consumer of libbsfa.so with no Python and no torch: builds a varlen causal plan
 * through the C ABI, runs the forward on HIP device buffers it allocates itself and
 * writes O and LSE for the Python test to compare with the oracle.  Also checks that
 * invalid calls return their documented status codes before touching the GPU, and that
 * the typed entry point's fp32 O rounds to the bf16 O bit for bit with the same LSE.
 *
 * usage: abi_forward DIR
 *   DIR/case.txt: sq hq hkv d n_docs scale, then n_docs + 1 cu_seqlens
 *   DIR/q.bin, k.bin, v.bin: bf16 bits, [sq, hq, d] / [sq, hkv, d] row-major
 *   writes DIR/o.bin (bf16 bits [sq, hq, d]) and DIR/lse.bin (fp32 [hq, sq]) */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/bsfa.h"

static int fail(const char *what, const char *detail)
{
    fprintf(stderr, "abi_forward: %s: %s\n", what, detail);
    return 1;
}

static void *read_file(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    void *buf = malloc(bytes ? bytes : 1);
    if (buf && fread(buf, 1, bytes, f) != bytes) {
        free(buf);
        buf = NULL;
    }
    fclose(f);
    return buf;
}

static int write_file(const char *dir, const char *name, const void *data, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 0;
    const int ok = fwrite(data, 1, bytes, f) == bytes;
    fclose(f);
    return ok;
}

int main(int argc, char **argv)
{
    if (argc != 2) return fail("usage", "abi_forward DIR");
    const char *dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/case.txt", dir);
    FILE *cf = fopen(path, "r");
    if (!cf) return fail("open", path);
    int sq, hq, hkv, d, n_docs;
    float scale;
    if (fscanf(cf, "%d %d %d %d %d %f", &sq, &hq, &hkv, &d, &n_docs, &scale) != 6) return fail("parse", path);
    int32_t *cu = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_docs + 1));
    for (int t = 0; t <= n_docs; ++t)
        if (fscanf(cf, "%d", &cu[t]) != 1) return fail("parse", "cu_seqlens");
    fclose(cf);

    /* documented rejections, before any device work */
    bsfa_plan *bad = NULL;
    if (bsfa_plan_from_varlen(cu, n_docs, 1, 3, 2, d, 128, 128, &bad) != BSFA_ERR_SHAPE)
        return fail("status", "hq % hkv != 0 must give BSFA_ERR_SHAPE");
    if (bsfa_plan_from_varlen(cu, n_docs, 1, hq, hkv, d, 128, 128, NULL) != BSFA_ERR_ARG)
        return fail("status", "a null out must give BSFA_ERR_ARG");
    if (strcmp(bsfa_status_str(BSFA_ERR_SHAPE), "shape mismatch") != 0) return fail("status", "string");

    const size_t nq = (size_t)sq * hq * d, nk = (size_t)sq * hkv * d;
    uint16_t *q = (uint16_t *)read_file(dir, "q.bin", nq * 2);
    uint16_t *k = (uint16_t *)read_file(dir, "k.bin", nk * 2);
    uint16_t *v = (uint16_t *)read_file(dir, "v.bin", nk * 2);
    if (!q || !k || !v) return fail("read", "q/k/v.bin");

    bsfa_plan *plan = NULL;
    bsfa_status st = bsfa_plan_from_varlen(cu, n_docs, 1, hq, hkv, d, 128, 128, &plan);
    if (st != BSFA_OK) return fail("bsfa_plan_from_varlen", bsfa_status_str(st));
    bsfa_plan_info info;
    if ((st = bsfa_plan_get_info(plan, &info)) != BSFA_OK) return fail("bsfa_plan_get_info", bsfa_status_str(st));

    void *dq = NULL, *dk = NULL, *dv = NULL, *dO = NULL, *dl = NULL;
    if (hipMalloc(&dq, nq * 2) != hipSuccess || hipMalloc(&dk, nk * 2) != hipSuccess ||
        hipMalloc(&dv, nk * 2) != hipSuccess || hipMalloc(&dO, nq * 2) != hipSuccess ||
        hipMalloc(&dl, (size_t)hq * sq * 4) != hipSuccess)
        return fail("hipMalloc", "device buffers");
    if (hipMemcpy(dq, q, nq * 2, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dk, k, nk * 2, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dv, v, nk * 2, hipMemcpyHostToDevice) != hipSuccess)
        return fail("hipMemcpy", "inputs");

    /* not yet uploaded: rejected */
    bsfa_tensor tq = {dq, (int64_t)hq * d, d}, tk = {dk, (int64_t)hkv * d, d}, tv = {dv, (int64_t)hkv * d, d};
    bsfa_tensor to = {dO, (int64_t)hq * d, d};
    if (bsfa_attn_fwd(&tq, &tk, &tv, plan, scale, &to, (float *)dl, sq, NULL, 0, NULL) != BSFA_ERR_STATE)
        return fail("status", "a plan not uploaded must give BSFA_ERR_STATE");
    if ((st = bsfa_plan_upload(plan, NULL)) != BSFA_OK) return fail("bsfa_plan_upload", bsfa_status_str(st));
    if ((st = bsfa_attn_fwd(&tq, &tk, &tv, plan, scale, &to, (float *)dl, sq, NULL, 0, NULL)) != BSFA_OK)
        return fail("bsfa_attn_fwd", bsfa_status_str(st));
    if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", "forward");

    uint16_t *o = (uint16_t *)malloc(nq * 2);
    float *lse = (float *)malloc((size_t)hq * sq * 4);
    if (hipMemcpy(o, dO, nq * 2, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(lse, dl, (size_t)hq * sq * 4, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy", "outputs");
    if (!write_file(dir, "o.bin", o, nq * 2) || !write_file(dir, "lse.bin", lse, (size_t)hq * sq * 4))
        return fail("write", "o/lse.bin");

    /* the typed entry point: fp32 O rounds (to nearest even) to the bf16 O, same LSE */
    void *dO32 = NULL, *dl32 = NULL;
    if (hipMalloc(&dO32, nq * 4) != hipSuccess || hipMalloc(&dl32, (size_t)hq * sq * 4) != hipSuccess)
        return fail("hipMalloc", "fp32 output");
    bsfa_tensor to32 = {dO32, (int64_t)hq * d, d};
    if (bsfa_attn_fwd_typed(&tq, &tk, &tv, plan, scale, &to32, 7, (float *)dl32, sq, NULL, 0, NULL) != BSFA_ERR_ARG)
        return fail("status", "an unknown output type must give BSFA_ERR_ARG");
    if ((st = bsfa_attn_fwd_typed(&tq, &tk, &tv, plan, scale, &to32, BSFA_DTYPE_F32, (float *)dl32, sq, NULL, 0,
                                  NULL)) != BSFA_OK)
        return fail("bsfa_attn_fwd_typed", bsfa_status_str(st));
    if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", "fp32 forward");
    uint32_t *o32 = (uint32_t *)malloc(nq * 4);
    float *lse32 = (float *)malloc((size_t)hq * sq * 4);
    if (hipMemcpy(o32, dO32, nq * 4, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(lse32, dl32, (size_t)hq * sq * 4, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy", "fp32 outputs");
    for (size_t i = 0; i < nq; ++i) {
        const uint32_t b = o32[i];
        const uint16_t r = (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);   /* finite values */
        if (r != o[i]) return fail("fp32 O", "does not round to the bf16 O");
    }
    if (memcmp(lse32, lse, (size_t)hq * sq * 4) != 0) return fail("fp32 O", "LSE differs from the bf16 call's");
    hipFree(dO32);
    hipFree(dl32);
    free(o32);
    free(lse32);
    bsfa_plan_destroy(plan);
    hipFree(dq);
    hipFree(dk);
    hipFree(dv);
    hipFree(dO);
    hipFree(dl);
    printf("abi_forward: %d tokens, %d heads, d %d: %lld tiles (%lld partial), %lld pairs per head\n", sq, hq, d,
           (long long)info.nnz, (long long)info.n_partial, (long long)info.pairs);
    free(q);
    free(k);
    free(v);
    free(o);
    free(lse);
    free(cu);
    return 0;
}
