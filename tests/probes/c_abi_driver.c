/*
 * c_abi_driver.c -- libbeaconkv.so called from plain C (no Python, no torch):
 * a random-selector eviction pass (Philox draws, top-B selection, in-place
 * compaction) on a small paged cache, through bkv_workspace_size and
 * bkv_evict_pass, plus one refused call.  Test-only: it prints what it got and
 * tests/test_gpu_c_abi.py checks the output against the oracle.
 *
 * The cache: 1 layer, 2 requests, 2 KV heads, 40 physical blocks of 16 slots;
 * request r owns physical blocks 20 r .. 20 r + 19, its block i being
 * 20 r + (7 i mod 20).  Every bf16 element of the pools is a fixed hash of its
 * flat index (pool_value below), so the test can rebuild the same cache.
 *
 * Output lines:
 *   abi <version>
 *   workspace <bytes>
 *   refused <code> <status string>        (a pass without its workspace)
 *   pass <return code> <device status word>
 *   hc <hc> keep <entries of the keep row, -1 padding dropped>
 *   hc <hc> draws <FNV-1a 64 of the draw row's N - P words, little-endian>
 *   hc <hc> rows <FNV-1a 64 of the first kept-count K rows> <... V rows>
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "beaconkv.h"

enum { L = 1, R = 2, H = 2, NBLK = 40, MAXB = 20, D = 128, BS = 16, HC = L * R * H };
static const int32_t SEQ[R] = {300, 213};
static const int32_t PROMPT[R] = {40, 7};
static const int32_t BUDGET = 128;

static uint16_t pool_value(uint32_t idx, uint32_t salt) {
    uint32_t x = idx * 2654435761u + salt;
    x ^= x >> 15;
    x *= 2246822519u;
    x ^= x >> 13;
    return (uint16_t)(x & 0xFFFFu);
}

static uint64_t fnv1a(const void* p, size_t n) {
    const unsigned char* b = (const unsigned char*)p;
    uint64_t h = 14695981039346656037ull;
    for (size_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 1099511628211ull;
    }
    return h;
}

#define CHECK(x)                                                          \
    do {                                                                  \
        hipError_t e_ = (x);                                              \
        if (e_ != hipSuccess) {                                           \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); \
            return 2;                                                     \
        }                                                                 \
    } while (0)

int main(void) {
    const size_t pool_elems = (size_t)NBLK * H * BS * D;
    uint16_t* hk = malloc(pool_elems * 2);
    uint16_t* hv = malloc(pool_elems * 2);
    int32_t bt[R * MAXB];
    for (size_t i = 0; i < pool_elems; ++i) {
        hk[i] = pool_value((uint32_t)i, 1u);
        hv[i] = pool_value((uint32_t)i, 2u);
    }
    for (int r = 0; r < R; ++r)
        for (int i = 0; i < MAXB; ++i) bt[r * MAXB + i] = 20 * r + (7 * i) % 20;
    const uint64_t rid[R] = {11, 12};
    const int32_t pass_idx[R] = {2, 3};

    void *dk, *dv, *dbt, *dseq, *dprompt, *drid, *dpass, *dscores, *dkeep, *dstatus;
    uint64_t pools_k[L];   /* device addresses of the per-layer pools */
    uint64_t pools_v[L];
    void* dpk;
    void* dpv;
    const int stride = MAXB * BS;
    CHECK(hipMalloc(&dk, pool_elems * 2));
    CHECK(hipMalloc(&dv, pool_elems * 2));
    CHECK(hipMalloc(&dbt, sizeof bt));
    CHECK(hipMalloc(&dseq, sizeof SEQ));
    CHECK(hipMalloc(&dprompt, sizeof PROMPT));
    CHECK(hipMalloc(&drid, sizeof rid));
    CHECK(hipMalloc(&dpass, sizeof pass_idx));
    CHECK(hipMalloc(&dscores, (size_t)HC * stride * 4));
    CHECK(hipMalloc(&dkeep, (size_t)HC * BUDGET * 4));
    CHECK(hipMalloc(&dstatus, 4));
    CHECK(hipMalloc(&dpk, sizeof pools_k));
    CHECK(hipMalloc(&dpv, sizeof pools_v));
    pools_k[0] = (uint64_t)(uintptr_t)dk;
    pools_v[0] = (uint64_t)(uintptr_t)dv;
    CHECK(hipMemcpy(dk, hk, pool_elems * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dv, hv, pool_elems * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dbt, bt, sizeof bt, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dseq, SEQ, sizeof SEQ, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dprompt, PROMPT, sizeof PROMPT, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(drid, rid, sizeof rid, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dpass, pass_idx, sizeof pass_idx, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dpk, pools_k, sizeof pools_k, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dpv, pools_v, sizeof pools_v, hipMemcpyHostToDevice));
    CHECK(hipMemset(dstatus, 0, 4));
    CHECK(hipMemset(dkeep, 0xff, (size_t)HC * BUDGET * 4));

    bkv_cache cache;
    memset(&cache, 0, sizeof cache);
    cache.n_layers = L;
    cache.n_requests = R;
    cache.n_kv_heads = H;
    cache.head_dim = D;
    cache.block_size = BS;
    cache.num_blocks = NBLK;
    cache.max_blocks = MAXB;
    cache.k_pools = (const uint64_t*)dpk;
    cache.v_pools = (const uint64_t*)dpv;
    cache.block_table = (const int32_t*)dbt;
    cache.seq_len = (const int32_t*)dseq;
    cache.prompt_len = (const int32_t*)dprompt;

    bkv_pass_args a;
    memset(&a, 0, sizeof a);
    a.selector = BKV_SELECT_RANDOM;
    a.budget = BUDGET;
    a.score_stride = stride;
    a.seed = 99;
    a.request_ids = (const uint64_t*)drid;
    a.pass_idx = (const int32_t*)dpass;
    a.scores_out = dscores;
    a.keep_out = (int32_t*)dkeep;

    printf("abi %d\n", (int)bkv_abi_version());
    size_t ws_bytes = 0;
    int32_t rc = bkv_workspace_size(&cache, &a, &ws_bytes);
    if (rc != BKV_OK) {
        fprintf(stderr, "bkv_workspace_size: %s\n", bkv_status_string(rc));
        return 3;
    }
    printf("workspace %zu\n", ws_bytes);

    /* the draws and keep lists go to the caller's buffers above, so this pass
     * needs no workspace; asked for a workspace-backed score buffer it refuses
     * a missing one before enqueueing anything */
    bkv_pass_args b = a;
    b.scores_out = NULL;
    size_t need = 0;
    if (bkv_workspace_size(&cache, &b, &need) != BKV_OK || need == 0) return 4;
    rc = bkv_evict_pass(&cache, &b, NULL, 0, NULL, NULL);
    printf("refused %d %s\n", (int)rc, bkv_status_string(rc));

    void* ws = NULL;
    if (ws_bytes) CHECK(hipMalloc(&ws, ws_bytes));
    hipStream_t s;
    CHECK(hipStreamCreate(&s));
    rc = bkv_evict_pass(&cache, &a, ws, ws_bytes, (int32_t*)dstatus, (bkv_stream_t)s);
    CHECK(hipStreamSynchronize(s));
    int32_t status = -1;
    CHECK(hipMemcpy(&status, dstatus, 4, hipMemcpyDeviceToHost));
    printf("pass %d %d\n", (int)rc, (int)status);

    uint32_t* scores = malloc((size_t)HC * stride * 4);
    int32_t* keep = malloc((size_t)HC * BUDGET * 4);
    CHECK(hipMemcpy(scores, dscores, (size_t)HC * stride * 4, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(keep, dkeep, (size_t)HC * BUDGET * 4, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(hk, dk, pool_elems * 2, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(hv, dv, pool_elems * 2, hipMemcpyDeviceToHost));

    uint16_t* rows_k = malloc((size_t)MAXB * BS * D * 2);
    uint16_t* rows_v = malloc((size_t)MAXB * BS * D * 2);
    for (int hc = 0; hc < HC; ++hc) {
        const int r = (hc / H) % R, h = hc % H;
        int nk = 0;
        printf("hc %d keep", hc);
        for (int i = 0; i < BUDGET; ++i)
            if (keep[hc * BUDGET + i] >= 0) {
                printf(" %d", (int)keep[hc * BUDGET + i]);
                ++nk;
            }
        printf("\n");
        printf("hc %d draws %016llx\n", hc,
               (unsigned long long)fnv1a(scores + (size_t)hc * stride,
                                         (size_t)(SEQ[r] - PROMPT[r]) * 4));
        for (int i = 0; i < nk; ++i) {
            const size_t src = (((size_t)bt[r * MAXB + i / BS] * H + h) * BS + i % BS) * D;
            memcpy(rows_k + (size_t)i * D, hk + src, D * 2);
            memcpy(rows_v + (size_t)i * D, hv + src, D * 2);
        }
        printf("hc %d rows %016llx %016llx\n", hc,
               (unsigned long long)fnv1a(rows_k, (size_t)nk * D * 2),
               (unsigned long long)fnv1a(rows_v, (size_t)nk * D * 2));
    }
    return 0;
}
