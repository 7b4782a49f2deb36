/* Drives the host side of libbeaconkv's C ABI without a GPU: argument
 * validation of every entry point, bkv_workspace_size over the whole range
 * of cache shapes (including ones whose buffer sizes would overflow 32-bit
 * or 64-bit arithmetic), and the status strings.  Device pointers are fake
 * addresses that validation rejects before anything is launched, so no
 * kernel runs.  Built by tests/test_sanitize_cpu.py from host-only objects
 * of the library sources with AddressSanitizer and UndefinedBehaviorSanitizer:
 * an out-of-bounds access, a signed overflow or a shift out of range in the
 * shell aborts with a non-zero exit. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "beaconkv.h"

static int failures = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);  \
            failures++;                                                      \
        }                                                                    \
    } while (0)

#define FAKE ((void*)(uintptr_t)0x100000)
#define FAKE_AT(off) ((void*)(uintptr_t)(0x100000 + (off)))

static bkv_cache cache(int L, int R, int H, int max_blocks, int64_t num_blocks) {
    bkv_cache c;
    memset(&c, 0, sizeof c);
    c.n_layers = L;
    c.n_requests = R;
    c.n_kv_heads = H;
    c.head_dim = 128;
    c.block_size = 16;
    c.max_blocks = max_blocks;
    c.num_blocks = num_blocks;
    c.k_pools = c.v_pools = FAKE;
    c.block_table = c.seq_len = c.prompt_len = FAKE;
    return c;
}

static void status_strings(void) {
    CHECK(bkv_abi_version() == BKV_ABI_VERSION);
    for (int code = -3; code < 40; ++code) {
        const char* s = bkv_status_string(code);
        CHECK(s != NULL && strlen(s) > 0);
    }
    CHECK(bkv_status_string(INT32_MIN) != NULL && bkv_status_string(INT32_MAX) != NULL);
}

static void entry_validation(void) {
    bkv_cache c = cache(2, 3, 8, 10, 30);
    /* maintenance */
    CHECK(bkv_beacon_update(4, 8, 2, 64, 16, FAKE, FAKE, FAKE, NULL, 0, NULL) ==
          BKV_ERR_UNSUPPORTED);
    CHECK(bkv_beacon_update(4, 8, 2, 128, 257, FAKE, FAKE, FAKE, NULL, 0, NULL) ==
          BKV_ERR_INVALID);
    CHECK(bkv_beacon_update(INT32_MAX, INT32_MAX, 8, 128, 256, FAKE, FAKE, FAKE, NULL, 0,
                            NULL) == BKV_ERR_INVALID);
    CHECK(bkv_beacon_update(4, 8, 2, 128, 16, NULL, FAKE, FAKE, NULL, 0, NULL) == BKV_ERR_NULL);
    CHECK(bkv_beacon_update(0, 8, 2, 128, 16, NULL, NULL, NULL, NULL, 0, NULL) == BKV_OK);
    /* scoring */
    CHECK(bkv_beacon_score(NULL, FAKE, FAKE, 8, 64, 1.0f, FAKE, 16, NULL, NULL, NULL) ==
          BKV_ERR_NULL);
    CHECK(bkv_beacon_score(&c, FAKE, FAKE, 0, 64, 1.0f, FAKE, 160, NULL, NULL, NULL) ==
          BKV_ERR_INVALID);
    CHECK(bkv_beacon_score(&c, FAKE, FAKE, 64, -1, 1.0f, FAKE, 160, NULL, NULL, NULL) ==
          BKV_ERR_INVALID);
    CHECK(bkv_beacon_score(&c, FAKE_AT(8), FAKE, 64, 64, 1.0f, FAKE, 160, NULL, NULL, NULL) ==
          BKV_ERR_INVALID);
    bkv_cache huge = cache(1 << 16, 1 << 12, 8, 10, 30);
    CHECK(bkv_beacon_score(&huge, FAKE, FAKE, 64, 64, 1.0f, FAKE, 160, NULL, NULL, NULL) ==
          BKV_ERR_INVALID);
    bkv_cache extreme = cache(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, INT64_MAX);
    CHECK(bkv_beacon_score(&extreme, FAKE, FAKE, 64, 64, 1.0f, FAKE, INT32_MAX, NULL, NULL,
                           NULL) == BKV_ERR_INVALID);
    /* random draws, selection, compaction */
    CHECK(bkv_random_score(&c, 1, NULL, FAKE, 0, FAKE, 160, NULL, NULL) == BKV_ERR_NULL);
    CHECK(bkv_random_score(&c, 1, FAKE, FAKE, 3, FAKE, 160, NULL, NULL) == BKV_ERR_INVALID);
    CHECK(bkv_topk_select(&c, FAKE, 7, 160, 64, FAKE, NULL, NULL) == BKV_ERR_INVALID);
    CHECK(bkv_topk_select(&c, FAKE, 0, INT32_MAX, INT32_MAX, FAKE, NULL, NULL) ==
          BKV_ERR_INVALID);
    CHECK(bkv_topk_select_shared(&c, FAKE, 0, 160, 9, 64, FAKE, NULL, NULL) == BKV_ERR_INVALID);
    CHECK(bkv_topk_select_shared(NULL, FAKE, 0, 160, 8, 64, FAKE, NULL, NULL) == BKV_ERR_NULL);
    CHECK(bkv_kv_compact(&c, FAKE, 0, 0, NULL, 0, NULL, NULL) == BKV_ERR_INVALID);
    CHECK(bkv_kv_compact(&c, FAKE, 64, 0, FAKE, 100, NULL, NULL) == BKV_ERR_INVALID);
    CHECK(bkv_kv_compact(&c, FAKE, INT32_MAX, 0, FAKE, 159, NULL, NULL) == BKV_ERR_INVALID);
    /* page retention, decode attention */
    CHECK(bkv_page_retain(&c, FAKE, 0, 160, BKV_ROWS_PER_HEAD, 40, FAKE, FAKE, FAKE, FAKE, NULL,
                          NULL) == BKV_ERR_INVALID);
    CHECK(bkv_page_retain(&c, FAKE, 0, 160, BKV_ROWS_PER_HEAD, 64, FAKE, NULL, FAKE, FAKE, NULL,
                          NULL) == BKV_ERR_NULL);
    CHECK(bkv_decode_attention(&c, FAKE, 9, 0.1f, FAKE, NULL, NULL) == BKV_ERR_INVALID);
    CHECK(bkv_decode_attention(&c, FAKE, 4, 0.1f, FAKE_AT(4), NULL, NULL) == BKV_ERR_INVALID);
}

/* bkv_workspace_size either refuses a shape or returns a size at least the
 * score buffer it must hold; never a wrapped-around small number. */
static void workspace_sizes(void) {
    const int Ls[] = {1, 36, 64, 4096, 1 << 16, INT32_MAX};
    const int Rs[] = {1, 128, 4096, 1 << 20, INT32_MAX};
    const int Hs[] = {1, 8, 64, INT32_MAX};
    const int MBs[] = {1, 136, 2048, 2049, INT32_MAX};
    const int Bs[] = {16, 2048, 15872, 32768, INT32_MAX - 15};
    int refused = 0, sized = 0;
    for (size_t a = 0; a < sizeof Ls / sizeof *Ls; ++a)
        for (size_t b = 0; b < sizeof Rs / sizeof *Rs; ++b)
            for (size_t h = 0; h < sizeof Hs / sizeof *Hs; ++h)
                for (size_t m = 0; m < sizeof MBs / sizeof *MBs; ++m)
                    for (size_t k = 0; k < sizeof Bs / sizeof *Bs; ++k)
                        for (int sel = 0; sel < 2; ++sel)
                            for (int mode = 0; mode < 4; ++mode) {
                                bkv_cache c = cache(Ls[a], Rs[b], Hs[h], MBs[m], 1 << 20);
                                bkv_pass_args p;
                                memset(&p, 0, sizeof p);
                                p.selector = sel;
                                p.budget = Bs[k];
                                p.shared_positions = mode == 1;
                                p.page_retention = mode == 2;
                                p.separate_steps = mode == 3;
                                size_t bytes = 0;
                                const int32_t rc = bkv_workspace_size(&c, &p, &bytes);
                                if (rc != BKV_OK) {
                                    CHECK(rc == BKV_ERR_INVALID);
                                    refused++;
                                    continue;
                                }
                                sized++;
                                /* at least one score row of max_blocks * 16 entries */
                                CHECK(bytes >= (size_t)MBs[m] * 16 * 4);
                                const unsigned __int128 rows =
                                    (unsigned __int128)Ls[a] * (unsigned __int128)Rs[b];
                                CHECK(rows * (unsigned __int128)MBs[m] * 64 >= (mode == 2 ? 0 : 1));
                            }
    CHECK(refused > 0 && sized > 0);
    /* the pass and its allocation-free variant refuse before any HIP call */
    bkv_cache c = cache(64, 512, 8, 128, 1 << 20);
    bkv_pass_args p;
    memset(&p, 0, sizeof p);
    p.selector = BKV_SELECT_RANDOM;
    p.budget = 64;
    p.request_ids = FAKE;
    p.pass_idx = FAKE;
    CHECK(bkv_evict_pass_noalloc(&c, &p, NULL, NULL) == BKV_ERR_SCRATCH);
    CHECK(bkv_evict_pass(&c, &p, NULL, 0, NULL, NULL) == BKV_ERR_WORKSPACE);
    p.selector = 5;
    CHECK(bkv_evict_pass(&c, &p, FAKE, (size_t)1 << 40, NULL, NULL) == BKV_ERR_INVALID);
    CHECK(bkv_evict_pass_noalloc(NULL, &p, NULL, NULL) == BKV_ERR_NULL);
}

int main(void) {
    status_strings();
    entry_validation();
    workspace_sizes();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ABI driver: all calls clean\n");
    return 0;
}
