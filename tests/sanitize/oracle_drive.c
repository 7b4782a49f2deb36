/* Drives every function of oracle/beacon_oracle.c once or more on small
 * inputs, including the degenerate cases (empty candidate sets, N <= B,
 * P = B, P > B refused, dead beacons, a forced index out of range, partial
 * last pages), with every buffer sized exactly as the function's contract
 * states.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize_cpu.py: an out-of-bounds access, a leak, a signed
 * overflow or a misaligned access aborts with a non-zero exit.  The checks
 * below are sanity checks on return values; the numerical pins of these
 * functions live in the Python tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_bf16_round(float f);
void oracle_beacon_update(int T, int G, int d, int K, const uint16_t* q, float* beacons,
                          int32_t* counts, int32_t* assign, int cap);
int oracle_beacon_update_forced(int T, int G, int d, int K, const uint16_t* q, float* beacons,
                                int32_t* counts, const int32_t* forced, double* gap, int cap);
void oracle_beacon_score(int N, int P, int d, int K, const uint16_t* keys, const float* beacons,
                         const int32_t* counts, int W, double bonus, double* scores, double* lse);
void oracle_philox4x64_10(const uint64_t* ctr_in, const uint64_t* key_in, uint64_t* out);
void oracle_random_score(uint64_t seed, uint64_t request_id, int32_t pass, int32_t layer,
                         int32_t head, int N, int P, uint32_t* out);
int oracle_topk_select(int N, int P, int B, const double* scores, int32_t* keep);
int oracle_shared_select(int H, int N, int P, int B, const double* scores, int32_t* keep);
int oracle_page_select(int n_rows, int N, int P, int B, int page, const double* scores,
                       int32_t* keep_pages);
int oracle_page_remap(int N, int page, const int32_t* block_row, int n_keep,
                      const int32_t* keep_pages, int32_t* new_row, int32_t* freed,
                      int32_t* n_freed);
void oracle_kv_compact(int n_keep, const int32_t* keep, int64_t row_bytes, const uint8_t* src,
                       uint8_t* dst);
void oracle_decode_attention(int N, int d, int G, const uint16_t* q, const uint16_t* keys,
                             const uint16_t* vals, double scale, double* out);
int oracle_num_threads(void);
int oracle_evict_batch(int H, int T, int G, int d, int K, int B, int W, double bonus, int Nmax,
                       const int32_t* N, const int32_t* P, const uint16_t* q, float* beacons,
                       int32_t* counts, const uint16_t* keys, const uint16_t* vals,
                       int32_t* keep, uint16_t* kout, uint16_t* vout);

enum { D = 128 };
static int failures = 0;
#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            failures++;                                                \
        }                                                              \
    } while (0)

/* splitmix64 (Steele, Lea, Flood 2014): seeded inputs only */
static uint64_t rng_state = 0x1234567u;
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float uniform_pm1(void) { return (float)((next_u64() >> 40) * 0x1p-23 - 1.0); }

/* exact-size heap buffers: ASan sees one element past the end */
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}
static uint16_t* bf16_rows(int rows) {
    uint16_t* p = xmalloc(sizeof(uint16_t) * (size_t)rows * D);
    for (size_t i = 0; i < (size_t)rows * D; ++i) p[i] = oracle_bf16_round(uniform_pm1());
    return p;
}
static double* doubles(int n) {
    double* p = xmalloc(sizeof(double) * (size_t)n);
    for (int i = 0; i < n; ++i) p[i] = (double)(next_u64() % 7) * 0.125;   /* many ties */
    return p;
}

static void maintenance(void) {
    const int T = 3, G = 2;
    for (int K = 1; K <= 9; K += 4) {
        for (int cap = 0; cap <= 2; cap += 2) {
            uint16_t* q = bf16_rows(T * G);
            float* b = xmalloc(sizeof(float) * (size_t)K * D);
            int32_t* c = xmalloc(sizeof(int32_t) * (size_t)K);
            int32_t* asg = xmalloc(sizeof(int32_t) * (size_t)(T * G));
            memset(b, 0, sizeof(float) * (size_t)K * D);
            memset(c, 0, sizeof(int32_t) * (size_t)K);
            oracle_beacon_update(T, G, D, K, q, b, c, asg, cap);
            for (int s = 0; s < T * G; ++s) CHECK(asg[s] >= 0 && asg[s] < K);
            oracle_beacon_update(T, G, D, K, q, b, c, NULL, cap);   /* assign nullable */
            /* teacher-forced replay of a valid sequence, then one that stops
             * at an index out of range */
            float* b2 = xmalloc(sizeof(float) * (size_t)K * D);
            int32_t* c2 = xmalloc(sizeof(int32_t) * (size_t)K);
            double* gap = xmalloc(sizeof(double) * (size_t)(T * G));
            memset(b2, 0, sizeof(float) * (size_t)K * D);
            memset(c2, 0, sizeof(int32_t) * (size_t)K);
            CHECK(oracle_beacon_update_forced(T, G, D, K, q, b2, c2, asg, gap, cap) == T * G);
            int32_t* bad = xmalloc(sizeof(int32_t) * (size_t)(T * G));
            for (int s = 0; s < T * G; ++s) bad[s] = s == 2 ? K : 0;
            CHECK(oracle_beacon_update_forced(T, G, D, K, q, b2, c2, bad, gap, cap) == 2);
            CHECK(isnan(gap[2]));
            free(q), free(b), free(c), free(asg), free(b2), free(c2), free(gap), free(bad);
        }
    }
    /* no queries */
    float b[D];
    int32_t c[1] = {0};
    oracle_beacon_update(0, 4, D, 1, NULL, b, c, NULL, 0);
    CHECK(c[0] == 0);
}

static void scoring(void) {
    const int K = 7;
    int32_t counts[7] = {3, 0, 1, 5, 0, 2, 9};   /* two dead beacons */
    float* b = xmalloc(sizeof(float) * K * D);
    for (int i = 0; i < K * D; ++i) b[i] = uniform_pm1();
    const int cases[][3] = {{0, 0, 4}, {1, 1, 0}, {37, 5, 64}, {48, 0, 8}, {20, 20, 3}};
    for (size_t t = 0; t < sizeof cases / sizeof cases[0]; ++t) {
        const int N = cases[t][0], P = cases[t][1], W = cases[t][2];
        uint16_t* keys = bf16_rows(N);
        double* sc = xmalloc(sizeof(double) * (size_t)(N - P));
        double* lse = xmalloc(sizeof(double) * K);
        oracle_beacon_score(N, P, D, K, keys, b, counts, W, 0.5, sc, lse);
        CHECK(isnan(lse[1]) && isnan(lse[4]));
        for (int n = 0; n < N - P; ++n) CHECK(sc[n] >= 0.0 && sc[n] <= 1.5);
        oracle_beacon_score(N, P, D, K, keys, b, counts, W, 0.5, sc, NULL);   /* lse nullable */
        free(keys), free(sc), free(lse);
    }
    /* no live beacon */
    int32_t dead[7] = {0};
    uint16_t* keys = bf16_rows(10);
    double sc[6];
    oracle_beacon_score(10, 4, D, K, keys, b, dead, 2, 1.0, sc, NULL);
    for (int n = 0; n < 6; ++n) CHECK(sc[n] == (n >= 4 ? 1.0 : 0.0));
    free(keys), free(b);
}

static void random_draws(void) {
    uint64_t ctr[4] = {0, 1, 2, 3}, key[2] = {5, 0}, out[4];
    oracle_philox4x64_10(ctr, key, out);
    for (int N = 0; N <= 9; N += 3) {
        uint32_t* d = xmalloc(sizeof(uint32_t) * (size_t)(N > 2 ? N - 2 : 0));
        oracle_random_score(7, 11, 3, 1, 2, N, N > 2 ? 2 : N, d);
        free(d);
    }
}

static void selection(void) {
    const int cases[][3] = {{40, 8, 16}, {10, 2, 16}, {30, 16, 16}, {30, 17, 16}, {0, 0, 4},
                            {33, 0, 1}};
    for (size_t t = 0; t < sizeof cases / sizeof cases[0]; ++t) {
        const int N = cases[t][0], P = cases[t][1], B = cases[t][2];
        double* sc = doubles(N - P);
        int32_t* keep = xmalloc(sizeof(int32_t) * (size_t)B);
        const int n = oracle_topk_select(N, P, B, sc, keep);
        CHECK(P > B ? n == -1 : n == (N < B ? N : B));
        for (int i = 1; i < n; ++i) CHECK(keep[i - 1] < keep[i]);
        double* sh = doubles(3 * (N - P));
        const int ns = oracle_shared_select(3, N, P, B, sh, keep);
        CHECK(P > B ? ns == -1 : ns == (N < B ? N : B));
        free(sc), free(sh), free(keep);
    }
}

static void pages(void) {
    const int page = 16;
    const int cases[][3] = {{100, 20, 64}, {40, 0, 64}, {130, 33, 48}, {70, 60, 48}, {5, 5, 16}};
    for (size_t t = 0; t < sizeof cases / sizeof cases[0]; ++t) {
        const int N = cases[t][0], P = cases[t][1], B = cases[t][2];
        const int npages = (N + page - 1) / page, Bp = B / page;
        double* sc = doubles(2 * (N - P));
        int32_t* kp = xmalloc(sizeof(int32_t) * (size_t)Bp);
        const int n = oracle_page_select(2, N, P, B, page, sc, kp);
        CHECK(n == -1 || (n >= 0 && n <= Bp && n <= npages));
        if (n >= 0) {
            int32_t* row = xmalloc(sizeof(int32_t) * (size_t)npages);
            int32_t* nrow = xmalloc(sizeof(int32_t) * (size_t)n);
            int32_t* freed = xmalloc(sizeof(int32_t) * (size_t)(npages - n));
            int32_t nf = -1;
            for (int j = 0; j < npages; ++j) row[j] = 100 + j;
            const int newN = oracle_page_remap(N, page, row, n, kp, nrow, freed, &nf);
            CHECK(nf == npages - n && newN <= N && newN <= n * page);
            free(row), free(nrow), free(freed);
        }
        free(sc), free(kp);
    }
}

static void compaction_and_attention(void) {
    uint16_t* src = bf16_rows(9);
    uint16_t* dst = xmalloc(sizeof(uint16_t) * 4 * D);
    const int32_t keep[4] = {0, 3, 4, 8};
    oracle_kv_compact(4, keep, (int64_t)D * 2, (const uint8_t*)src, (uint8_t*)dst);
    CHECK(memcmp(dst + 3 * D, src + 8 * D, D * 2) == 0);
    for (int N = 0; N <= 20; N += 10) {
        const int G = 3;
        uint16_t* q = bf16_rows(G);
        uint16_t* k = bf16_rows(N);
        uint16_t* v = bf16_rows(N);
        double* out = xmalloc(sizeof(double) * G * D);
        oracle_decode_attention(N, D, G, q, k, v, 1.0 / sqrt((double)D), out);
        if (N == 0) CHECK(out[0] == 0.0);
        free(q), free(k), free(v), free(out);
    }
    free(src), free(dst);
}

static void whole_batch(void) {
    enum { H = 5, T = 2, G = 2, K = 5, B = 24, W = 4, NMAX = 40 };
    const int32_t N[H] = {40, 17, 24, 30, 0};
    const int32_t P[H] = {8, 3, 24, 25, 0};   /* P > B refused on head 3 */
    uint16_t* q = bf16_rows(H * T * G);
    float* b = xmalloc(sizeof(float) * H * K * D);
    int32_t* c = xmalloc(sizeof(int32_t) * H * K);
    memset(b, 0, sizeof(float) * H * K * D);
    memset(c, 0, sizeof(int32_t) * H * K);
    uint16_t* keys = bf16_rows(H * NMAX);
    uint16_t* vals = bf16_rows(H * NMAX);
    int32_t* keep = xmalloc(sizeof(int32_t) * H * B);
    uint16_t* kout = xmalloc(sizeof(uint16_t) * H * B * D);
    uint16_t* vout = xmalloc(sizeof(uint16_t) * H * B * D);
    CHECK(oracle_evict_batch(H, T, G, D, K, B, W, 0.25, NMAX, N, P, q, b, c, keys, vals, keep,
                             kout, vout) == 1);
    free(q), free(b), free(c), free(keys), free(vals), free(keep), free(kout), free(vout);
}

int main(void) {
    CHECK(oracle_num_threads() >= 1);
    maintenance();
    scoring();
    random_draws();
    selection();
    pages();
    compaction_and_attention();
    whole_batch();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all calls clean\n");
    return 0;
}
