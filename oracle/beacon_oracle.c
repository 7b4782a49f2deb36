/*
 * beacon_oracle.c -- plain, slow CPU reference of the decode-time KV-cache
 * eviction pass (beacon maintenance, beacon scoring, Philox random scoring,
 * top-B selection with prompt protection, order-preserving compaction).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or constant table with the
 * HIP library; the two are written independently and compared.
 *
 * Sources it follows (pages are cited by title and section):
 *  - "BeaconKV: 用"信标查询"指导 KV cache 压缩" (papers.ananclaw.com explainer),
 *    section 3.2 (the beacon mechanism: nearest-beacon assignment of each new
 *    query, incremental beacon update) and section 3.3 (O(K) beacon state).
 *  - "BeaconKV" abstract (chatpaper.ai, English abstract): beacon queries are
 *    compact representatives of global query clusters.
 *  - "随机保留 KV Cache 竟不输精心设计的 eviction 策略?" (aiinking.com), the
 *    section "Random Attention: 不判断重要性, 只随机保留": prompt KV is always
 *    kept; generated KV is sampled independently per head and the top-K kept;
 *    one random draw plus one top-K per eviction.  Section "发现四" for the
 *    shared cache-compaction step; section "发现二" for the variant in which
 *    every head uses one common set of positions.
 *  - Where the pages leave a rule open, one plain reading is fixed and stated
 *    at each function (softmax-max beacon score with a recent-window bonus,
 *    online k-means running-mean update, cosine nearest beacon, Philox4x64-10).
 *  - Philox4x64-10 follows Salmon, Moraes, Dror, Shaw, "Parallel random
 *    numbers: as easy as 1, 2, 3", SC'11 (multiplier and Weyl constants as
 *    published there).
 *
 * Precision: every score/logit/cosine is computed in double from exactly
 * converted bf16 / fp32 inputs.  The beacon running-mean update is the one
 * place where the fixed reading pins fp32 arithmetic (IEEE single, round to
 * nearest even, no fused multiply-add): build with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* bf16 / fp32 conversions (own implementation)                        */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> exact value (bf16 is the top half of an fp32). */
static double bf16_value(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp32 -> bf16 with round-to-nearest-even on the 16 dropped bits
 * (finite inputs only; non-finite inputs are a precondition violation). */
static uint16_t bf16_round(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

uint16_t oracle_bf16_round(float f) { return bf16_round(f); }

/* ------------------------------------------------------------------ */
/* Beacon maintenance: nearest beacon by cosine, online k-means update */
/* ------------------------------------------------------------------ */

/* Cosine of x with beacon row b (both read exactly).  Zero norm on either
 * side gives cosine 0 (fixed reading for the degenerate case). */
static double cosine(const uint16_t* x, const float* b, int d) {
    double xx = 0.0, bb = 0.0, xb = 0.0;
    for (int i = 0; i < d; ++i) {
        double xi = bf16_value(x[i]);
        double bi = (double)b[i];
        xx += xi * xi;
        bb += bi * bi;
        xb += xi * bi;
    }
    if (xx == 0.0 || bb == 0.0) return 0.0;
    return xb / (sqrt(xx) * sqrt(bb));
}

/* The row a query goes to: the first never-filled beacon if one exists
 * (MacQueen initialisation: the first K observations seed the beacons in
 * order), else the beacon of highest cosine, ties to the lowest index. */
static int first_empty(const int32_t* counts, int K) {
    for (int j = 0; j < K; ++j)
        if (counts[j] == 0) return j;
    return -1;
}

static int nearest_beacon(const uint16_t* x, const float* beacons, int K, int d,
                          double* best_cos) {
    int best = 0;
    double bc = -INFINITY;
    for (int j = 0; j < K; ++j) {
        double c = cosine(x, beacons + (size_t)j * d, d);
        if (c > bc) {
            bc = c;
            best = j;
        }
    }
    if (best_cos) *best_cos = bc;
    return best;
}

/* Absorb observation x into beacon row j.  count 0 -> the row becomes x;
 * otherwise the running mean b += (x - b) / c with c the incremented count,
 * each operation an IEEE fp32 operation.  With a count cap C > 0 the
 * incremented count is clamped to C, so once a row has absorbed C
 * observations each new one moves it by 1/C of the difference: an
 * exponential moving average that keeps the beacon evolving during decoding
 * (BeaconKV explainer, section 3.2: beacons are not frozen, or early beacons
 * would be useless for late queries).  C = 0: no cap. */
static void absorb(const uint16_t* x, float* b, int32_t* count, int d, int cap) {
    if (*count == 0) {
        for (int i = 0; i < d; ++i) b[i] = (float)bf16_value(x[i]);
        *count = 1;
        return;
    }
    *count += 1;
    if (cap > 0 && *count > cap) *count = cap;
    const float cf = (float)(*count);
    for (int i = 0; i < d; ++i) {
        float xi = (float)bf16_value(x[i]);
        float diff = xi - b[i];
        float step = diff / cf;
        b[i] = b[i] + step;
    }
}

/* Process the T*G buffered decode queries q[T][G][d] in (t, g) order. */
void oracle_beacon_update(int T, int G, int d, int K, const uint16_t* q,
                          float* beacons, int32_t* counts, int32_t* assign, int cap) {
    for (int s = 0; s < T * G; ++s) {
        const uint16_t* x = q + (size_t)s * d;
        int j = first_empty(counts, K);
        if (j < 0) j = nearest_beacon(x, beacons, K, d, NULL);
        absorb(x, beacons + (size_t)j * d, counts + j, d, cap);
        if (assign) assign[s] = j;
    }
}

/* Teacher-forced replay: apply the given assignment sequence instead of the
 * oracle's own argmax, and report for every step how far the forced row is
 * from the best cosine (gap >= 0; 0 means it is an exact argmax).  A forced
 * row that contradicts the empty-slot rule gets gap = +inf; an index out of
 * range gets gap = NaN and stops the replay.  Returns the number of steps
 * replayed. */
int oracle_beacon_update_forced(int T, int G, int d, int K, const uint16_t* q,
                                float* beacons, int32_t* counts,
                                const int32_t* forced, double* gap, int cap) {
    for (int s = 0; s < T * G; ++s) {
        const uint16_t* x = q + (size_t)s * d;
        int f = forced[s];
        if (f < 0 || f >= K) {
            gap[s] = NAN;
            return s;
        }
        int e = first_empty(counts, K);
        if (e >= 0) {
            gap[s] = (f == e) ? 0.0 : INFINITY;
        } else {
            double best;
            (void)nearest_beacon(x, beacons, K, d, &best);
            double cf = cosine(x, beacons + (size_t)f * d, d);
            gap[s] = best - cf;
        }
        absorb(x, beacons + (size_t)f * d, counts + f, d, cap);
    }
    return T * G;
}

/* ------------------------------------------------------------------ */
/* Beacon scoring                                                      */
/* ------------------------------------------------------------------ */

/* keys[N][d] bf16 (one head-cache, slot order); beacons[K][d] fp32,
 * counts[K].  Live beacons J = {j : counts[j] > 0} are rounded to bf16 for
 * the contraction.  For j in J:
 *     s_jn   = (bf16(b_j) . k_n) / sqrt(d)          n in [0, N)
 *     lse_j  = log sum_n exp(s_jn)                  (all N slots)
 * and for n in [P, N):
 *     sigma(n) = max_{j in J} exp(s_jn - lse_j)     (0 when J is empty)
 *     score(n) = sigma(n) + bonus * [n >= N - W].
 * scores[] receives N - P values (index n - P); lse[] receives K values
 * (NaN for beacons outside J). */
void oracle_beacon_score(int N, int P, int d, int K, const uint16_t* keys,
                         const float* beacons, const int32_t* counts, int W,
                         double bonus, double* scores, double* lse) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double* bh = (double*)malloc(sizeof(double) * (size_t)d);
    double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* sigma = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    for (int n = 0; n < N; ++n) sigma[n] = 0.0;

    for (int j = 0; j < K; ++j) {
        if (counts[j] <= 0) {
            if (lse) lse[j] = NAN;
            continue;
        }
        for (int i = 0; i < d; ++i)
            bh[i] = bf16_value(bf16_round(beacons[(size_t)j * d + i]));
        double m = -INFINITY;
        for (int n = 0; n < N; ++n) {
            const uint16_t* k = keys + (size_t)n * d;
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += bh[i] * bf16_value(k[i]);
            s[n] = acc * inv_sqrt_d;
            if (s[n] > m) m = s[n];
        }
        /* log-sum-exp, evaluated around the maximum so no term overflows */
        double sum = 0.0;
        for (int n = 0; n < N; ++n) sum += exp(s[n] - m);
        double l = (N > 0) ? m + log(sum) : -INFINITY;
        if (lse) lse[j] = l;
        for (int n = 0; n < N; ++n) {
            double p = exp(s[n] - l);
            if (p > sigma[n]) sigma[n] = p;
        }
    }
    for (int n = P; n < N; ++n)
        scores[n - P] = sigma[n] + ((n >= N - W) ? bonus : 0.0);
    free(bh);
    free(s);
    free(sigma);
}

/* ------------------------------------------------------------------ */
/* Philox4x64-10 and the random selector's scores                      */
/* ------------------------------------------------------------------ */

static void mul_hi_lo(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *lo = (uint64_t)p;
    *hi = (uint64_t)(p >> 64);
}

/* Ten rounds; the key is bumped by the Weyl constants before every round
 * after the first. */
void oracle_philox4x64_10(const uint64_t* ctr_in, const uint64_t* key_in,
                          uint64_t* out) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t hi0, lo0, hi1, lo1;
        mul_hi_lo(M0, x0, &hi0, &lo0);
        mul_hi_lo(M1, x2, &hi1, &lo1);
        uint64_t y0 = hi1 ^ x1 ^ k0;
        uint64_t y1 = lo1;
        uint64_t y2 = hi0 ^ x3 ^ k1;
        uint64_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Random-selector score of slot n in [P, N) of one head-cache: the high 32
 * bits of output word (n mod 4) of Philox4x64-10 with
 *   counter = (n div 4, pass, (layer << 32) | head, request_id)
 *   key     = (seed, 0).
 * Every eviction pass has a fresh pass index, so every pass draws anew. */
void oracle_random_score(uint64_t seed, uint64_t request_id, int32_t pass,
                         int32_t layer, int32_t head, int N, int P,
                         uint32_t* out) {
    uint64_t key[2] = {seed, 0};
    for (int n = P; n < N; ++n) {
        uint64_t ctr[4] = {(uint64_t)(n / 4), (uint64_t)(uint32_t)pass,
                           ((uint64_t)(uint32_t)layer << 32) | (uint64_t)(uint32_t)head,
                           request_id};
        uint64_t w[4];
        oracle_philox4x64_10(ctr, key, w);
        out[n - P] = (uint32_t)(w[n % 4] >> 32);
    }
}

/* ------------------------------------------------------------------ */
/* Top-B selection with full prompt protection                         */
/* ------------------------------------------------------------------ */

typedef struct {
    double score;
    int32_t slot;
} cand_t;

/* Higher score first; equal scores: lower slot (earlier position) first. */
static int cand_order(const void* a, const void* b) {
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->slot < y->slot) ? -1 : (x->slot > y->slot);
}

/* Budget B counts the prompt.  P > B (or bad lengths) -> -1.  N <= B -> all
 * N slots kept.  Otherwise the prompt [0, P) plus the best B - P of [P, N);
 * the kept slots are written in ascending order.  Returns the kept count. */
int oracle_topk_select(int N, int P, int B, const double* scores, int32_t* keep) {
    if (P < 0 || N < P || B < 0 || P > B) return -1;
    if (N <= B) {
        for (int n = 0; n < N; ++n) keep[n] = n;
        return N;
    }
    int m = N - P;
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)m);
    unsigned char* kept = (unsigned char*)calloc((size_t)N, 1);
    for (int i = 0; i < m; ++i) {
        c[i].score = scores[i];
        c[i].slot = P + i;
    }
    qsort(c, (size_t)m, sizeof(cand_t), cand_order);
    for (int n = 0; n < P; ++n) kept[n] = 1;
    for (int i = 0; i < B - P; ++i) kept[c[i].slot] = 1;
    int o = 0;
    for (int n = 0; n < N; ++n)
        if (kept[n]) keep[o++] = n;
    free(c);
    free(kept);
    return o;
}

/* Shared positions (Random Attention article, section "发现二": forcing all
 * heads onto one common set of positions leaves accuracy almost unchanged).
 * One selection serves the H KV heads of one (layer, request).  Reading taken
 * here: a candidate's merged score is the largest of its H per-head scores,
 * and the prompt-protected top-B above runs once on the merged scores.  For
 * the random selector the heads share one draw (H = 1 here, the draw of head
 * 0).  scores is [H][N - P] row-major; keep as for oracle_topk_select. */
int oracle_shared_select(int H, int N, int P, int B, const double* scores, int32_t* keep) {
    if (H < 1 || P < 0 || N < P) return -1;
    const int m = N - P;
    double* merged = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    for (int i = 0; i < m; ++i) {
        double best = scores[i];
        for (int h = 1; h < H; ++h)
            if (scores[(size_t)h * m + i] > best) best = scores[(size_t)h * m + i];
        merged[i] = best;
    }
    int n = oracle_topk_select(N, P, B, merged, keep);
    free(merged);
    return n;
}

/* Page retention (Random Attention article, section "发现二": keeping
 * contiguous blocks of 1 to 64 tokens instead of scattered tokens leaves
 * accuracy almost unchanged, and so does forcing all heads onto one common
 * set of positions).  Reading taken here: the retained unit is a whole cache
 * page of `page` slots, chosen once per request for every layer and head, so
 * the cache shrinks by dropping pages from the request's block table.
 *   - page j covers slots [j*page, min((j+1)*page, N)); npages = ceil(N/page);
 *   - pages holding a prompt slot (j*page < P) and a partial last page
 *     (N mod page != 0) are always kept;
 *   - a page's score is the largest score of any of its candidate slots in
 *     any of the n_rows score rows of the request;
 *   - Bp = B / page pages survive: the forced pages plus the best remaining
 *     pages by (score descending, page ascending); npages <= Bp keeps all;
 *     forced pages > Bp is refused (-1).
 * scores is [n_rows][N - P] row-major.  keep_pages receives the kept page
 * indices in ascending order; returns their count. */
int oracle_page_select(int n_rows, int N, int P, int B, int page, const double* scores,
                       int32_t* keep_pages) {
    if (n_rows < 1 || page < 1 || P < 0 || N < P || B < 0) return -1;
    const int m = N - P;
    const int npages = (N + page - 1) / page;
    const int Bp = B / page;
    if (npages <= Bp) {
        for (int j = 0; j < npages; ++j) keep_pages[j] = j;
        return npages;
    }
    unsigned char* forced = (unsigned char*)calloc((size_t)(npages ? npages : 1), 1);
    int n_forced = 0;
    for (int j = 0; j < npages; ++j) {
        const int last_partial = (j == npages - 1) && (N % page != 0);
        if ((long)j * page < P || last_partial) {
            forced[j] = 1;
            ++n_forced;
        }
    }
    if (n_forced > Bp) {
        free(forced);
        return -1;
    }
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)npages);
    int nc = 0;
    for (int j = 0; j < npages; ++j) {
        if (forced[j]) continue;
        double best = -INFINITY;
        for (int n = j * page; n < (j + 1) * page && n < N; ++n)
            for (int r = 0; r < n_rows; ++r) {
                const double v = scores[(size_t)r * m + (n - P)];
                if (v > best) best = v;
            }
        c[nc].score = best;
        c[nc].slot = j;
        ++nc;
    }
    qsort(c, (size_t)nc, sizeof(cand_t), cand_order);
    unsigned char* kept = forced;  /* forced pages, then the best candidates */
    for (int i = 0; i < Bp - n_forced; ++i) kept[c[i].slot] = 1;
    int o = 0;
    for (int j = 0; j < npages; ++j)
        if (kept[j]) keep_pages[o++] = j;
    free(c);
    free(forced);
    return o;
}

/* The block-table rewrite that page retention replaces compaction with: the
 * kept pages' blocks move to the front in page order, the dropped pages'
 * blocks are released (ascending page order), and the new length counts the
 * valid slots of the kept pages.  Returns the new N. */
int oracle_page_remap(int N, int page, const int32_t* block_row, int n_keep,
                      const int32_t* keep_pages, int32_t* new_row, int32_t* freed,
                      int32_t* n_freed) {
    const int npages = (N + page - 1) / page;
    unsigned char* kept = (unsigned char*)calloc((size_t)(npages ? npages : 1), 1);
    int new_n = 0;
    for (int i = 0; i < n_keep; ++i) {
        const int j = keep_pages[i];
        kept[j] = 1;
        new_row[i] = block_row[j];
        new_n += ((j + 1) * page <= N) ? page : N - j * page;
    }
    int f = 0;
    for (int j = 0; j < npages; ++j)
        if (!kept[j]) freed[f++] = block_row[j];
    *n_freed = f;
    free(kept);
    return new_n;
}

/* ------------------------------------------------------------------ */
/* Compaction                                                          */
/* ------------------------------------------------------------------ */

/* Out-of-place gather: dst row i = src row keep[i], rows of row_bytes. */
void oracle_kv_compact(int n_keep, const int32_t* keep, int64_t row_bytes,
                       const uint8_t* src, uint8_t* dst) {
    for (int i = 0; i < n_keep; ++i)
        memcpy(dst + (size_t)i * row_bytes, src + (size_t)keep[i] * row_bytes,
               (size_t)row_bytes);
}

/* ------------------------------------------------------------------ */
/* Decode attention over a compacted head-cache                        */
/* ------------------------------------------------------------------ */

/* The step after the pass (Random Attention article, section "发现四": every
 * selector shares the same attention kernels over the compacted paged
 * cache).  For each of the G query heads of one KV head, single-query softmax
 * attention over the N cached rows:
 *   s_n = scale * (q . k_n),  p_n = exp(s_n - max s) / sum exp(s - max s),
 *   out = sum_n p_n v_n.
 * Slot order and positions play no part (the keys were stored with their
 * positions already applied), so a compacted cache is attended as is.
 * q[G][d], keys/vals[N][d] bf16 bits; out[G][d] in double.  N = 0 gives 0. */
void oracle_decode_attention(int N, int d, int G, const uint16_t* q, const uint16_t* keys,
                             const uint16_t* vals, double scale, double* out) {
    double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    for (int g = 0; g < G; ++g) {
        double* o = out + (size_t)g * d;
        for (int j = 0; j < d; ++j) o[j] = 0.0;
        if (N == 0) continue;
        double mx = -INFINITY;
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += bf16_value(q[(size_t)g * d + j]) * bf16_value(keys[(size_t)n * d + j]);
            s[n] = scale * acc;
            if (s[n] > mx) mx = s[n];
        }
        double z = 0.0;
        for (int n = 0; n < N; ++n) {
            s[n] = exp(s[n] - mx);
            z += s[n];
        }
        for (int n = 0; n < N; ++n)
            for (int j = 0; j < d; ++j) o[j] += (s[n] / z) * bf16_value(vals[(size_t)n * d + j]);
    }
    free(s);
}

/* ------------------------------------------------------------------ */
/* Whole pass over many independent head-caches (CPU baseline)         */
/* ------------------------------------------------------------------ */

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One beacon eviction pass per head-cache, head-caches in parallel.
 * Dense per-head inputs: q[H][T][G][d], beacons[H][K][d], counts[H][K],
 * keys/vals[H][N][d] (bf16 bits), lengths N[H], P[H].  Outputs: beacons and
 * counts updated in place, keep[H][B], kout/vout[H][B][d] (compacted rows;
 * rows past the kept count are left untouched).  Returns the number of
 * head-caches whose selection failed (P > B). */
int oracle_evict_batch(int H, int T, int G, int d, int K, int B, int W,
                       double bonus, int Nmax, const int32_t* N, const int32_t* P,
                       const uint16_t* q, float* beacons, int32_t* counts,
                       const uint16_t* keys, const uint16_t* vals,
                       int32_t* keep, uint16_t* kout, uint16_t* vout) {
    int failures = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : failures)
    for (int h = 0; h < H; ++h) {
        const int n = N[h], p = P[h];
        float* bh = beacons + (size_t)h * K * d;
        int32_t* ch = counts + (size_t)h * K;
        oracle_beacon_update(T, G, d, K, q + (size_t)h * T * G * d, bh, ch, NULL, 0);
        double* sc = (double*)malloc(sizeof(double) * (size_t)(n - p > 0 ? n - p : 1));
        oracle_beacon_score(n, p, d, K, keys + (size_t)h * Nmax * d, bh, ch, W,
                            bonus, sc, NULL);
        int32_t* kh = keep + (size_t)h * B;
        int nk = oracle_topk_select(n, p, B, sc, kh);
        if (nk < 0) {
            failures += 1;
        } else {
            oracle_kv_compact(nk, kh, (int64_t)d * 2,
                              (const uint8_t*)(keys + (size_t)h * Nmax * d),
                              (uint8_t*)(kout + (size_t)h * B * d));
            oracle_kv_compact(nk, kh, (int64_t)d * 2,
                              (const uint8_t*)(vals + (size_t)h * Nmax * d),
                              (uint8_t*)(vout + (size_t)h * B * d));
        }
        free(sc);
    }
    return failures;
}
