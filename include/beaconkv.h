/*
 * beaconkv.h -- C ABI of libbeaconkv.so: the decode-time KV-cache eviction
 * pass (beacon maintenance, beacon scoring, random scoring, top-B selection,
 * order-preserving compaction) as hand-written HIP kernels for MI355X
 * (gfx950, CDNA4), with its variants (a count cap on the beacon update, one
 * selection shared by the heads of a layer, whole-page retention through the
 * block table) and the decode attention that consumes the compacted cache.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller (for example
 *    the storage of torch tensors).  The library never allocates or frees
 *    memory.  Its one piece of global state is the scratch array of
 *    bkv_evict_pass_noalloc (one copy per GPU); every other call is
 *    reentrant.
 *  - Work is enqueued asynchronously on the caller's HIP stream (`stream`,
 *    a hipStream_t; NULL means the legacy default stream).  Outputs are valid
 *    once that stream has been synchronised.
 *  - Return value: BKV_OK, or a host-detected error code.  A host-detected
 *    error enqueues nothing (atomic failure: no buffer is touched).
 *  - `status` (nullable) is a caller-zeroed device int32.  Kernels OR the bit
 *    (1 << code) into it for every error they detect from device-resident data
 *    (lengths, block ids, keep lists).  A head-cache whose request fails such a
 *    check is left untouched by that kernel (and, inside bkv_evict_pass, by
 *    every kernel of the pass).
 *  - Head-cache order: hc = (layer * n_requests + request) * n_kv_heads + head,
 *    HC = n_layers * n_requests * n_kv_heads.  Per-head-cache arrays are
 *    indexed [hc][...].
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - Only head_dim == 128 and block_size == 16 are supported.
 *
 * The method (pages cited by title and section):
 *  - BeaconKV explainer ("BeaconKV: 用"信标查询"指导 KV cache 压缩",
 *    papers.ananclaw.com), section 3.2: each new decode query is assigned to
 *    its nearest beacon and the beacons are updated incrementally; section
 *    3.3: the beacon state is O(K), not O(sequence).
 *  - BeaconKV abstract (chatpaper.ai): beacons are compact representatives of
 *    global query clusters, used to anticipate which KV pairs are revisited.
 *  - Random Attention article ("随机保留 KV Cache 竟不输精心设计的 eviction
 *    策略?", aiinking.com), section "Random Attention: 不判断重要性, 只随机保留":
 *    the prompt's KV is always kept, the generated KV is sampled independently
 *    per head and the top-K kept, at the cost of one random draw and one
 *    top-K; section "发现四": every selector ends in the same cache compaction,
 *    run for a batch of requests at a synchronized point every 64 tokens, and
 *    shares the attention kernels; section "发现二": contiguous blocks instead
 *    of scattered tokens, and one common set of positions for all heads, both
 *    leave accuracy almost unchanged.
 *  Rules the pages leave open are fixed as follows (see each function):
 *  cosine nearest beacon with ties to the lowest row, MacQueen fill of empty
 *  rows, fp32 running-mean update; score(n) = max over live beacons of the
 *  softmax over all N slots of bf16(b)·k/sqrt(d), plus `bonus` on the last
 *  `window` slots; budget B includes the prompt; ties go to the earlier slot;
 *  Philox4x64-10 (Salmon et al., SC'11) for the random selector.
 */
#ifndef BEACONKV_H
#define BEACONKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BKV_ABI_VERSION 8

typedef void* bkv_stream_t; /* hipStream_t */

/* Return / status codes.  Device-detected codes appear in *status as bits. */
enum {
    BKV_OK = 0,
    BKV_ERR_NULL = 1,        /* a required pointer is NULL */
    BKV_ERR_INVALID = 2,     /* bad size, count, stride or alignment; or (device) a keep
                                list that is not strictly ascending inside [0, N) */
    BKV_ERR_BUDGET = 3,      /* (device) a request's prompt length exceeds the budget */
    BKV_ERR_UNSUPPORTED = 4, /* head_dim != 128 or block_size != 16 */
    BKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than bkv_workspace_size */
    BKV_ERR_HIP = 6,         /* a HIP launch failed (hipGetLastError) */
    BKV_ERR_LENGTH = 7,      /* (device) seq_len / prompt_len out of range */
    BKV_ERR_BLOCK_TABLE = 8, /* (device) a block id outside [0, num_blocks) */
    BKV_ERR_SCRATCH = 9,     /* bkv_evict_pass_noalloc: the pass needs more than
                                BKV_NOALLOC_SCRATCH_BYTES of scratch */
};

enum { BKV_SCORE_F32 = 0, BKV_SCORE_U32 = 1 };           /* score buffer element type */
enum { BKV_SELECT_BEACON = 0, BKV_SELECT_RANDOM = 1 };   /* selector of bkv_evict_pass */
/* Row layout of a score buffer: one row per head-cache (hc), per (layer,
 * request) (row layer * n_requests + r), or per request (row r). */
enum { BKV_ROWS_PER_HEAD = 0, BKV_ROWS_PER_LAYER_REQUEST = 1, BKV_ROWS_PER_REQUEST = 2 };
/* bkv_pass_args.page_retention */
enum { BKV_PAGES_OFF = 0, BKV_PAGES_PER_REQUEST = 1, BKV_PAGES_PER_HEAD = 2 };

#define BKV_MAX_BEACONS 256
#define BKV_MAX_CANDIDATES 32768 /* largest score_stride bkv_topk_select accepts */
#define BKV_MAX_QUERY_HEADS 8     /* largest G bkv_decode_attention accepts */
/* Largest score_stride + budget for which bkv_evict_pass fuses scoring,
 * selection and compaction (the candidate keys and keep list of a head-cache
 * then fit in the scoring kernel's LDS). */
#define BKV_FUSED_MAX_ENTRIES 15872
/* Bytes of the scratch array bkv_evict_pass_noalloc holds on each GPU
 * (256 MiB). */
#define BKV_NOALLOC_SCRATCH_BYTES 268435456

/* A paged bf16 KV cache (vLLM-style pools, one K and one V pool per layer).
 * Layer pool l holds bf16 [num_blocks][n_kv_heads][block_size][head_dim];
 * slot n of request r, head h lives in block block_table[r][n / block_size]
 * at row n % block_size.  A dense cache is an identity block table.  Every
 * pool address must be 16-byte aligned.  A request holds at most
 * max_blocks * block_size <= 32768 slots (the kernels stage a request's block
 * table in LDS); n_layers * n_requests * n_kv_heads and num_blocks must fit
 * in int32.  Violations return BKV_ERR_INVALID before anything is enqueued.
 *
 * Per-head page tables (head_block_table and head_seq_len, both set or both
 * NULL; bkv_page_retain_heads writes them): head-cache
 * hc = (layer * n_requests + r) * n_kv_heads + h then reads its slots through
 * row hc of head_block_table and has head_seq_len[hc] of them, in place of
 * the request's block_table row and seq_len (prompt_len stays per request).
 * The kernels then check each head-cache's own row and length, so a bad
 * block id or length skips that head-cache only.  Selections shared by the
 * heads of a request (bkv_topk_select_shared, shared keep lists of
 * bkv_kv_compact, bkv_page_retain, draw rows per (layer, request) or per
 * request, shared_positions in a pass) are refused with BKV_ERR_INVALID on
 * such a cache. */
typedef struct bkv_cache {
    int32_t n_layers;
    int32_t n_requests;
    int32_t n_kv_heads;
    int32_t head_dim;             /* must be 128 */
    int32_t block_size;           /* must be 16 */
    int32_t max_blocks;           /* columns of block_table */
    int64_t num_blocks;           /* physical blocks in every layer pool */
    const uint64_t* k_pools;      /* device [n_layers] device addresses of K pools */
    const uint64_t* v_pools;      /* device [n_layers] device addresses of V pools */
    const int32_t* block_table;   /* device [n_requests][max_blocks] */
    const int32_t* seq_len;       /* device [n_requests] N: valid slots [0, N) */
    const int32_t* prompt_len;    /* device [n_requests] P: prompt slots [0, P) */
    const int32_t* head_block_table; /* nullable device [n_layers][n_requests][n_kv_heads]
                                        [max_blocks] per-head page tables */
    const int32_t* head_seq_len;     /* nullable device [n_layers][n_requests][n_kv_heads] */
} bkv_cache;

/* ABI version of the loaded library (BKV_ABI_VERSION when it was built). */
int32_t bkv_abi_version(void);

/* Static English text of a code; never NULL. */
const char* bkv_status_string(int32_t code);

/* Beacon maintenance (BeaconKV explainer, section 3.2: nearest beacon,
 * incremental update).  For each of HC head-caches, absorbs the T*G buffered
 * decode queries queries[hc][t][g][:] (bf16, 128 wide) in (t, then g) order:
 *   - if some row has count 0, the smallest such row j takes the query:
 *     beacons[hc][j] = x exactly, counts[hc][j] = 1;
 *   - otherwise j = the row of highest cosine(x, b_j) (ties -> lowest j; a
 *     zero norm on either side counts as cosine 0), then counts[j] += 1 and
 *     b_j = b_j + (x - b_j) / counts[j], with IEEE fp32 subtract, divide and
 *     add (no fused multiply-add; bit-exact).
 * count_cap > 0 clamps every incremented count to count_cap (a full row then
 * moves by 1/count_cap of each new query's difference, an exponential moving
 * average that keeps beacons evolving during decoding; explainer section
 * 3.2); 0 keeps the plain running mean.  A fill still sets count 1.
 * beacons fp32 [HC][K][128] and counts int32 [HC][K] are updated in place;
 * assign (nullable) int32 [HC][T*G] receives every chosen row.  Cosines are
 * evaluated in fp32, so on a near tie the chosen row is the best to within
 * fp32 rounding of the cosines.  1 <= K <= 256, T*G >= 1, count_cap >= 0.
 * queries and beacons must be 16-byte aligned. */
int32_t bkv_beacon_update(int32_t n_head_caches, int32_t T, int32_t G, int32_t head_dim,
                          int32_t K, const uint16_t* queries, float* beacons, int32_t* counts,
                          int32_t* assign, int32_t count_cap, bkv_stream_t stream);

/* Beacon scoring of every cached key (the traversal of the paged KV
 * state that content-dependent selectors need; Random Attention article,
 * section "发现四").  With live beacons J = {j : counts[hc][j] > 0} rounded to
 * bf16 (round to nearest even) and s_jn = (bf16(b_j) . k_n) / sqrt(128)
 * accumulated in fp32:
 *   lse_j    = log sum_{n < N} exp(s_jn)                 (all N slots)
 *   score(n) = max_{j in J} exp(s_jn - lse_j) + bonus * [n >= N - window]
 * for n in [P, N), written to scores[hc * score_stride + (n - P)] (fp32).
 * An empty J gives 0 + bonus.  lse (nullable) fp32 [HC][K] receives lse_j
 * (natural log; NaN for rows outside J).  Requires N - P <= score_stride for
 * every request (device-checked: BKV_ERR_LENGTH).  The keys are read twice
 * (the second read is expected to hit the GPU caches). */
int32_t bkv_beacon_score(const bkv_cache* cache, const float* beacons, const int32_t* counts,
                         int32_t K, int32_t window, float bonus, float* scores,
                         int32_t score_stride, float* lse, int32_t* status,
                         bkv_stream_t stream);

/* Random-selector scores (Random Attention article, section "Random
 * Attention": independent per-head random retention; no key is read).  For
 * slot n in [P, N) of head-cache (layer, r, head):
 *   scores[hc * score_stride + (n - P)] = high 32 bits of word (n mod 4) of
 *   Philox4x64-10(counter = (n div 4, pass_idx[r], (layer << 32) | head,
 *                  request_ids[r]), key = (seed, 0)).
 * request_ids uint64 [n_requests], pass_idx int32 [n_requests] are device
 * arrays; a new pass index gives fresh draws.
 * rows selects the row layout (same article, section "发现二": all heads on
 * one common set of random positions): BKV_ROWS_PER_HEAD draws one row per
 * head-cache; BKV_ROWS_PER_LAYER_REQUEST one row per (layer, request), row
 * layer * n_requests + r, with the head field 0 (shared positions);
 * BKV_ROWS_PER_REQUEST one row per request, row r, with the layer and head
 * fields 0 (page retention).  Any other value is BKV_ERR_INVALID. */
int32_t bkv_random_score(const bkv_cache* cache, uint64_t seed, const uint64_t* request_ids,
                         const int32_t* pass_idx, int32_t rows, uint32_t* scores,
                         int32_t score_stride, int32_t* status, bkv_stream_t stream);

/* Top-B selection with full prompt protection (Random Attention article,
 * section "Random Attention": the prompt is always kept, the rest is a per-head
 * top-K).  The budget includes the prompt.  Per head-cache, keep_idx[hc][:]
 * (int32 [HC][budget]) receives the kept slots in ascending order:
 *   N <= budget : 0..N-1, then -1 padding;
 *   P <= budget < N : [0, P) plus the budget - P best candidates of [P, N) by
 *                     (score descending, slot ascending);
 *   P > budget : device error BKV_ERR_BUDGET, row untouched.
 * score_kind BKV_SCORE_F32 compares non-negative fp32 scores (negative values
 * count as 0), BKV_SCORE_U32 unsigned 32-bit draws; candidates are read from
 * scores[hc * score_stride + (n - P)].  score_stride <= BKV_MAX_CANDIDATES.
 * The selection is an exact radix select: results are bit-reproducible. */
int32_t bkv_topk_select(const bkv_cache* cache, const void* scores, int32_t score_kind,
                        int32_t score_stride, int32_t budget, int32_t* keep_idx,
                        int32_t* status, bkv_stream_t stream);

/* Shared positions (Random Attention article, section "发现二": forcing
 * every head onto one common set of positions leaves accuracy almost
 * unchanged).  One selection per (layer, request), u = layer * n_requests + r,
 * for all its KV heads.  The candidate key of slot n is the largest of the
 * score_heads per-head keys scores[(u * score_heads + h) * score_stride +
 * (n - P)], h < score_heads (1 <= score_heads <= n_kv_heads: n_kv_heads for
 * per-head beacon scores, 1 for one shared random draw row); keys are ranked
 * and the prompt protected exactly as in bkv_topk_select.  keep_idx is int32
 * [n_layers * n_requests][budget]; use it with bkv_kv_compact(keep_shared=1). */
int32_t bkv_topk_select_shared(const bkv_cache* cache, const void* scores, int32_t score_kind,
                               int32_t score_stride, int32_t score_heads, int32_t budget,
                               int32_t* keep_idx, int32_t* status, bkv_stream_t stream);

/* Cache compaction (Random Attention article, section "发现四": the one
 * step every selector shares).  In place, for i < min(N, budget):
 *   K[i] <- K[keep[i]], V[i] <- V[keep[i]]   (every layer pool, per head)
 *   pos_ids[hc][i] <- pos_ids[hc][keep[i]]   (when pos_ids is not NULL)
 * through the block table, preserving order.  The keep list must be strictly
 * ascending inside [0, N) (device-checked: BKV_ERR_INVALID, head-cache left
 * untouched); slots past min(N, budget) keep stale data and can be released by
 * the caller (every head keeps the same count, so whole tail blocks free up).
 * seq_len is not modified.  keep_shared = 0: keep_idx is [HC][budget], one
 * list per head-cache; keep_shared = 1: keep_idx is [n_layers *
 * n_requests][budget] and head-cache hc applies row hc / n_kv_heads (shared
 * positions, see bkv_topk_select_shared). */
int32_t bkv_kv_compact(const bkv_cache* cache, const int32_t* keep_idx, int32_t budget,
                       int32_t keep_shared, int32_t* pos_ids, int32_t pos_stride,
                       int32_t* status, bkv_stream_t stream);

/* Page retention (Random Attention article, section "发现二": keeping
 * contiguous blocks of up to 64 tokens instead of scattered tokens, and one
 * common set of positions for all heads, both leave accuracy almost
 * unchanged).  One selection of whole 16-slot pages per request, for every
 * layer and head, so no K/V row moves: the request's block table is rewritten.
 * For request r with N slots, P prompt slots and npages = ceil(N / 16):
 *   - pages holding a prompt slot and a partial last page are always kept;
 *   - a page's key is the largest score of its slots over the request's score
 *     rows: score_rows = BKV_ROWS_PER_HEAD reads every head-cache row of the
 *     request ((layer * n_requests + r) * n_kv_heads + h), BKV_ROWS_PER_REQUEST
 *     reads row r (one shared random draw row); column n - P as usual;
 *   - budget / 16 pages survive (budget must be a multiple of 16): the forced
 *     pages plus the best remaining pages by (key descending, page ascending);
 *     npages <= budget / 16 keeps every page; more forced pages than that is
 *     the device error BKV_ERR_BUDGET (request untouched).
 * Outputs, for every request that passes its checks:
 *   keep_pages int32 [n_requests][budget / 16]: kept page indices ascending,
 *     -1 padded;
 *   block_table_out int32 [n_requests][max_blocks]: entry i < kept = the block
 *     of the i-th kept page, entries [kept, npages) = -1, the rest untouched;
 *     it may be the cache's own block_table (rewritten in place);
 *   seq_len_out int32 [n_requests]: the new slot count (may be the cache's
 *     own seq_len); prompt_len is unchanged, since prompt pages stay in front;
 *   freed_blocks int32 [n_requests][max_blocks]: the blocks of the dropped
 *     pages in page order, then -1; the caller returns them to its allocator.
 * scores is read exactly as written by bkv_beacon_score (BKV_SCORE_F32) or
 * bkv_random_score (BKV_SCORE_U32, rows BKV_ROWS_PER_REQUEST). */
int32_t bkv_page_retain(const bkv_cache* cache, const void* scores, int32_t score_kind,
                        int32_t score_stride, int32_t score_rows, int32_t budget,
                        int32_t* keep_pages, int32_t* block_table_out, int32_t* seq_len_out,
                        int32_t* freed_blocks, int32_t* status, bkv_stream_t stream);

/* Page retention per head-cache (block-granular retention with per-head
 * block tables; Random Attention article, section "发现二": blocks of up to 64
 * tokens keep accuracy with every head selecting on its own, an independence
 * the section credits with redundancy across heads).  Every head-cache hc
 * selects its own pages exactly as bkv_page_retain selects a request's, from
 * its own score row scores[hc][:] (BKV_ROWS_PER_HEAD; f32 beacon scores or
 * u32 draws) and over its own pages: the cache's head_block_table row hc and
 * head_seq_len[hc] when the cache has them, else its request's block_table
 * row and seq_len.  No K/V row moves.  Outputs per head-cache, written for
 * every head-cache that passes its checks (a failing one is untouched):
 *   keep_pages int32 [HC][budget / 16]: kept page indices ascending, -1 padded;
 *   head_table_out int32 [HC][max_blocks]: entry i < kept = the block of the
 *     i-th kept page, entries [kept, npages) = -1, the rest untouched (it may
 *     be the cache's own head_block_table);
 *   head_seq_len_out int32 [HC]: the new slot count (may be head_seq_len);
 *   dropped_blocks int32 [HC][max_blocks]: the blocks of the head-cache's
 *     dropped pages in page order, then -1.  A block id is shared by every
 *     layer and head of its request, so the caller frees a block once no
 *     head-cache's row holds it any more (for example with a count of the
 *     rows holding each block).
 * To read the cache through the new rows, pass head_table_out and
 * head_seq_len_out as the cache's head_block_table and head_seq_len. */
int32_t bkv_page_retain_heads(const bkv_cache* cache, const void* scores, int32_t score_kind,
                              int32_t score_stride, int32_t budget, int32_t* keep_pages,
                              int32_t* head_table_out, int32_t* head_seq_len_out,
                              int32_t* dropped_blocks, int32_t* status, bkv_stream_t stream);

/* Decode attention over the (compacted) cache: the step every selector hands
 * its cache to (Random Attention article, section "发现四": the selectors share
 * the attention kernels and the paging).  For every head-cache hc and query
 * head g < G (1 <= G <= BKV_MAX_QUERY_HEADS), over the slots n < N of its
 * request:
 *   s_n = scale * (q . k_n),  out[hc][g][:] = sum_n softmax(s)_n v_n
 * with fp32 products and sums (bf16 inputs); N = 0 gives zeros.  queries bf16
 * [HC][G][128], out fp32 [HC][G][128], both 16-byte aligned.  Slot order does
 * not matter: keys are stored with their positions already applied, so after
 * compaction set seq_len to the kept count and attend. */
int32_t bkv_decode_attention(const bkv_cache* cache, const uint16_t* queries, int32_t G,
                             float scale, float* out, int32_t* status, bkv_stream_t stream);

/* One whole eviction pass at a synchronized batch point: maintenance,
 * scoring, selection and compaction for every layer, request and head. */
typedef struct bkv_pass_args {
    int32_t selector;          /* BKV_SELECT_BEACON or BKV_SELECT_RANDOM */
    int32_t budget;            /* B, prompt included */
    int32_t score_stride;      /* 0 -> max_blocks * block_size */
    int32_t shared_positions;  /* 0: per-head selection; 1: one selection per (layer,
                                  request) for all its heads (bkv_topk_select_shared:
                                  beacon merges the per-head scores by their maximum,
                                  random draws one row); keep lists then have
                                  n_layers * n_requests rows, and so does the random
                                  selector's score buffer */
    int32_t page_retention;    /* BKV_PAGES_PER_REQUEST: bkv_page_retain replaces
                                  selection and compaction (budget a multiple of 16,
                                  shared_positions 0, pos_ids NULL); keep lists are the
                                  kept pages [n_requests][budget / 16], the random
                                  selector draws one row per request, and the three
                                  outputs below are required.  BKV_PAGES_PER_HEAD:
                                  bkv_page_retain_heads instead, with keep lists
                                  [HC][budget / 16], per-head draw rows and the outputs
                                  below per head-cache */
    int32_t* block_table_out;  /* page retention: [n_requests][max_blocks] (per head:
                                  [HC][max_blocks]), may alias */
    int32_t* seq_len_out;      /* page retention: [n_requests] ([HC]), may alias */
    int32_t* freed_blocks;     /* page retention: [n_requests][max_blocks] (per head:
                                  the dropped blocks, [HC][max_blocks]) */
    /* beacon selector */
    int32_t n_beacons;         /* K */
    int32_t T, G;              /* buffered decode steps, query heads per KV head */
    int32_t window;            /* recent-window length W */
    float bonus;               /* recent-window bonus */
    const uint16_t* queries;   /* bf16 [HC][T][G][128] */
    float* beacons;            /* fp32 [HC][K][128], updated */
    int32_t* counts;           /* int32 [HC][K], updated */
    int32_t* assign;           /* nullable int32 [HC][T*G] */
    int32_t count_cap;         /* 0: running mean; > 0: counts clamp there */
    float* lse;                /* nullable fp32 [HC][K] */
    /* random selector */
    uint64_t seed;
    const uint64_t* request_ids; /* device [n_requests] */
    const int32_t* pass_idx;     /* device [n_requests] */
    /* optional outputs / buffers */
    int32_t* pos_ids;          /* nullable int32 [HC][pos_stride], compacted with the cache */
    int32_t pos_stride;
    void* scores_out;          /* nullable [rows][score_stride] scores; else workspace */
    int32_t* keep_out;         /* nullable [rows][budget] keep lists (kept pages
                                  [n_requests][budget / 16] with page retention);
                                  else workspace */
    /* optional profiling hook: caller-created hipEvent_t handles, recorded on
     * `stream` before the first kernel and after every step of the pass
     * (beacon: 5 events around update, score, select, compact; random: 4
     * events around score, select, compact; one fewer with page retention,
     * whose one kernel replaces select and compact).  When the fused kernel
     * runs (below), the events after score, select and compact are all
     * recorded after it, so the score interval covers the three steps and
     * the other two are empty.  Ignored when NULL or when n_timing_events is
     * smaller than that. */
    void* const* timing_events;
    int32_t n_timing_events;
    /* Row compaction with per-head selection (either selector) or with
     * shared positions (beacon selector): scoring (or the random draws),
     * selection and compaction run as one kernel, each workgroup taking its
     * head-cache -- or, shared, the H heads of its (layer, request) --
     * through all three (same results as the separate kernels; scores are
     * still written), whenever score_stride + budget <=
     * BKV_FUSED_MAX_ENTRIES.  1 runs them as three kernels instead (for
     * per-step timing). */
    int32_t separate_steps;
} bkv_pass_args;

/* Bytes of workspace bkv_evict_pass needs for these arguments (the score and
 * keep buffers it is not given, and the partial log-sum-exps of a split
 * beacon scoring, below).  The workspace is a caller-owned device buffer
 * aligned to 256 bytes. */
int32_t bkv_workspace_size(const bkv_cache* cache, const bkv_pass_args* args, size_t* bytes);

/* One eviction pass at a compression point.  The beacon pass's order --
 * absorb the buffered queries into the beacons, score every key against
 * them, keep the budget -- is the mechanism of the BeaconKV explainer,
 * section 3.2; the random pass is the random-retention rule of the Random
 * Attention article (section "Random Attention：不判断重要性，只随机保留":
 * prompt kept, one draw and one top-k per head); both end in the cache
 * compaction that the article's section "发现四" counts as a cost every
 * selector shares.
 * Runs, on `stream`: (beacon) maintenance -> beacon scoring -> selection ->
 * compaction, or (random) random scoring -> selection -> compaction; with
 * page_retention, bkv_page_retain takes the place of the last two.  Scoring,
 * selection and compaction run as one fused kernel where separate_steps
 * allows it (see there); the results are those of the separate kernels.
 * A beacon pass that no fused kernel could run (score_stride + budget >
 * BKV_FUSED_MAX_ENTRIES) with at most 256 head-caches splits each
 * head-cache's keys over several workgroups to fill the GPU: its scores and
 * lse then match bkv_beacon_score's to within fp32 rounding (another
 * summation order), not bit for bit.
 * A request that fails a device check (lengths, block ids, budget) is left
 * entirely untouched -- beacons, counts, cache and pos_ids -- and flagged in
 * *status. */
int32_t bkv_evict_pass(const bkv_cache* cache, const bkv_pass_args* args, void* workspace,
                       size_t workspace_bytes, int32_t* status, bkv_stream_t stream);

/* bkv_evict_pass without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of bkv_evict_pass; the buffers bkv_workspace_size counts (the score and
 * keep buffers the pass is not given) live in a scratch array of
 * BKV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * from the loading of its code on that GPU until the process ends.  The call
 * allocates and frees nothing.  Returns BKV_ERR_SCRATCH, with nothing
 * enqueued, when bkv_workspace_size exceeds BKV_NOALLOC_SCRATCH_BYTES (the
 * 128-request, 36-layer, B = 2048 serving pass needs 160 MB).  The array's
 * address on the stream's GPU is looked up on the first call on that GPU
 * (BKV_ERR_HIP if that fails).  All calls on one GPU share its array, which
 * keeps the last call's contents (nothing in it needs to start at zero): two
 * calls whose work overlaps on one GPU -- on different streams, or enqueued
 * from different host threads without ordering -- race, and their results
 * are undefined. */
int32_t bkv_evict_pass_noalloc(const bkv_cache* cache, const bkv_pass_args* args,
                               int32_t* status, bkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BEACONKV_H */
