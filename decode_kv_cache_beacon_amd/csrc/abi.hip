// abi.hip -- extern "C" entry points of libbeaconkv.so: synchronous argument
// validation (nothing is enqueued on failure), then kernel launches on the
// caller's stream.  No allocation; the one piece of global state is the
// scratch array of bkv_evict_pass_noalloc and its per-device addresses.

#include <limits.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "bkv_internal.h"

using namespace bkv;

// Scratch of bkv_evict_pass_noalloc (the score and keep buffers a pass is not
// given).  Each GPU the library's code is loaded on holds its own copy, at its
// own address, until the process ends.  In host code the name below is a
// host-side stand-in, not a device address: host code only ever uses the
// address hipGetSymbolAddress returns for the device (scratch_address below).
static __device__ __align__(256) uint8_t scratch[BKV_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t check_cache(const bkv_cache* cache, CacheView* v) {
    if (!cache) return BKV_ERR_NULL;
    if (!cache->k_pools || !cache->v_pools || !cache->block_table || !cache->seq_len ||
        !cache->prompt_len)
        return BKV_ERR_NULL;
    if (cache->head_dim != kHeadDim || cache->block_size != kBlock) return BKV_ERR_UNSUPPORTED;
    if (cache->n_layers < 1 || cache->n_requests < 1 || cache->n_kv_heads < 1 ||
        cache->max_blocks < 1 || cache->num_blocks < 1)
        return BKV_ERR_INVALID;
    // L * R fits int64 for any int32 operands; it is bounded before the third
    // factor so that L * R * H cannot overflow either
    const int64_t lr = (int64_t)cache->n_layers * cache->n_requests;
    if (lr > INT_MAX || lr * cache->n_kv_heads > INT_MAX ||
        (int64_t)cache->max_blocks * kBlock > kMaxSlots ||
        cache->num_blocks > INT_MAX)
        return BKV_ERR_INVALID;
    if (!aligned(cache->k_pools, 8) || !aligned(cache->v_pools, 8) ||
        !aligned(cache->block_table, 4) || !aligned(cache->seq_len, 4) ||
        !aligned(cache->prompt_len, 4))
        return BKV_ERR_INVALID;
    // per-head page tables come as a pair
    if ((cache->head_block_table == nullptr) != (cache->head_seq_len == nullptr))
        return BKV_ERR_INVALID;
    if (!aligned(cache->head_block_table, 4) || !aligned(cache->head_seq_len, 4))
        return BKV_ERR_INVALID;
    v->L = cache->n_layers;
    v->R = cache->n_requests;
    v->H = cache->n_kv_heads;
    v->max_blocks = cache->max_blocks;
    v->num_blocks = cache->num_blocks;
    v->k_pools = cache->k_pools;
    v->v_pools = cache->v_pools;
    v->block_table = cache->block_table;
    v->seq_len = cache->seq_len;
    v->prompt_len = cache->prompt_len;
    v->head_table = cache->head_block_table;
    v->head_len = cache->head_seq_len;
    return BKV_OK;
}

int64_t head_caches(const CacheView& v) { return (int64_t)v.L * v.R * v.H; }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? BKV_OK : BKV_ERR_HIP; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct PassLayout {
    int stride;
    int parts;  // beacon scoring: workgroups per head-cache (1: unsplit)
    size_t scores_off, keep_off, part_off, pkey_off, total;
};

// Row layout of the random selector's draws in a pass: per head-cache, per
// (layer, request) with shared positions, per request with page retention
// (per head-cache with per-head page retention).
int random_rows(const bkv_pass_args* a) {
    return a->page_retention == BKV_PAGES_PER_REQUEST ? BKV_ROWS_PER_REQUEST
           : a->shared_positions                      ? BKV_ROWS_PER_LAYER_REQUEST
                                                      : BKV_ROWS_PER_HEAD;
}
size_t layout_rows(const CacheView& v, int rows) {
    return rows == BKV_ROWS_PER_REQUEST        ? (size_t)v.R
           : rows == BKV_ROWS_PER_LAYER_REQUEST ? (size_t)v.L * v.R
                                                : (size_t)v.L * v.R * v.H;
}
// Rows of the score buffer and of the keep buffer of a pass (beacon scores
// are always per head-cache).
size_t score_rows(const CacheView& v, const bkv_pass_args* a) {
    return a->selector == BKV_SELECT_RANDOM ? layout_rows(v, random_rows(a))
                                            : layout_rows(v, BKV_ROWS_PER_HEAD);
}
size_t keep_rows(const CacheView& v, const bkv_pass_args* a) {
    return a->page_retention == BKV_PAGES_PER_REQUEST ? (size_t)v.R
           : a->shared_positions                      ? (size_t)v.L * v.R
                                                      : (size_t)v.L * v.R * v.H;
}
size_t keep_cols(const bkv_pass_args* a) {
    return a->page_retention ? (size_t)(a->budget / kBlock) : (size_t)a->budget;
}

// Row compaction runs scoring (or the draws), selection and compaction as
// one kernel when its LDS holds the candidates and keep list: per head for
// either selector, or shared positions for the beacon selector.  The fused
// kernels keep the keep list on chip (written out only to keep_out).
bool fused_pass(const bkv_pass_args* a, int stride) {
    return !a->page_retention && !a->separate_steps &&
           (!a->shared_positions || a->selector == BKV_SELECT_BEACON) &&
           (int64_t)stride + a->budget <= kFusedMaxEntries;
}

// Workgroups per head-cache of a pass's beacon scoring.  A pass that no fused
// kernel can run (more candidates and keep entries than its LDS holds) and
// that has no more head-caches than the GPU has CUs (256) splits each
// head-cache's keys over up to eight workgroups (about 1024 in all).  Every
// pass a fused kernel could run scores unsplit, so that its separate steps
// reproduce it bit for bit.
int score_parts(const CacheView& v, const bkv_pass_args* a, int stride) {
    if (a->selector != BKV_SELECT_BEACON) return 1;
    if ((int64_t)stride + a->budget <= kFusedMaxEntries) return 1;
    const int64_t hc = head_caches(v);
    if (hc == 0 || hc > 256) return 1;
    return (int)std::min<int64_t>(8, std::max<int64_t>(1, 1024 / hc));
}

int32_t pass_layout(const CacheView& v, const bkv_pass_args* a, PassLayout* L) {
    const int max_slots = v.max_blocks * kBlock;
    const int stride = a->score_stride > 0 ? a->score_stride : max_slots;
    if (stride > BKV_MAX_CANDIDATES) return BKV_ERR_INVALID;
    if (a->budget < 1) return BKV_ERR_INVALID;
    if (a->shared_positions != 0 && a->shared_positions != 1) return BKV_ERR_INVALID;
    if (a->page_retention != 0 && a->page_retention != BKV_PAGES_PER_REQUEST &&
        a->page_retention != BKV_PAGES_PER_HEAD)
        return BKV_ERR_INVALID;
    if (a->page_retention && (a->budget % kBlock != 0 || a->shared_positions))
        return BKV_ERR_INVALID;
    // a cache read through per-head page tables: every selection is per head
    if (v.head_table && (a->shared_positions || a->page_retention == BKV_PAGES_PER_REQUEST))
        return BKV_ERR_INVALID;
    size_t off = 0;
    L->stride = stride;
    L->parts = score_parts(v, a, stride);
    L->scores_off = L->keep_off = L->part_off = L->pkey_off = 0;
    if (!a->scores_out) {
        L->scores_off = off;
        off = round_up(off + score_rows(v, a) * (size_t)stride * 4, 256);
    }
    if (!a->keep_out && !fused_pass(a, stride)) {
        L->keep_off = off;
        off = round_up(off + keep_rows(v, a) * keep_cols(a) * 4, 256);
    }
    if (L->parts > 1) {  // the parts' log-sum-exps
        L->part_off = off;
        off = round_up(off + (size_t)head_caches(v) * L->parts * BKV_MAX_BEACONS * 4, 256);
    }
    if (a->page_retention == BKV_PAGES_PER_REQUEST && a->selector == BKV_SELECT_BEACON) {
        L->pkey_off = off;  // the requests' page keys
        off = round_up(off + (size_t)v.R * v.max_blocks * 4, 256);
    }
    L->total = off;
    return BKV_OK;
}

// The pass after the cache, the selector and the buffer layout have been
// checked and `ws` holds L.total bytes: validates the remaining arguments,
// then launches on the stream (nothing is enqueued on a failed check).
int32_t run_pass(const CacheView& v, const PassLayout& L, const bkv_pass_args* a, uint8_t* ws,
                 int32_t* status, bkv_stream_t stream) {
    if (status && !aligned(status, 4)) return BKV_ERR_INVALID;
    if (a->pos_ids && (a->pos_stride < v.max_blocks * kBlock || !aligned(a->pos_ids, 4)))
        return BKV_ERR_INVALID;
    if ((a->scores_out && !aligned(a->scores_out, 4)) || (a->keep_out && !aligned(a->keep_out, 4)))
        return BKV_ERR_INVALID;
    const bool beacon = a->selector == BKV_SELECT_BEACON;
    const int shared = a->shared_positions;
    const bool pages = a->page_retention != 0;
    const bool head_pages = a->page_retention == BKV_PAGES_PER_HEAD;
    if (pages) {
        if (!a->block_table_out || !a->seq_len_out || !a->freed_blocks) return BKV_ERR_NULL;
        if (a->pos_ids || !aligned(a->block_table_out, 4) || !aligned(a->seq_len_out, 4) ||
            !aligned(a->freed_blocks, 4))
            return BKV_ERR_INVALID;
    }
    if (beacon) {
        if (!a->queries || !a->beacons || !a->counts) return BKV_ERR_NULL;
        if (a->n_beacons < 1 || a->n_beacons > BKV_MAX_BEACONS || a->T < 1 || a->G < 1 ||
            a->count_cap < 0 ||
            a->window < 0 || (int64_t)a->T * a->G > INT_MAX / kHeadDim)
            return BKV_ERR_INVALID;
        if (!aligned(a->queries, 16) || !aligned(a->beacons, 16) || !aligned(a->counts, 4) ||
            (a->assign && !aligned(a->assign, 4)) || (a->lse && !aligned(a->lse, 4)))
            return BKV_ERR_INVALID;
    } else {
        if (!a->request_ids || !a->pass_idx) return BKV_ERR_NULL;
        if (!aligned(a->request_ids, 8) || !aligned(a->pass_idx, 4)) return BKV_ERR_INVALID;
    }

    void* sc = a->scores_out ? a->scores_out : ws + L.scores_off;
    int32_t* keep = a->keep_out ? a->keep_out : reinterpret_cast<int32_t*>(ws + L.keep_off);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // every kernel applies every check, so a failing request is skipped by all steps
    const Check all{a->budget, L.stride, 1, pages ? 1 : 0};
    const int HC = (int)head_caches(v);
    const int n_marks = (beacon ? 5 : 4) - (pages ? 1 : 0);
    const bool timed = a->timing_events && a->n_timing_events >= n_marks;
    if (timed)
        for (int i = 0; i < n_marks; ++i)
            if (!a->timing_events[i]) return BKV_ERR_NULL;
    int mark_i = 0;
    auto mark = [&]() -> hipError_t {
        return timed ? hipEventRecord(static_cast<hipEvent_t>(a->timing_events[mark_i++]), s)
                     : hipSuccess;
    };
    hipError_t he = mark();
    if (he != hipSuccess) return BKV_ERR_HIP;
    // row compaction: one kernel for score, select and compact when its LDS
    // holds the candidates and keep list (per head for either selector, or
    // shared positions for the beacon selector)
    const bool fused = fused_pass(a, L.stride);
    if (fused && beacon) {
        he = launch_beacon_update(HC, a->T, a->G, a->n_beacons, a->queries, a->beacons, a->counts,
                                  a->assign, a->count_cap, &v, all, status, s);
        if (he == hipSuccess) he = mark();
        if (he == hipSuccess)
            he = (shared ? launch_beacon_evict_shared : launch_beacon_evict)(
                v, a->beacons, a->counts, a->n_beacons, a->window, a->bonus,
                static_cast<float*>(sc), L.stride, a->lse, a->budget, a->keep_out, a->pos_ids,
                a->pos_stride, all, status, s);
        for (int i = 0; i < 3 && he == hipSuccess; ++i) he = mark();
        return hip_status(he);
    }
    if (fused) {
        he = launch_random_evict(v, a->seed, a->request_ids, a->pass_idx, static_cast<uint32_t*>(sc),
                                 L.stride, a->budget, a->keep_out, a->pos_ids, a->pos_stride, all,
                                 status, s);
        for (int i = 0; i < 3 && he == hipSuccess; ++i) he = mark();
        return hip_status(he);
    }
    if (beacon) {
        he = launch_beacon_update(HC, a->T, a->G, a->n_beacons, a->queries, a->beacons, a->counts,
                                  a->assign, a->count_cap, &v, all, status, s);
        if (he == hipSuccess) he = mark();
        if (he == hipSuccess && L.parts > 1)
            he = launch_beacon_score_split(v, a->beacons, a->counts, a->n_beacons, a->window,
                                           a->bonus, static_cast<float*>(sc), L.stride, a->lse,
                                           reinterpret_cast<float*>(ws + L.part_off), L.parts,
                                           all, status, s);
        else if (he == hipSuccess)
            he = launch_beacon_score(v, a->beacons, a->counts, a->n_beacons, a->window, a->bonus,
                                     static_cast<float*>(sc), L.stride, a->lse, all, status, s);
        if (he == hipSuccess) he = mark();
        if (he == hipSuccess && head_pages)
            he = launch_page_retain_heads(v, sc, BKV_SCORE_F32, L.stride, a->budget, keep,
                                          a->block_table_out, a->seq_len_out, a->freed_blocks,
                                          all, status, s);
        else if (he == hipSuccess && pages)
            he = launch_page_retain(v, sc, BKV_SCORE_F32, L.stride, BKV_ROWS_PER_HEAD, a->budget,
                                    keep, a->block_table_out, a->seq_len_out, a->freed_blocks,
                                    reinterpret_cast<uint32_t*>(ws + L.pkey_off), all, status, s);
        else if (he == hipSuccess)  // shared: the largest of the H per-head scores
            he = launch_topk_select(v, sc, BKV_SCORE_F32, L.stride, v.H, shared, a->budget, keep,
                                    all, status, s);
    } else {
        he = launch_random_score(v, a->seed, a->request_ids, a->pass_idx, random_rows(a),
                                 static_cast<uint32_t*>(sc), L.stride, all, status, s);
        if (he == hipSuccess) he = mark();
        if (he == hipSuccess && head_pages)
            he = launch_page_retain_heads(v, sc, BKV_SCORE_U32, L.stride, a->budget, keep,
                                          a->block_table_out, a->seq_len_out, a->freed_blocks,
                                          all, status, s);
        else if (he == hipSuccess && pages)
            he = launch_page_retain(v, sc, BKV_SCORE_U32, L.stride, BKV_ROWS_PER_REQUEST,
                                    a->budget, keep, a->block_table_out, a->seq_len_out,
                                    a->freed_blocks, nullptr, all, status, s);
        else if (he == hipSuccess)  // shared: one draw row per (layer, request)
            he = launch_topk_select(v, sc, BKV_SCORE_U32, L.stride, 1, shared, a->budget, keep,
                                    all, status, s);
    }
    if (he == hipSuccess) he = mark();
    if (he == hipSuccess && !pages) {
        he = launch_kv_compact(v, keep, a->budget, shared, a->pos_ids, a->pos_stride, all, status,
                               s);
        if (he == hipSuccess) he = mark();
    }
    return hip_status(he);
}

constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the GPU that runs `stream` (the null stream:
// the current device).  It is looked up once per device, with that device
// current, and kept; later calls read the kept address.
int32_t scratch_address(bkv_stream_t stream, uint8_t** out) {
    int dev = -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (s) {
        if (hipStreamGetDevice(s, &dev) != hipSuccess) return BKV_ERR_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return BKV_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return BKV_ERR_HIP;
    uint8_t* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess) return BKV_ERR_HIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess) return BKV_ERR_HIP;
            void* q = nullptr;
            const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (cur != dev) (void)hipSetDevice(cur);
            if (e != hipSuccess || !q) return BKV_ERR_HIP;
            p = static_cast<uint8_t*>(q);
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BKV_OK;
}

}  // namespace

extern "C" {

int32_t bkv_abi_version(void) { return BKV_ABI_VERSION; }

const char* bkv_status_string(int32_t code) {
    switch (code) {
        case BKV_OK: return "ok";
        case BKV_ERR_NULL: return "a required pointer is NULL";
        case BKV_ERR_INVALID: return "invalid size, count, stride, alignment or keep list";
        case BKV_ERR_BUDGET: return "a request's prompt length exceeds the budget";
        case BKV_ERR_UNSUPPORTED: return "unsupported head_dim or block_size (need 128 and 16)";
        case BKV_ERR_WORKSPACE: return "workspace missing or too small";
        case BKV_ERR_HIP: return "HIP launch error";
        case BKV_ERR_LENGTH: return "seq_len / prompt_len out of range";
        case BKV_ERR_BLOCK_TABLE: return "block id outside the pool";
        case BKV_ERR_SCRATCH:
            return "the pass needs more scratch than bkv_evict_pass_noalloc holds "
                   "(BKV_NOALLOC_SCRATCH_BYTES); use bkv_evict_pass with a workspace";
        default: return "unknown status code";
    }
}

int32_t bkv_beacon_update(int32_t n_head_caches, int32_t T, int32_t G, int32_t head_dim, int32_t K,
                          const uint16_t* queries, float* beacons, int32_t* counts,
                          int32_t* assign, int32_t count_cap, bkv_stream_t stream) {
    if (head_dim != kHeadDim) return BKV_ERR_UNSUPPORTED;
    if (n_head_caches < 0 || T < 1 || G < 1 || K < 1 || K > BKV_MAX_BEACONS || count_cap < 0)
        return BKV_ERR_INVALID;
    if ((int64_t)T * G > INT_MAX / kHeadDim) return BKV_ERR_INVALID;
    if (n_head_caches == 0) return BKV_OK;
    if (!queries || !beacons || !counts) return BKV_ERR_NULL;
    if (!aligned(queries, 16) || !aligned(beacons, 16) || !aligned(counts, 4) ||
        (assign && !aligned(assign, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_beacon_update(n_head_caches, T, G, K, queries, beacons, counts, assign,
                                           count_cap, nullptr, Check{-1, -1, 0}, nullptr,
                                           static_cast<hipStream_t>(stream)));
}

int32_t bkv_beacon_score(const bkv_cache* cache, const float* beacons, const int32_t* counts,
                         int32_t K, int32_t window, float bonus, float* scores,
                         int32_t score_stride, float* lse, int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!beacons || !counts || !scores) return BKV_ERR_NULL;
    if (K < 1 || K > BKV_MAX_BEACONS || score_stride < 1 || window < 0) return BKV_ERR_INVALID;
    if (!aligned(beacons, 16) || !aligned(counts, 4) || !aligned(scores, 4) ||
        (lse && !aligned(lse, 4)) || (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_beacon_score(v, beacons, counts, K, window, bonus, scores,
                                          score_stride, lse, Check{-1, score_stride, 1}, status,
                                          static_cast<hipStream_t>(stream)));
}

int32_t bkv_random_score(const bkv_cache* cache, uint64_t seed, const uint64_t* request_ids,
                         const int32_t* pass_idx, int32_t rows, uint32_t* scores,
                         int32_t score_stride, int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!request_ids || !pass_idx || !scores) return BKV_ERR_NULL;
    if (score_stride < 1 || rows < BKV_ROWS_PER_HEAD || rows > BKV_ROWS_PER_REQUEST)
        return BKV_ERR_INVALID;
    if (v.head_table && rows != BKV_ROWS_PER_HEAD) return BKV_ERR_INVALID;
    if (!aligned(request_ids, 8) || !aligned(pass_idx, 4) || !aligned(scores, 4) ||
        (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_random_score(v, seed, request_ids, pass_idx, rows, scores,
                                          score_stride, Check{-1, score_stride, 0}, status,
                                          static_cast<hipStream_t>(stream)));
}

int32_t bkv_topk_select(const bkv_cache* cache, const void* scores, int32_t score_kind,
                        int32_t score_stride, int32_t budget, int32_t* keep_idx, int32_t* status,
                        bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!scores || !keep_idx) return BKV_ERR_NULL;
    if (score_kind != BKV_SCORE_F32 && score_kind != BKV_SCORE_U32) return BKV_ERR_INVALID;
    if (score_stride < 1 || score_stride > BKV_MAX_CANDIDATES || budget < 1) return BKV_ERR_INVALID;
    if (!aligned(scores, 4) || !aligned(keep_idx, 4) || (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_topk_select(v, scores, score_kind, score_stride, 1, 0, budget,
                                         keep_idx, Check{budget, score_stride, 0}, status,
                                         static_cast<hipStream_t>(stream)));
}

int32_t bkv_topk_select_shared(const bkv_cache* cache, const void* scores, int32_t score_kind,
                               int32_t score_stride, int32_t score_heads, int32_t budget,
                               int32_t* keep_idx, int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!scores || !keep_idx) return BKV_ERR_NULL;
    if (score_kind != BKV_SCORE_F32 && score_kind != BKV_SCORE_U32) return BKV_ERR_INVALID;
    if (score_stride < 1 || score_stride > BKV_MAX_CANDIDATES || budget < 1) return BKV_ERR_INVALID;
    if (score_heads < 1 || score_heads > v.H || v.head_table) return BKV_ERR_INVALID;
    if (!aligned(scores, 4) || !aligned(keep_idx, 4) || (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_topk_select(v, scores, score_kind, score_stride, score_heads, 1,
                                         budget, keep_idx, Check{budget, score_stride, 0}, status,
                                         static_cast<hipStream_t>(stream)));
}

int32_t bkv_kv_compact(const bkv_cache* cache, const int32_t* keep_idx, int32_t budget,
                       int32_t keep_shared, int32_t* pos_ids, int32_t pos_stride,
                       int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!keep_idx) return BKV_ERR_NULL;
    if (budget < 1 || (keep_shared != 0 && keep_shared != 1) || (keep_shared && v.head_table))
        return BKV_ERR_INVALID;
    if (pos_ids && pos_stride < v.max_blocks * kBlock) return BKV_ERR_INVALID;
    if (!aligned(keep_idx, 4) || (pos_ids && !aligned(pos_ids, 4)) ||
        (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_kv_compact(v, keep_idx, budget, keep_shared, pos_ids, pos_stride,
                                        Check{budget, -1, 1}, status,
                                        static_cast<hipStream_t>(stream)));
}

int32_t bkv_page_retain(const bkv_cache* cache, const void* scores, int32_t score_kind,
                        int32_t score_stride, int32_t score_rows, int32_t budget,
                        int32_t* keep_pages, int32_t* block_table_out, int32_t* seq_len_out,
                        int32_t* freed_blocks, int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!scores || !keep_pages || !block_table_out || !seq_len_out || !freed_blocks)
        return BKV_ERR_NULL;
    if (score_kind != BKV_SCORE_F32 && score_kind != BKV_SCORE_U32) return BKV_ERR_INVALID;
    if ((score_rows != BKV_ROWS_PER_HEAD && score_rows != BKV_ROWS_PER_REQUEST) || v.head_table)
        return BKV_ERR_INVALID;
    if (score_stride < 1 || budget < kBlock || budget % kBlock != 0) return BKV_ERR_INVALID;
    if (!aligned(scores, 4) || !aligned(keep_pages, 4) || !aligned(block_table_out, 4) ||
        !aligned(seq_len_out, 4) || !aligned(freed_blocks, 4) || (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_page_retain(v, scores, score_kind, score_stride, score_rows, budget,
                                         keep_pages, block_table_out, seq_len_out, freed_blocks,
                                         nullptr, Check{budget, score_stride, 1, 1}, status,
                                         static_cast<hipStream_t>(stream)));
}

int32_t bkv_page_retain_heads(const bkv_cache* cache, const void* scores, int32_t score_kind,
                              int32_t score_stride, int32_t budget, int32_t* keep_pages,
                              int32_t* head_table_out, int32_t* head_seq_len_out,
                              int32_t* dropped_blocks, int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!scores || !keep_pages || !head_table_out || !head_seq_len_out || !dropped_blocks)
        return BKV_ERR_NULL;
    if (score_kind != BKV_SCORE_F32 && score_kind != BKV_SCORE_U32) return BKV_ERR_INVALID;
    if (score_stride < 1 || budget < kBlock || budget % kBlock != 0) return BKV_ERR_INVALID;
    if (!aligned(scores, 4) || !aligned(keep_pages, 4) || !aligned(head_table_out, 4) ||
        !aligned(head_seq_len_out, 4) || !aligned(dropped_blocks, 4) ||
        (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_page_retain_heads(v, scores, score_kind, score_stride, budget,
                                               keep_pages, head_table_out, head_seq_len_out,
                                               dropped_blocks, Check{budget, score_stride, 1, 1},
                                               status, static_cast<hipStream_t>(stream)));
}

int32_t bkv_decode_attention(const bkv_cache* cache, const uint16_t* queries, int32_t G,
                             float scale, float* out, int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!queries || !out) return BKV_ERR_NULL;
    if (G < 1 || G > BKV_MAX_QUERY_HEADS) return BKV_ERR_INVALID;
    if (!aligned(queries, 16) || !aligned(out, 16) || (status && !aligned(status, 4)))
        return BKV_ERR_INVALID;
    return hip_status(launch_decode_attention(v, queries, G, scale, out, status,
                                              static_cast<hipStream_t>(stream)));
}

int32_t bkv_workspace_size(const bkv_cache* cache, const bkv_pass_args* args, size_t* bytes) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!args || !bytes) return BKV_ERR_NULL;
    PassLayout L;
    e = pass_layout(v, args, &L);
    if (e) return e;
    *bytes = L.total;
    return BKV_OK;
}

int32_t bkv_evict_pass(const bkv_cache* cache, const bkv_pass_args* a, void* workspace,
                       size_t workspace_bytes, int32_t* status, bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!a) return BKV_ERR_NULL;
    if (a->selector != BKV_SELECT_BEACON && a->selector != BKV_SELECT_RANDOM)
        return BKV_ERR_INVALID;
    PassLayout L;
    e = pass_layout(v, a, &L);
    if (e) return e;
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return BKV_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 256)) return BKV_ERR_INVALID;
    return run_pass(v, L, a, static_cast<uint8_t*>(workspace), status, stream);
}

int32_t bkv_evict_pass_noalloc(const bkv_cache* cache, const bkv_pass_args* a, int32_t* status,
                               bkv_stream_t stream) {
    CacheView v;
    int32_t e = check_cache(cache, &v);
    if (e) return e;
    if (!a) return BKV_ERR_NULL;
    if (a->selector != BKV_SELECT_BEACON && a->selector != BKV_SELECT_RANDOM)
        return BKV_ERR_INVALID;
    PassLayout L;
    e = pass_layout(v, a, &L);
    if (e) return e;
    if (L.total > (size_t)BKV_NOALLOC_SCRATCH_BYTES) return BKV_ERR_SCRATCH;
    uint8_t* ws = nullptr;
    if (L.total > 0) {
        e = scratch_address(stream, &ws);
        if (e) return e;
    }
    // every byte a kernel of the pass reads from the scratch was written
    // earlier in the same pass, so nothing in it needs to start at zero
    return run_pass(v, L, a, ws, status, stream);
}

}  // extern "C"
