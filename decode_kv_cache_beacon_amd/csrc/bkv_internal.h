// bkv_internal.h -- shared device helpers of the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "beaconkv.h"

namespace bkv {

constexpr int kHeadDim = 128;
constexpr int kBlock = 16;
constexpr int kRowBytes = kHeadDim * 2;  // one bf16 key or value row
constexpr int kWave = 64;

// Kernel-argument copy of a bkv_cache (plain values, passed by value).
struct CacheView {
    int32_t L, R, H, max_blocks;
    int64_t num_blocks;
    const uint64_t* k_pools;
    const uint64_t* v_pools;
    const int32_t* block_table;
    const int32_t* seq_len;
    const int32_t* prompt_len;
    // per-head page tables (both null, or both set): head-cache hc reads its
    // slots through row hc and has head_len[hc] of them
    const int32_t* head_table;
    const int32_t* head_len;
};

// The block-table row and the slot count of head-cache hc of request r (hc <
// 0: the request's own row, for kernels that serve whole requests, which the
// entry points never launch on a cache with per-head tables).
__device__ __forceinline__ const int32_t* table_row(const CacheView& c, int hc, int r) {
    return (c.head_table && hc >= 0) ? c.head_table + (size_t)hc * c.max_blocks
                                     : c.block_table + (size_t)r * c.max_blocks;
}
__device__ __forceinline__ int slot_count(const CacheView& c, int hc, int r) {
    return (c.head_len && hc >= 0) ? c.head_len[hc] : c.seq_len[r];
}

struct HeadIdx {
    int layer, req, head;
};

__device__ __forceinline__ HeadIdx split_hc(const CacheView& c, int hc) {
    HeadIdx x;
    x.head = hc % c.H;
    const int lr = hc / c.H;
    x.req = lr % c.R;
    x.layer = lr / c.R;
    return x;
}

__device__ __forceinline__ void raise_status(int32_t* status, int bits) {
    if (status && bits) atomicOr(status, bits);
}

// Which per-request checks a kernel applies.  A standalone entry point checks
// what its own kernel reads; inside a whole pass every kernel applies the union
// of all checks, so a request that fails any of them is skipped by every step.
struct Check {
    int budget;     // < 0: no budget check
    int cand_cap;   // < 0: no candidate-capacity check (N - P <= cand_cap)
    int blocks;     // non-zero: validate pool alignment and every block id in use
    int pages;      // non-zero: page retention -- the budget counts whole pages (the prompt
                    // pages and a partial last page must fit in budget / 16 pages) and, as
                    // one selection spans every layer, every layer's pools must be aligned
};

// OR of a predicate over the threads that check a request: the whole
// workgroup, or only the calling wave (kernels whose waves serve different
// head-caches, or one-wave workgroups that need no LDS for it).
template <bool kWave_>
__device__ __forceinline__ bool any_thread(bool p) {
    if constexpr (kWave_) return __ballot(p) != 0ull;
    else return __syncthreads_or(p) != 0;
}

// Checks of head-cache hc of request r (hc < 0: of the request's own row) by
// `nthreads` cooperating threads (this one is `tid`); `any` ORs a predicate
// over them.  Errors are OR-ed into *status by tid 0.  Without per-head page
// tables every head-cache of a request reads the same row and lengths, so the
// outcome is the request's; with them the row and the slot count checked are
// the head-cache's own.
template <class Any>
__device__ inline bool request_ok_impl(const CacheView& c, int layer, int r, int hc,
                                       const Check& ck, int32_t* status, int tid, int nthreads,
                                       Any any) {
    const int N = slot_count(c, hc, r);
    const int P = c.prompt_len[r];
    int err = 0;
    if (P < 0 || N < P || N > c.max_blocks * kBlock) err |= 1 << BKV_ERR_LENGTH;
    if (ck.budget >= 0 && P > ck.budget) err |= 1 << BKV_ERR_BUDGET;
    if (ck.cand_cap >= 0 && !(err & (1 << BKV_ERR_LENGTH)) && N - P > ck.cand_cap)
        err |= 1 << BKV_ERR_LENGTH;
    if (ck.pages && ck.budget >= 0 && !(err & (1 << BKV_ERR_LENGTH))) {
        const int npages = (N + kBlock - 1) / kBlock;
        const int prompt_pages = (P + kBlock - 1) / kBlock;
        const int forced = prompt_pages + ((N % kBlock) != 0 && npages - 1 >= prompt_pages);
        if (npages > ck.budget / kBlock && forced > ck.budget / kBlock)
            err |= 1 << BKV_ERR_BUDGET;
    }
    bool bad = false;
    if (ck.pages) {
        bool mis = false;
        for (int l = tid; l < c.L; l += nthreads)
            mis |= ((c.k_pools[l] | c.v_pools[l]) & 15u) != 0;
        if (any(mis)) err |= 1 << BKV_ERR_INVALID;
    }
    if (ck.blocks) {
        if (((c.k_pools[layer] | c.v_pools[layer]) & 15u) != 0) err |= 1 << BKV_ERR_INVALID;
        const int nb = (err & (1 << BKV_ERR_LENGTH)) ? 0 : (N + kBlock - 1) / kBlock;
        const int32_t* row = table_row(c, hc, r);
        for (int i = tid; i < nb; i += nthreads) {
            const int b = row[i];
            bad |= (b < 0) || ((int64_t)b >= c.num_blocks);
        }
    }
    bad = any(bad);
    if (bad) err |= 1 << BKV_ERR_BLOCK_TABLE;
    if (err && tid == 0) raise_status(status, err);
    return err == 0;
}

// Validates head-cache hc of request r (hc < 0: the request's own row).
// Every thread of the block (kWaveOnly: of the wave) must call it; the result
// is uniform.  Errors are OR-ed into *status by thread (lane) 0.
template <bool kWaveOnly = false>
__device__ inline bool request_ok(const CacheView& c, int layer, int r, int hc, const Check& ck,
                                  int32_t* status) {
    const int tid = kWaveOnly ? (int)(threadIdx.x % kWave) : (int)threadIdx.x;
    const int nthreads = kWaveOnly ? kWave : (int)blockDim.x;
    return request_ok_impl(c, layer, r, hc, ck, status, tid, nthreads,
                           [](bool p) { return any_thread<kWaveOnly>(p); });
}

// The same for groups of G consecutive lanes of one wave (G = 32 or 64), each
// group checking its own request r: every lane of the wave must call it, and
// the result is uniform within each group.
template <int G>
__device__ inline bool request_ok_lanes(const CacheView& c, int layer, int r, int hc,
                                        const Check& ck, int32_t* status) {
    const int lane = (int)(threadIdx.x % kWave);
    const unsigned long long gmask =
        G >= kWave ? ~0ull : (((1ull << G) - 1ull) << (lane / G * G));
    return request_ok_impl(c, layer, r, hc, ck, status, lane % G, G,
                           [gmask](bool p) { return (__ballot(p) & gmask) != 0ull; });
}

// Address of the bf16 row of (block, head, row-in-block) in a layer pool.
__device__ __forceinline__ size_t row_offset(int blk, int H, int h, int off) {
    return (((size_t)blk * H + h) * kBlock + off) * kRowBytes;
}

// 16-byte loads/stores at a byte address in the global address space.  Pool
// addresses arrive as integers; casting them straight to global pointers lets
// the compiler emit global_load/store instead of generic flat accesses (which
// would also wait on the LDS counter).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 global_cu32x4;
typedef __attribute__((address_space(1))) u32x4 global_u32x4;
__device__ __forceinline__ u32x4 load16(uint64_t addr) { return *(global_cu32x4*)addr; }
__device__ __forceinline__ void store16(uint64_t addr, u32x4 v) { *(global_u32x4*)addr = v; }
// Streaming (non-temporal) variants for data touched once.
__device__ __forceinline__ u32x4 load16_nt(uint64_t addr) {
    return __builtin_nontemporal_load((global_cu32x4*)addr);
}
__device__ __forceinline__ void store16_nt(uint64_t addr, u32x4 v) {
    __builtin_nontemporal_store(v, (global_u32x4*)addr);
}

// Largest slot count of one request the kernels accept (block table staged in
// LDS: 2048 blocks of 16 slots).
constexpr int kMaxSlots = 32768;
constexpr int kMaxBlocksPerReq = kMaxSlots / kBlock;

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Host-side launchers (defined next to each kernel).  `cache` of the update
// launcher is NULL for the standalone entry point (no request checks).
hipError_t launch_beacon_update(int HC, int T, int G, int K, const uint16_t* q, float* beacons,
                                int32_t* counts, int32_t* assign, int cap, const CacheView* cache,
                                Check ck, int32_t* status, hipStream_t s);
hipError_t launch_beacon_score(const CacheView& c, const float* beacons, const int32_t* counts,
                               int K, int window, float bonus, float* scores, int stride,
                               float* lse, Check ck, int32_t* status, hipStream_t s);
// The same scores with every head-cache's keys split over `nparts` workgroups
// (two launches: partial log-sum-exps into part_lse, [HC][nparts][256]
// floats, then the merge and each part's share of the scores).  Their last
// bits differ from the unsplit kernel's (another summation order); the pass
// uses it only where no fused kernel could run.
hipError_t launch_beacon_score_split(const CacheView& c, const float* beacons,
                                     const int32_t* counts, int K, int window, float bonus,
                                     float* scores, int stride, float* lse, float* part_lse,
                                     int nparts, Check ck, int32_t* status, hipStream_t s);
// Scoring, top-B selection and compaction of every head-cache in one kernel
// (per-head selection).  `scores` is still written (the selection reads it
// back); keep_out and pos_ids are nullable.  Requires stride + budget <=
// kFusedMaxEntries, the candidate keys and keep list the kernel holds in LDS.
constexpr int kFusedMaxEntries = BKV_FUSED_MAX_ENTRIES;
hipError_t launch_beacon_evict(const CacheView& c, const float* beacons, const int32_t* counts,
                               int K, int window, float bonus, float* scores, int stride,
                               float* lse, int budget, int32_t* keep_out, int32_t* pos_ids,
                               int pos_stride, Check ck, int32_t* status, hipStream_t s);
// The same with shared positions: one workgroup per (layer, request) scores
// its H heads, selects once from their largest scores (keep_out rows per
// (layer, request)) and compacts every head.
hipError_t launch_beacon_evict_shared(const CacheView& c, const float* beacons,
                                      const int32_t* counts, int K, int window, float bonus,
                                      float* scores, int stride, float* lse, int budget,
                                      int32_t* keep_out, int32_t* pos_ids, int pos_stride,
                                      Check ck, int32_t* status, hipStream_t s);
// `shared`: one row / keep list per (layer, request) instead of per head-cache.
// `rows` of the random scorer: BKV_ROWS_PER_HEAD, _PER_LAYER_REQUEST or _PER_REQUEST.
hipError_t launch_random_score(const CacheView& c, uint64_t seed, const uint64_t* req_ids,
                               const int32_t* pass_idx, int rows, uint32_t* scores, int stride,
                               Check ck, int32_t* status, hipStream_t s);
// Random draws, top-B selection and compaction of every head-cache in one
// kernel (per-head selection; draws still written to `scores`; keep_out and
// pos_ids nullable).  Requires stride + budget <= kFusedMaxEntries.
hipError_t launch_random_evict(const CacheView& c, uint64_t seed, const uint64_t* req_ids,
                               const int32_t* pass_idx, uint32_t* scores, int stride, int budget,
                               int32_t* keep_out, int32_t* pos_ids, int pos_stride, Check ck,
                               int32_t* status, hipStream_t s);
hipError_t launch_decode_attention(const CacheView& c, const uint16_t* q, int G, float scale,
                                   float* out, int32_t* status, hipStream_t s);
// key_ws (nullable, [R][max_blocks] u32): with per-head score rows, the page
// keys are formed first by one workgroup per (layer, request) into it.
hipError_t launch_page_retain(const CacheView& c, const void* scores, int kind, int stride,
                              int rows, int budget, int32_t* keep_pages, int32_t* block_table_out,
                              int32_t* seq_len_out, int32_t* freed, uint32_t* key_ws, Check ck,
                              int32_t* status, hipStream_t s);
// Page retention per head-cache: each head-cache keeps budget / 16 pages of
// its own (its own score row), written to its own page-table row.
hipError_t launch_page_retain_heads(const CacheView& c, const void* scores, int kind, int stride,
                                    int budget, int32_t* keep_pages, int32_t* head_table_out,
                                    int32_t* head_len_out, int32_t* dropped, Check ck,
                                    int32_t* status, hipStream_t s);
hipError_t launch_topk_select(const CacheView& c, const void* scores, int kind, int stride,
                              int score_heads, int shared, int budget, int32_t* keep, Check ck,
                              int32_t* status, hipStream_t s);
hipError_t launch_kv_compact(const CacheView& c, const int32_t* keep, int budget,
                             int keep_shared, int32_t* pos_ids, int pos_stride, Check ck,
                             int32_t* status, hipStream_t s);

}  // namespace bkv
