// beacon_score.hip -- beacon scoring of every cached key of a head-cache.
//
// What it computes (BeaconKV explainer section 3.2 leaves the importance rule
// open; the rule fixed for this library): with live beacons J (count > 0)
// rounded to bf16 and s_jn = bf16(b_j) . k_n / sqrt(128),
//     lse_j    = log sum_{n < N} exp(s_jn)
//     score(n) = max_{j in J} exp(s_jn - lse_j) + bonus * [n >= N - window].
// The traversal of the paged keys is the extra pass a content-dependent
// selector costs (Random Attention article, section "发现四").
//
// How (one workgroup per head-cache, two workgroups per CU, gfx950):
//   - The beacon.key logits are a [K x 128] x [128 x N] contraction: bf16 MFMA
//     v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Beacons are the A
//     operand (rows, kept in registers for the whole head), 32 keys form the B
//     operand (columns), so each lane owns one key column and 16 beacon rows of
//     a 32x32 result.  The rows are split between NG groups of NQ waves (32 or
//     64 rows per wave); wave (group g, phase q) consumes key tiles q, q+NQ,
//     q+2NQ, ...  Each tile is read from LDS once per group.
//   - Key tiles (32 keys = 8 KiB) stream through an LDS ring of 4 NQ tiles
//     filled by direct-to-LDS DMA (global_load_lds_dwordx4): each load
//     instruction moves 1 KiB of whole key rows, the ring is refilled three
//     iterations ahead, and each tile serves all row groups.  A row's 16-byte
//     chunks are XOR-swizzled by the row index so that the fragment reads are
//     free of bank conflicts.  The waves of the last group issue all the DMA,
//     so their vmcnt counts ring loads only; one barrier per iteration hands
//     the tiles over.  The load stream runs on from phase 1 into phase 2.
//   - Two workgroups share a CU, so one head-cache's set-up (request checks,
//     block table, beacon loads) overlaps the other's streaming.
//   - Phase 1 (log-sum-exp per beacon): per lane and row a running sum of
//     exp2(acc * log2(e)/sqrt(d) - M) with one reference M per wave taken from
//     the wave's first tile; lanes (DPP), then waves (LDS) are merged.  If any
//     live row's sum overflows or underflows (logit spread beyond the fp32
//     exponent range) the head is redone exactly with direct loads: an all-key
//     maximum per row first, then the sums against that maximum.
//   - Phase 2 (score): the keys stream through the ring again (the re-read is
//     mostly served by the memory-side cache) and the MFMA accumulator starts
//     from C = -lse_j (in accumulator units), so the subtraction is free; each
//     lane takes the max over its rows, the row groups are merged through LDS
//     one iteration later, and one exp2 per key gives sigma(n).
// Scaling by 1/sqrt(d) happens in fp32 after accumulation; the bf16 beacons
// are never pre-scaled.
//
// Fused eviction (beacon_evict_kernel): the same workgroup then selects the
// head-cache's top-B slots from the scores it has just written and compacts
// the head-cache in place.  Selection and compaction are per head-cache, so
// nothing waits on other workgroups; the compaction's key reads follow the
// phase-2 stream of the same keys closely enough to be served mostly by the
// memory-side cache, and one workgroup's compaction overlaps the other's
// scoring on the CU.  The LDS ring, idle once phase 2 is done, holds the
// candidate keys, the keep list and the radix-select scratch.  With shared
// positions (beacon_evict_shared_kernel) a workgroup scores the H heads of a
// (layer, request) in turn, then selects once from their largest scores and
// compacts every head.

#include "compact_util.h"

namespace bkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kCs = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
constexpr float kInvCs = 7.842065147748378f;  // sqrt(128) / log2(e)
constexpr int kTileKeys = 32;
constexpr int kTileBytes = kTileKeys * kRowBytes;  // 8 KiB
constexpr int kDepth = 3;                          // ring refilled this many iterations ahead
constexpr int kRingIters = kDepth + 1;
constexpr int kDmaPerTile = kTileBytes / 1024;     // instructions of 64 lanes x 16 B

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within its 32-row block) of accumulator element i for lane half hh.
__device__ __forceinline__ int acc_row(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

// Workgroup barrier without a memory fence.  The ring's DMA completion is
// awaited explicitly (wait_ring) by the waves that issued it; this wave's own
// LDS traffic is completed first, and the compiler may not move memory
// operations across the barrier.  (A fenced __syncthreads would also wait for
// every ring load still in flight and serialise the pipeline.)
__device__ __forceinline__ void ring_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most 8*n of this wave's ring loads are in flight (n <= 2).
__device__ __forceinline__ void wait_ring(int n) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (n <= 0)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else if (n == 1)
        __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    else
        __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 64-lane direct-to-LDS load: lane l copies 16 bytes from `g` to LDS
// address m0 + 16 l.  Written as inline assembly so that the compiler, which
// does not see these loads, does not make every later LDS access of the wave
// wait for all of them; their completion is awaited by wait_ring only.  The
// compiler sets M0 for the statement; the s_nop covers the wait state the
// hardware needs between writing M0 and an LDS DMA that reads it.
__device__ __forceinline__ void dma16(uint64_t g, uint32_t m0) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(g), "{m0}"(m0)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

struct Tile {
    bf16x8_t b[8];
};

// Direct loads of one key's B fragment (d in [16s + 8hh, +8) for k-step s),
// used by the exact fallback only.  Lanes past the last key re-read key N-1.
__device__ __forceinline__ void load_key(Tile& t, uint64_t kbase, const int* s_bt, int H, int h,
                                         int n, int N, int hh) {
    n = min(n, N - 1);
    const uint64_t p = kbase + row_offset(s_bt[n >> 4], H, h, n & 15) + 16 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) t.b[s] = as_bf16x8(load16(p + 32 * s));
}

__device__ __forceinline__ f32x16_t logits(const bf16x8_t (&a)[8], const Tile& t, f32x16_t c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = mfma(a[s], t.b[s], c);
    return c;
}

// Cross-lane reductions on the VALU (DPP and lane swaps, no LDS traffic).
// DPP move of v (lanes without a source keep `old`).
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp(float v, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), kCtrl,
                                                      kRowMask, 0xF, false));
}
// op over the 32 lanes of each wave half; the result is valid in lanes 16-31
// (lower half) and 48-63 (upper half): pairs within quads, quads within 8,
// 8 within rows of 16 (mirrors), then row 0 into row 1 and row 2 into row 3.
template <typename Op>
__device__ __forceinline__ float half_reduce(float v, Op op) {
    v = op(v, dpp<0xB1>(v, v));        // quad_perm [1,0,3,2]
    v = op(v, dpp<0x4E>(v, v));        // quad_perm [2,3,0,1]
    v = op(v, dpp<0x141>(v, v));       // row_half_mirror
    v = op(v, dpp<0x140>(v, v));       // row_mirror
    return op(v, dpp<0x142, 0xA>(v, v));  // row_bcast:15 into rows 1 and 3
}
constexpr int kHalfLead = 16;  // a lane (per half) holding the half_reduce result
// max(v, v of lane l ^ 32), in every lane
__device__ __forceinline__ float max_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
struct AddOp {
    __device__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
__device__ __forceinline__ float half_sum(float v) { return half_reduce(v, AddOp{}); }
__device__ __forceinline__ float half_max(float v) { return half_reduce(v, MaxOp{}); }
// maximum over the wave, uniform
__device__ __forceinline__ float wave_max(float v) {
    const float h = max_halves(half_max(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), kHalfLead));
}

// Layout of the idle ring for the fused selection: radix scratch, one scan
// slot per wave and the first dropped candidate, then the candidate keys
// followed by the keep list (kFusedMaxEntries entries between them).
constexpr int kFuseWsumOff = (sizeof(RadixScratch) + 15) & ~15;
constexpr int kFuseKeyOff = 2048;
static_assert(kFuseWsumOff + 4 * (16 + 1) <= kFuseKeyOff, "fused scratch overlaps the keys");

// Top-B selection from the scores the workgroup has just written, then the
// in-place compaction.  `rows` holds n score rows of the N - P candidates
// (stride apart), merged by their maximum: one row for a head-cache, or the H
// heads of a (layer, request) with shared positions.  The selection is
// applied to the n heads x.head0 .. x.head0 + n - 1 (pos0: the first one's
// pos ids row).  Same results as topk_select_kernel (or its shared form)
// followed by kv_compact_kernel: the prompt is kept, the B - P best
// candidates survive with ties to the earlier slot, and the survivors move to
// the front in slot order.
template <int kThreads>
__device__ void select_compact(const CacheView& c, int layer, int head0, int n, int N, int P,
                               int B, const float* rows, int stride, const int* s_bt,
                               uint8_t* scratch, int32_t* keep_row, int32_t* pos0,
                               int pos_stride) {
    const int tid = threadIdx.x;
    if (N <= B) {  // nothing to evict: every slot stays where it is
        if (keep_row)
            for (int i = tid; i < B; i += kThreads) keep_row[i] = (i < N) ? i : -1;
        return;
    }
    if (keep_row)
        for (int i = tid; i < P; i += kThreads) keep_row[i] = i;
    const int m = N - P, k = B - P;
    if (k == 0) return;  // only the prompt survives, and it does not move
    int* s_wsum = reinterpret_cast<int*>(scratch + kFuseWsumOff);
    uint32_t* s_key = reinterpret_cast<uint32_t*>(scratch + kFuseKeyOff);
    __syncthreads();  // the scores written by group 0 are visible to every thread
    for (int i = tid; i < m; i += kThreads) {
        uint32_t v = 0;
        for (int h = 0; h < n; ++h) {
            const uint32_t w = __float_as_uint(rows[(size_t)h * stride + i]);
            v = max(v, (w >> 31) ? 0u : w);  // non-negative fp32 orders like its bits
        }
        s_key[i] = v;
    }
    // Four rounds per barrier (64 rows with 256 threads): shorter rounds than
    // the standalone compaction's interleave better with the CU's other
    // workgroup, which is scoring (about 2% faster than eight at the serving
    // shape).
    select_and_move<kThreads, 4>(c, layer, head0, n, P, B, m, s_key,
                                 reinterpret_cast<int*>(s_key + m),
                                 reinterpret_cast<RadixScratch*>(scratch), s_wsum,
                                 s_wsum + kThreads / kWave, s_bt, keep_row, pos0, pos_stride);
}

// What the score body does after scoring: nothing, the per-head selection
// and compaction, or (shared positions) the selection and compaction of the
// (layer, request) once its last head is scored.
// kSplitLse / kSplitScore: a head-cache's keys split over `nparts` workgroups
// in two launches -- each part reduces its share of the key tiles to a
// log-sum-exp per row (kSplitLse, written to part_lse), then each part merges
// the partials and scores its share of the candidate tiles (kSplitScore).
enum { kScoreOnly = 0, kEvictHead = 1, kEvictShared = 2, kSplitLse = 3, kSplitScore = 4 };
// row stride of the per-part log-sum-exp partials (log2 units)
constexpr int kPartRow = BKV_MAX_BEACONS;

// The body of the kernels below, for head-cache hc: NG row groups of NQ waves
// (NQ tile phases), MBW 32-row blocks per wave; kMode as above (budget B,
// nullable keep_out and pos_ids rows).  Returns false when the request fails
// its checks.
template <int NG, int NQ, int MBW, int kMode>
__device__ __forceinline__ bool score_head(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    int window, float bonus, float* __restrict__ scores, int stride, float* __restrict__ lse_out,
    int B, int32_t* __restrict__ keep_out, int32_t* __restrict__ pos_ids, int pos_stride,
    Check ck, int32_t* status, const int hc, const int part = 0, const int nparts = 1,
    float* __restrict__ part_lse = nullptr) {
    constexpr int kGroups = NG, kQ = NQ, kWaves = NG * NQ;
    constexpr bool kScoreLike = kMode == kScoreOnly || kMode == kSplitLse || kMode == kSplitScore;
    // the streaming ring; the fused kernels reuse it for the selection, which
    // needs 64 KiB, so a one-phase layout allocates more than it streams
    constexpr int kRingTiles =
        (!kScoreLike && kQ * kRingIters < 8) ? 8 : kQ * kRingIters;
    static_assert(kScoreLike ||
                      kRingTiles * kTileBytes >= kFuseKeyOff + 4 * kFusedMaxEntries,
                  "the ring cannot hold the fused selection");
    static_assert(kWaves <= 16, "fused scan slots");
    __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kRingTiles * kTileBytes];
    __shared__ int s_bt[kMaxBlocksPerReq];
    __shared__ float s_part[kWaves][32 * MBW];  // per wave, its own rows
    __shared__ float s_M[kWaves];
    __shared__ float s_lse2[BKV_MAX_BEACONS];
    __shared__ float s_ref[BKV_MAX_BEACONS];
    __shared__ int s_live[BKV_MAX_BEACONS];
    __shared__ float s_pmax[3][kGroups - 1][kQ][32];
    __shared__ int s_rescue;

    const HeadIdx x = split_hc(c, hc);
    if (!request_ok(c, x.layer, x.req, hc, ck, status)) return false;
    const int N = slot_count(c, hc, x.req);
    const int P = c.prompt_len[x.req];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int lane = tid & (kWave - 1);
    const int hh = lane >> 5;
    const int col = lane & 31;
    const int group = w / kQ;
    const int q = w % kQ;
    const bool loader = group == kGroups - 1;
    const int Kp = (K + 31) & ~31;
    const int MB = Kp / 32;
    const int mb0 = group * MBW;
    const bool computes = mb0 < MB;

    const int nb = (N + kBlock - 1) / kBlock;
    const int32_t* bt = table_row(c, hc, x.req);
    for (int i = tid; i < nb; i += blockDim.x) s_bt[i] = bt[i];
    for (int j = tid; j < Kp; j += blockDim.x)
        s_live[j] = (j < K) && counts[(size_t)hc * K + j] > 0;
    if (tid == 0) s_rescue = 0;
    __syncthreads();

    // the keep-list row: per head-cache, or per (layer, request) when shared
    int32_t* keep_row = nullptr;
    if (!kScoreLike && keep_out)
        keep_row = keep_out + (size_t)(kMode == kEvictShared ? hc / c.H : hc) * B;
    const bool last_head = x.head == c.H - 1;
    if (N == 0) {  // empty cache: nothing to score, every live lse is log(0)
        if constexpr (kMode == kSplitLse) {
            for (int j = tid; j < K; j += blockDim.x)
                part_lse[((size_t)hc * nparts + part) * kPartRow + j] = -INFINITY;
            return true;
        }
        for (int j = tid; j < K; j += blockDim.x)
            if (lse_out && part == 0)
                lse_out[(size_t)hc * K + j] = s_live[j] ? -INFINITY : __int_as_float(0x7fc00000);
        if (kMode == kEvictHead || (kMode == kEvictShared && last_head))
            for (int i = tid; i < B; i += blockDim.x)
                if (keep_row) keep_row[i] = -1;
        return true;
    }

    // a scalar load: a vector one would still count as outstanding inside the
    // ring loop below and make the loaders wait for their ring loads there
    const uint64_t kpool =
        *(const __attribute__((address_space(4))) uint64_t*)(c.k_pools + x.layer);
    const int ntiles = (N + kTileKeys - 1) / kTileKeys;
    // Phase 2 scores only the candidates [P, N): its tiles start at the one
    // holding slot P.
    const int t2 = P / kTileKeys;
    const int ntiles2 = ntiles - t2;
    // this workgroup's tiles: phase 1 over [p1a, p1a + p1n), phase 2 over
    // [p2a, p2a + p2n) (a split part takes its share of one of them)
    int p1a = 0, p1n = ntiles, p2a = t2, p2n = ntiles2;
    if constexpr (kMode == kSplitLse) {
        p1a = ntiles * part / nparts;
        p1n = ntiles * (part + 1) / nparts - p1a;
        p2n = 0;
    }
    if constexpr (kMode == kSplitScore) {
        const int a = ntiles2 * part / nparts;
        p1n = 0;
        p2a = t2 + a;
        p2n = ntiles2 * (part + 1) / nparts - a;
    }
    if (kMode == kSplitLse && p1n == 0) {  // no keys in this part: log(0)
        for (int j = tid; j < K; j += blockDim.x)
            part_lse[((size_t)hc * nparts + part) * kPartRow + j] = -INFINITY;
        return true;
    }
    const int iters = (p1n + kQ - 1) / kQ;   // phase-1 iterations
    const int iters2 = (p2n + kQ - 1) / kQ;  // phase-2 iterations
    const int G = iters + iters2;            // the stream: phase 1, then phase 2
    // last iteration of a phase in which this wave's phase q has a tile (-1 if none)
    const int jlast = (q < p1n) ? (p1n - 1 - q) / kQ : -1;
    const int jlast2 = (q < p2n) ? (p2n - 1 - q) / kQ : -1;

    // DMA of key tile t into ring slot `slot` (issued by a group-1 wave).  Lane
    // l of instruction i fills LDS bytes [1024 i + 16 l, +16) of the slot: row
    // r = 4i + l/16, chunk position p = l%16, which holds global chunk
    // p ^ (r & 15) of key 32t + r (key N-1 past the end, so a tile past the
    // last one re-reads one cached row and is never consumed).
    const uint32_t ring0 = lds_addr(s_ring);
    auto issue_tile = [&](int t, int slot) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(ring0 + slot * kTileBytes);
        // Every row of a tile lies in block 2t (rows 0-15) or 2t+1 (rows
        // 16-31), clamped rows included, and a tile past the end reads the
        // last block.
        const int b_lo = __builtin_amdgcn_readfirstlane(s_bt[min(2 * t, nb - 1)]);
        const int b_hi = __builtin_amdgcn_readfirstlane(s_bt[min(2 * t + 1, nb - 1)]);
        const uint64_t base_lo = kpool + row_offset(b_lo, c.H, x.head, 0);
        const uint64_t base_hi = kpool + row_offset(b_hi, c.H, x.head, 0);
#pragma unroll
        for (int i = 0; i < kDmaPerTile; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int ch = (lane & 15) ^ (r & 15);
            const int n = min(kTileKeys * t + r, N - 1);
            const uint32_t off = (uint32_t)(n & (kBlock - 1)) * kRowBytes + 16 * ch;
            dma16((i < kDmaPerTile / 2 ? base_lo : base_hi) + off, dst + 1024 * i);
        }
    };
    // Stream iteration g covers tile NQ j + q of phase 1 (g < iters, j = g)
    // or tile t2 + NQ j + q of phase 2 (j = g - iters).  Every loader issues
    // one tile per iteration, so a wave's outstanding loads are always whole
    // iterations.
    auto slot_of = [&](int g) { return (g % kRingIters) * kQ + q; };
    auto tile_of = [&](int g) { return g < iters ? p1a + kQ * g + q : p2a + kQ * (g - iters) + q; };
    // this lane's key column from a ring slot: the B fragment of k-step s is
    // global chunk 2s + hh of row `col`
    auto read_tile = [&](Tile& t, int slot) {
        const uint8_t* row = s_ring + slot * kTileBytes + col * kRowBytes;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int p = (2 * s + hh) ^ (col & 15);
            t.b[s] = *reinterpret_cast<const bf16x8_t*>(row + 16 * p);
        }
    };
    // hand-over of iteration g: the loaders wait for their DMA of g, all waves
    // pass the barrier (iteration g-1's reads are then done), and the slot read
    // in g-1 is refilled with iteration g + kDepth
    auto begin_iter = [&](int g) {
        if (loader) wait_ring(min(kDepth - 1, G - 1 - g));
        ring_barrier();
        if (loader && g + kDepth < G) issue_tile(tile_of(g + kDepth), slot_of(g + kDepth));
    };

    // A fragments: beacon row 32*(mb0+m) + col, bf16 (RNE) of the fp32 state.
    // Dead rows, and the rows of blocks past K, load row 0 (always present)
    // and are zeroed.  The loads of the first blocks (both of two, one of four)
    // go out before the first ring tiles and are converted on every path: the
    // compiler, which does not see the ring loads, would otherwise count them
    // as outstanding inside the ring loop and make the loaders wait there for
    // their own ring loads.
    bf16x8_t A[MBW][8];
    auto row_live = [&](int m) {
        const int j = 32 * (mb0 + m) + col;
        return mb0 + m < MB && s_live[j < BKV_MAX_BEACONS ? j : 0];
    };
    auto load_block = [&](int m, float4 (&r)[8][2]) {
        const int j = 32 * (mb0 + m) + col;
        const float* br = beacons + ((size_t)hc * K + (row_live(m) ? j : 0)) * kHeadDim + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            r[s][0] = *reinterpret_cast<const float4*>(br + 16 * s);
            r[s][1] = *reinterpret_cast<const float4*>(br + 16 * s + 4);
        }
    };
    auto convert_block = [&](int m, const float4 (&r)[8][2]) {
        const uint32_t keep = row_live(m) ? 0xffffffffu : 0u;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float4 lo = r[s][0], hi = r[s][1];
            u32x4 pk;
            pk.x = ((uint32_t)to_bf16_rne(lo.x) | ((uint32_t)to_bf16_rne(lo.y) << 16)) & keep;
            pk.y = ((uint32_t)to_bf16_rne(lo.z) | ((uint32_t)to_bf16_rne(lo.w) << 16)) & keep;
            pk.z = ((uint32_t)to_bf16_rne(hi.x) | ((uint32_t)to_bf16_rne(hi.y) << 16)) & keep;
            pk.w = ((uint32_t)to_bf16_rne(hi.z) | ((uint32_t)to_bf16_rne(hi.w) << 16)) & keep;
            A[m][s] = as_bf16x8(pk);
        }
    };
    constexpr int kPre = MBW <= 2 ? MBW : 1;
    float4 raw[kPre][8][2];
#pragma unroll
    for (int m = 0; m < kPre; ++m) load_block(m, raw[m]);
    if (loader)  // the first ring tiles are in flight while the beacons are prepared
        for (int g = 0; g < kDepth && g < G; ++g) issue_tile(tile_of(g), slot_of(g));
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
        if (m < kPre) {
            convert_block(m, raw[m < kPre ? m : 0]);
        } else if (mb0 + m < MB) {
            float4 r[8][2];
            load_block(m, r);
            convert_block(m, r);
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) A[m][s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
    }
    uint32_t live_bits[MBW];
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
        uint32_t bits = 0;
        if (mb0 + m < MB) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                bits |= (uint32_t)(s_live[32 * (mb0 + m) + acc_row(i, hh)] != 0) << i;
        }
        live_bits[m] = bits;
    }
    const f32x16_t zero = {};

    // ---------------- phase 1: per-row log-sum-exp ----------------
    float Mw = -INFINITY;  // wave reference (log2 units), from the wave's first tile
    float sum[MBW][16];
#pragma unroll
    for (int m = 0; m < MBW; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum[m][i] = 0.f;

    for (int it = 0; it < iters; ++it) {
        begin_iter(it);  // stream iteration g = it
        if (!computes || it > jlast) continue;
        const int tt = p1a + kQ * it + q;
        const int n = kTileKeys * tt + col;
        Tile t;
        read_tile(t, slot_of(it));
        if (it == 0) {  // the wave's reference: max live logit of its first tile
            float mx = -INFINITY;
#pragma unroll
            for (int m = 0; m < MBW; ++m) {
                if (mb0 + m >= MB) continue;
                const f32x16_t acc = logits(A[m], t, zero);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (((live_bits[m] >> i) & 1u) && n < N) mx = fmaxf(mx, acc[i]);
            }
            mx = wave_max(mx);
            Mw = (mx == -INFINITY) ? 0.f : mx * kCs;
        }
        const bool full = kTileKeys * tt + kTileKeys <= N;
#pragma unroll
        for (int m = 0; m < MBW; ++m) {
            if (mb0 + m >= MB) continue;
            const f32x16_t acc = logits(A[m], t, zero);
            if (full) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sum[m][i] += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], kCs, -Mw));
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], kCs, -Mw));
                    sum[m][i] += (n < N) ? e : 0.f;
                }
            }
        }
    }
    if constexpr (kMode == kSplitScore) {
        // the parts' log-sum-exps, merged: lse = m + log2(sum 2^(lse_s - m))
        const float* pl = part_lse + (size_t)hc * nparts * kPartRow;
        for (int j = tid; j < Kp; j += blockDim.x) {
            float m = -INFINITY, total = 0.f;
            if (j < K) {
                for (int p2 = 0; p2 < nparts; ++p2) m = fmaxf(m, pl[p2 * kPartRow + j]);
                if (m != -INFINITY)
                    for (int p2 = 0; p2 < nparts; ++p2) total += exp2f(pl[p2 * kPartRow + j] - m);
            }
            s_lse2[j] = s_live[j] ? (m == -INFINITY ? -INFINITY : m + log2f(total)) : INFINITY;
        }
        ring_barrier();
    } else {
        // lanes -> waves -> rows.  The first phase-2 tiles are in flight, so the
        // exchange uses ring barriers (LDS only) rather than fenced ones.
    #pragma unroll
        for (int m = 0; m < MBW; ++m) {
            if (mb0 + m >= MB) continue;
    #pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float v = half_sum(sum[m][i]);
                if (col == kHalfLead) s_part[w][32 * m + acc_row(i, hh)] = v;
            }
        }
        if (lane == 0) s_M[w] = (jlast >= 0 && computes) ? Mw : -INFINITY;
        ring_barrier();
        // row j belongs to group g = (j / 32) / MBW, at local row lj of its waves
        for (int j = tid; j < Kp; j += blockDim.x) {
            const int g = (j / 32) / MBW;
            const int lj = j - 32 * MBW * g;
            float Mg = -INFINITY;
            for (int k2 = 0; k2 < kQ; ++k2) Mg = fmaxf(Mg, s_M[g * kQ + k2]);
            float total = 0.f;
            for (int k2 = 0; k2 < kQ; ++k2) {
                const float Mk = s_M[g * kQ + k2];
                if (Mk != -INFINITY) total += s_part[g * kQ + k2][lj] * exp2f(Mk - Mg);
            }
            const bool lv = s_live[j];
            const bool ok = total >= 0x1p-100f && total < INFINITY;
            if (lv && !ok) s_rescue = 1;
            s_lse2[j] = lv ? Mg + log2f(total) : INFINITY;
        }
        ring_barrier();

        if (s_rescue) {
            // Exact fallback with direct loads: per-row maximum over all keys
            // first, then the sums against it (every term <= 1, the maximum == 1).
    #pragma unroll
            for (int m = 0; m < MBW; ++m)
    #pragma unroll
                for (int i = 0; i < 16; ++i) sum[m][i] = -INFINITY;
            if (computes) {
                for (int tt = p1a + q; tt < p1a + p1n; tt += kQ) {
                    Tile t;
                    const int n = kTileKeys * tt + col;
                    load_key(t, kpool, s_bt, c.H, x.head, n, N, hh);
    #pragma unroll
                    for (int m = 0; m < MBW; ++m) {
                        if (mb0 + m >= MB) continue;
                        const f32x16_t acc = logits(A[m], t, zero);
    #pragma unroll
                        for (int i = 0; i < 16; ++i)
                            if (n < N) sum[m][i] = fmaxf(sum[m][i], acc[i]);
                    }
                }
            }
    #pragma unroll
            for (int m = 0; m < MBW; ++m) {
                if (mb0 + m >= MB) continue;
    #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float v = half_max(sum[m][i]);
                    if (col == kHalfLead) s_part[w][32 * m + acc_row(i, hh)] = v;
                }
            }
            __syncthreads();
            for (int j = tid; j < Kp; j += blockDim.x) {
                const int g = (j / 32) / MBW;
                const int lj = j - 32 * MBW * g;
                float R = -INFINITY;
                for (int k2 = 0; k2 < kQ; ++k2) R = fmaxf(R, s_part[g * kQ + k2][lj]);
                s_ref[j] = R * kCs;
            }
            __syncthreads();
    #pragma unroll
            for (int m = 0; m < MBW; ++m) {
                if (mb0 + m >= MB) continue;
                float ref[16], acc_sum[16];
    #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    ref[i] = s_ref[32 * (mb0 + m) + acc_row(i, hh)];
                    acc_sum[i] = 0.f;
                }
                for (int tt = p1a + q; tt < p1a + p1n; tt += kQ) {
                    Tile t;
                    const int n = kTileKeys * tt + col;
                    load_key(t, kpool, s_bt, c.H, x.head, n, N, hh);
                    const f32x16_t acc = logits(A[m], t, zero);
    #pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], kCs, -ref[i]));
                        acc_sum[i] += (n < N) ? e : 0.f;
                    }
                }
    #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float v = half_sum(acc_sum[i]);
                    if (col == kHalfLead) s_part[w][32 * m + acc_row(i, hh)] = v;
                }
            }
            __syncthreads();
            for (int j = tid; j < Kp; j += blockDim.x) {
                const int g = (j / 32) / MBW;
                const int lj = j - 32 * MBW * g;
                float total = 0.f;
                for (int k2 = 0; k2 < kQ; ++k2) total += s_part[g * kQ + k2][lj];
                s_lse2[j] = s_live[j] ? s_ref[j] + log2f(total) : INFINITY;
            }
            __syncthreads();
        }
    }
    if constexpr (kMode == kSplitLse) {
        for (int j = tid; j < K; j += blockDim.x)
            part_lse[((size_t)hc * nparts + part) * kPartRow + j] = s_live[j] ? s_lse2[j] : INFINITY;
        // the ring loads issued past this part's phase 1 (none: the stream
        // ends with it) have all landed before the loaders' last hand-over
        return true;
    }
    // written by group 0, which issues no ring loads
    if (lse_out && group == 0 && part == 0) {
        for (int j = tid; j < K; j += kQ * kWave)
            lse_out[(size_t)hc * K + j] = s_live[j] ? s_lse2[j] * kLn2 : __int_as_float(0x7fc00000);
    }

    // ---------------- phase 2: sigma(n) = exp(max_j s_jn - lse_j) ----------------
    f32x16_t Cf[MBW];
#pragma unroll
    for (int m = 0; m < MBW; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float l2 = (mb0 + m < MB) ? s_lse2[32 * (mb0 + m) + acc_row(i, hh)] : INFINITY;
            Cf[m][i] = -l2 * kInvCs;
        }
    float* out = scores + (size_t)hc * stride;
    // The other groups' partial maxima of tile j pass through s_pmax[j % 3];
    // group 0 finishes tile j once they have crossed a barrier.
    auto finalize = [&](int j, float mx) {
        const int n = kTileKeys * (p2a + kQ * j + q) + col;
        if (j <= jlast2 && hh == 0 && n >= P && n < N) {
#pragma unroll
            for (int g = 0; g < kGroups - 1; ++g) mx = fmaxf(mx, s_pmax[j % 3][g][q][col]);
            const float sigma = __builtin_amdgcn_exp2f(mx * kCs);
            out[n - P] = sigma + ((n >= N - window) ? bonus : 0.f);
        }
    };
    auto publish = [&](int j, float mx) {
        if (group > 0 && hh == 0) s_pmax[j % 3][group - 1][q][col] = mx;
    };
    float mx_prev = -INFINITY;
    for (int it = 0; it < iters2; ++it) {
        begin_iter(iters + it);  // stream iteration g = iters + it
        if (group == 0 && it > 0) finalize(it - 1, mx_prev);
        float mx = -INFINITY;
        if (it <= jlast2 && computes) {
            Tile t;
            read_tile(t, slot_of(iters + it));
#pragma unroll
            for (int m = 0; m < MBW; ++m) {
                if (mb0 + m >= MB) continue;
                const f32x16_t acc = logits(A[m], t, Cf[m]);
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[i]);
            }
            mx = max_halves(mx);
        }
        publish(it, mx);
        mx_prev = mx;
    }
    ring_barrier();
    if (group == 0 && iters2 > 0) finalize(iters2 - 1, mx_prev);
    // Every ring load has landed (the loaders waited for all of them before
    // the last hand-over) and every ring read is done: the ring is free.
    if constexpr (kMode == kEvictHead)
        select_compact<kWaves * kWave>(c, x.layer, x.head, 1, N, P, B, out, stride, s_bt,
                                       s_ring, keep_row,
                                       pos_ids ? pos_ids + (size_t)hc * pos_stride : nullptr,
                                       pos_stride);
    if constexpr (kMode == kEvictShared)
        if (last_head)  // every head of the (layer, request) is scored
            select_compact<kWaves * kWave>(
                c, x.layer, 0, c.H, N, P, B, scores + (size_t)(hc - x.head) * stride, stride,
                s_bt, s_ring, keep_row,
                pos_ids ? pos_ids + (size_t)(hc - x.head) * pos_stride : nullptr, pos_stride);
    return true;
}

// Scoring alone (WPE: register budget for that many waves per SIMD).
template <int NG, int NQ, int MBW, int WPE>
__global__ __launch_bounds__(NG * NQ * kWave, WPE) void beacon_score_kernel(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    int window, float bonus, float* __restrict__ scores, int stride, float* __restrict__ lse_out,
    int B, int32_t* __restrict__ keep_out, int32_t* __restrict__ pos_ids, int pos_stride,
    Check ck, int32_t* status) {
    score_head<NG, NQ, MBW, kScoreOnly>(c, beacons, counts, K, window, bonus, scores, stride,
                                        lse_out, B, keep_out, pos_ids, pos_stride, ck, status,
                                        blockIdx.x);
}

// Scoring, selection and compaction of each head-cache by its workgroup.
template <int NG, int NQ, int MBW, int WPE>
__global__ __launch_bounds__(NG * NQ * kWave, WPE) void beacon_evict_kernel(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    int window, float bonus, float* __restrict__ scores, int stride, float* __restrict__ lse_out,
    int B, int32_t* __restrict__ keep_out, int32_t* __restrict__ pos_ids, int pos_stride,
    Check ck, int32_t* status) {
    score_head<NG, NQ, MBW, kEvictHead>(c, beacons, counts, K, window, bonus, scores, stride,
                                        lse_out, B, keep_out, pos_ids, pos_stride, ck, status,
                                        blockIdx.x);
}

// Shared positions: one workgroup per (layer, request) scores its H heads in
// turn, then selects once and compacts every head.
template <int NG, int NQ, int MBW, int WPE>
__global__ __launch_bounds__(NG * NQ * kWave, WPE) void beacon_evict_shared_kernel(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    int window, float bonus, float* __restrict__ scores, int stride, float* __restrict__ lse_out,
    int B, int32_t* __restrict__ keep_out, int32_t* __restrict__ pos_ids, int pos_stride,
    Check ck, int32_t* status) {
    for (int h = 0; h < c.H; ++h) {
        if (h) __syncthreads();  // the previous head's body is done with every LDS array
        if (!score_head<NG, NQ, MBW, kEvictShared>(c, beacons, counts, K, window, bonus, scores,
                                                   stride, lse_out, B, keep_out, pos_ids,
                                                   pos_stride, ck, status, blockIdx.x * c.H + h))
            return;
    }
}

// A head-cache's keys split over `nparts` workgroups (workgroup b takes part
// b % nparts of head-cache b / nparts): the partial log-sum-exps of each
// part's key tiles ...
template <int NG, int NQ, int MBW, int WPE>
__global__ __launch_bounds__(NG * NQ * kWave, WPE) void beacon_lse_split_kernel(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    float* __restrict__ part_lse, int nparts, Check ck, int32_t* status) {
    score_head<NG, NQ, MBW, kSplitLse>(c, beacons, counts, K, 0, 0.f, nullptr, 0, nullptr, 0,
                                       nullptr, nullptr, 0, ck, status, blockIdx.x / nparts,
                                       blockIdx.x % nparts, nparts, part_lse);
}

// ... then, after they are merged, each part's share of the candidate scores.
template <int NG, int NQ, int MBW, int WPE>
__global__ __launch_bounds__(NG * NQ * kWave, WPE) void beacon_score_split_kernel(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    int window, float bonus, float* __restrict__ scores, int stride, float* __restrict__ lse_out,
    float* __restrict__ part_lse, int nparts, Check ck, int32_t* status) {
    score_head<NG, NQ, MBW, kSplitScore>(c, beacons, counts, K, window, bonus, scores, stride,
                                         lse_out, 0, nullptr, nullptr, 0, ck, status,
                                         blockIdx.x / nparts, blockIdx.x % nparts, nparts,
                                         part_lse);
}

template <int NG, int NQ, int MBW, int WPE>
void launch_split_cfg(const CacheView& c, const float* beacons, const int32_t* counts, int K,
                      int window, float bonus, float* scores, int stride, float* lse,
                      float* part_lse, int nparts, Check ck, int32_t* status, hipStream_t s) {
    const unsigned grid = (unsigned)(c.L * c.R * c.H) * (unsigned)nparts;
    hipLaunchKernelGGL((beacon_lse_split_kernel<NG, NQ, MBW, WPE>), dim3(grid),
                       dim3(NG * NQ * kWave), 0, s, c, beacons, counts, K, part_lse, nparts, ck,
                       status);
    hipLaunchKernelGGL((beacon_score_split_kernel<NG, NQ, MBW, WPE>), dim3(grid),
                       dim3(NG * NQ * kWave), 0, s, c, beacons, counts, K, window, bonus, scores,
                       stride, lse, part_lse, nparts, ck, status);
}

template <int NG, int NQ, int MBW, int WPE, int kMode>
void launch_cfg(const CacheView& c, const float* beacons, const int32_t* counts, int K,
                int window, float bonus, float* scores, int stride, float* lse, int B,
                int32_t* keep_out, int32_t* pos_ids, int pos_stride, Check ck, int32_t* status,
                hipStream_t s) {
    if constexpr (kMode == kEvictShared)
        hipLaunchKernelGGL((beacon_evict_shared_kernel<NG, NQ, MBW, WPE>), dim3(c.L * c.R),
                           dim3(NG * NQ * kWave), 0, s, c, beacons, counts, K, window, bonus,
                           scores, stride, lse, B, keep_out, pos_ids, pos_stride, ck, status);
    else if constexpr (kMode == kEvictHead)
        hipLaunchKernelGGL((beacon_evict_kernel<NG, NQ, MBW, WPE>), dim3(c.L * c.R * c.H),
                           dim3(NG * NQ * kWave), 0, s, c, beacons, counts, K, window, bonus,
                           scores, stride, lse, B, keep_out, pos_ids, pos_stride, ck, status);
    else
        hipLaunchKernelGGL((beacon_score_kernel<NG, NQ, MBW, WPE>), dim3(c.L * c.R * c.H),
                           dim3(NG * NQ * kWave), 0, s, c, beacons, counts, K, window, bonus,
                           scores, stride, lse, B, keep_out, pos_ids, pos_stride, ck, status);
}

// Layouts measured at 2112 keys per head-cache (two workgroups per CU in
// each case):
//   K <= 64 : 2 groups x 2 phases, 32 rows per wave (4 waves per workgroup)
//   K <= 128: 2 groups x 2 phases, 64 rows per wave; every tile is read
//             from LDS by two waves (four 32-row waves took 5% longer)
//   K <= 256: 8 groups x 1 phase, 32 rows per wave (8 waves of 112
//             registers: two workgroups per CU, where 4 groups x 2 phases of
//             64-row waves, with 199 registers, allowed one; 8.25 against
//             9.07 ms for the 64-layer B = 2048 fused pass).  Every tile is
//             read from LDS by all 8 waves.  With shared positions the
//             kernel's extra state does not fit 128 registers, so it runs
//             the same layout (the layout fixes the summation order, and the
//             fused kernels must reproduce the separate ones) with more
//             registers, one workgroup per CU.
template <int kMode>
hipError_t launch_any(const CacheView& c, const float* beacons, const int32_t* counts, int K,
                      int window, float bonus, float* scores, int stride, float* lse, int B,
                      int32_t* keep_out, int32_t* pos_ids, int pos_stride, Check ck,
                      int32_t* status, hipStream_t s) {
    if (c.L * c.R * c.H == 0) return hipSuccess;
    // At most one workgroup per CU (a small batch, a single head-cache): with
    // K <= 128, four tile phases instead of two keep twice the key tiles in
    // flight in the CU's one workgroup (the ring takes 128 KiB; one workgroup
    // per CU fits).  The fused kernel of one 4096-key head-cache at K = 64
    // took 100 us instead of 146.  At K = 256 the 4 x 2 layout of 64-row
    // waves serves such launches (1.44 against 2.00 ms for the 32k layer's
    // scoring: the one-phase layout reads every tile 8 times and gains
    // nothing without a second workgroup on the CU).  The layout fixes the
    // order of the log-sum-exp sums, so it is chosen from the head-cache
    // count for every kernel, the shared-position ones included: a fused pass
    // then reproduces its separate kernels bit for bit.
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    const long units = (long)c.L * c.R * c.H;
    if (units <= cus && K > 128) {
        launch_cfg<4, 2, 2, 2, kMode>(c, beacons, counts, K, window, bonus, scores, stride, lse, B,
                                      keep_out, pos_ids, pos_stride, ck, status, s);
        return hipGetLastError();
    }
    if (units <= cus) {
        if (K <= 64)
            launch_cfg<2, 4, 1, 2, kMode>(c, beacons, counts, K, window, bonus, scores, stride, lse,
                                          B, keep_out, pos_ids, pos_stride, ck, status, s);
        else
            launch_cfg<2, 4, 2, 2, kMode>(c, beacons, counts, K, window, bonus, scores, stride, lse,
                                          B, keep_out, pos_ids, pos_stride, ck, status, s);
        return hipGetLastError();
    }
    if (K <= 64)
        launch_cfg<2, 2, 1, 2, kMode>(c, beacons, counts, K, window, bonus, scores, stride, lse, B,
                                      keep_out, pos_ids, pos_stride, ck, status, s);
    else if (K <= 128)
        launch_cfg<2, 2, 2, 2, kMode>(c, beacons, counts, K, window, bonus, scores, stride, lse, B,
                                      keep_out, pos_ids, pos_stride, ck, status, s);
    else if (kMode == kEvictShared)  // the same layout (hence the same scores), more registers
        launch_cfg<8, 1, 1, 2, kMode>(c, beacons, counts, K, window, bonus, scores, stride, lse, B,
                                      keep_out, pos_ids, pos_stride, ck, status, s);
    else
        launch_cfg<8, 1, 1, 4, kMode>(c, beacons, counts, K, window, bonus, scores, stride, lse, B,
                                      keep_out, pos_ids, pos_stride, ck, status, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_beacon_score(const CacheView& c, const float* beacons, const int32_t* counts,
                               int K, int window, float bonus, float* scores, int stride,
                               float* lse, Check ck, int32_t* status, hipStream_t s) {
    return launch_any<kScoreOnly>(c, beacons, counts, K, window, bonus, scores, stride, lse, 0,
                                  nullptr, nullptr, 0, ck, status, s);
}

hipError_t launch_beacon_score_split(const CacheView& c, const float* beacons,
                                     const int32_t* counts, int K, int window, float bonus,
                                     float* scores, int stride, float* lse, float* part_lse,
                                     int nparts, Check ck, int32_t* status, hipStream_t s) {
    if (c.L * c.R * c.H == 0) return hipSuccess;
    // the workgroups of every part fill the chip, so the layouts of wide
    // launches serve (at K = 256, two workgroups per CU)
    if (K <= 64)
        launch_split_cfg<2, 2, 1, 2>(c, beacons, counts, K, window, bonus, scores, stride, lse,
                                     part_lse, nparts, ck, status, s);
    else if (K <= 128)
        launch_split_cfg<2, 2, 2, 2>(c, beacons, counts, K, window, bonus, scores, stride, lse,
                                     part_lse, nparts, ck, status, s);
    else
        launch_split_cfg<8, 1, 1, 4>(c, beacons, counts, K, window, bonus, scores, stride, lse,
                                     part_lse, nparts, ck, status, s);
    return hipGetLastError();
}

hipError_t launch_beacon_evict(const CacheView& c, const float* beacons, const int32_t* counts,
                               int K, int window, float bonus, float* scores, int stride,
                               float* lse, int budget, int32_t* keep_out, int32_t* pos_ids,
                               int pos_stride, Check ck, int32_t* status, hipStream_t s) {
    return launch_any<kEvictHead>(c, beacons, counts, K, window, bonus, scores, stride, lse,
                                  budget, keep_out, pos_ids, pos_stride, ck, status, s);
}

hipError_t launch_beacon_evict_shared(const CacheView& c, const float* beacons,
                                      const int32_t* counts, int K, int window, float bonus,
                                      float* scores, int stride, float* lse, int budget,
                                      int32_t* keep_out, int32_t* pos_ids, int pos_stride,
                                      Check ck, int32_t* status, hipStream_t s) {
    return launch_any<kEvictShared>(c, beacons, counts, K, window, bonus, scores, stride, lse,
                                    budget, keep_out, pos_ids, pos_stride, ck, status, s);
}

}  // namespace bkv
