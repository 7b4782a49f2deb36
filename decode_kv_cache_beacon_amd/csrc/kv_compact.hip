// kv_compact.hip -- in-place, order-preserving compaction of a paged bf16 KV
// cache (the cache-compaction step every selector shares; Random Attention
// article, section "发现四").
//
// One workgroup per head-cache.  Survivor i moves from slot keep[i] >= i to
// slot i.  The keep list is strictly ascending, so every source slot of a
// later chunk lies beyond every destination slot of the current chunk; a
// workgroup walks the survivors in ascending chunks of kRowsPerIter rows,
// reads the whole chunk (K, V and pos ids) into registers, waits at a barrier
// and only then writes the chunk.  That makes the in-place move race-free
// without a second buffer.  Rows before the first evicted slot (the prompt at
// least) are never touched.
//
// Memory: a row is 256 contiguous bytes; 16 lanes move one row with 16-byte
// accesses, so each wave instruction moves 4 whole rows (1 KiB).  The rows
// are touched once, so loads and stores are non-temporal.
//
// With shared positions every head of a (layer, request) applies the one keep
// list of that (layer, request).

#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerRow = kRowBytes / 16;               // 16 x 16-byte pieces
constexpr int kRowsPerRound = kThreads / kChunksPerRow;     // 16 rows per instruction round
constexpr int kRounds = 8;
constexpr int kRowsPerIter = kRowsPerRound * kRounds;       // 128 rows per barrier

__global__ __launch_bounds__(kThreads) void kv_compact_kernel(CacheView c,
                                                              const int32_t* __restrict__ keep,
                                                              int B, int keep_shared,
                                                              int32_t* __restrict__ pos_ids,
                                                              int pos_stride, Check ck,
                                                              int32_t* status) {
    const int hc = blockIdx.x;
    const HeadIdx x = split_hc(c, hc);
    if (!request_ok(c, x.layer, x.req, ck, status)) return;

    const int N = c.seq_len[x.req];
    const int nk = min(N, B);
    const int32_t* kp = keep + (size_t)(keep_shared ? hc / c.H : hc) * B;

    // The keep list must be strictly ascending inside [0, N): that is what
    // keeps every access in bounds and the in-place move race-free.
    __shared__ int s_first;
    __shared__ int s_bt[kMaxBlocksPerReq];
    if (threadIdx.x == 0) s_first = nk;
    bool bad = false;
    int first = nk;
    for (int i = threadIdx.x; i < nk; i += kThreads) {
        const int v = kp[i];
        const int prev = i ? kp[i - 1] : -1;
        bad |= (v <= prev) || (v >= N);
        if (v != i) first = min(first, i);
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        if (threadIdx.x == 0) raise_status(status, 1 << BKV_ERR_INVALID);
        return;
    }
    if (first < nk) atomicMin(&s_first, first);
    __syncthreads();
    const int i0 = s_first;
    if (i0 >= nk) return;

    const uint64_t kbase = c.k_pools[x.layer];
    const uint64_t vbase = c.v_pools[x.layer];
    const int32_t* bt = c.block_table + (size_t)x.req * c.max_blocks;
    const int nb = (N + kBlock - 1) / kBlock;
    for (int i = threadIdx.x; i < nb; i += kThreads) s_bt[i] = bt[i];
    __syncthreads();

    const int piece = (threadIdx.x % kChunksPerRow) * 16;
    const int rsub = threadIdx.x / kChunksPerRow;
    int32_t* pos = pos_ids ? pos_ids + (size_t)hc * pos_stride : nullptr;
    const bool pos_lane = pos && piece == 0;

    for (int base = i0; base < nk; base += kRowsPerIter) {
        u32x4 kr[kRounds], vr[kRounds];
        int pr[kRounds];
        // Branch-free load phase: rows past the end re-read the last survivor
        // (always in bounds) and are simply not stored.
        int src[kRounds];
#pragma unroll
        for (int u = 0; u < kRounds; ++u) src[u] = kp[min(base + rsub + u * kRowsPerRound, nk - 1)];
#pragma unroll
        for (int u = 0; u < kRounds; ++u) {
            const int s = src[u];
            const uint64_t off = row_offset(s_bt[s >> 4], c.H, x.head, s & 15) + piece;
            kr[u] = load16_nt(kbase + off);
            vr[u] = load16_nt(vbase + off);
        }
#pragma unroll
        for (int u = 0; u < kRounds; ++u) pr[u] = pos_lane ? pos[src[u]] : 0;
        __syncthreads();  // all reads of this chunk are done before any write
#pragma unroll
        for (int u = 0; u < kRounds; ++u) {
            const int i = base + rsub + u * kRowsPerRound;
            if (i < nk) {
                const uint64_t off = row_offset(s_bt[i >> 4], c.H, x.head, i & 15) + piece;
                store16_nt(kbase + off, kr[u]);
                store16_nt(vbase + off, vr[u]);
                if (pos_lane) pos[i] = pr[u];
            }
        }
    }
}

}  // namespace

hipError_t launch_kv_compact(const CacheView& c, const int32_t* keep, int budget,
                             int keep_shared, int32_t* pos_ids, int pos_stride, Check ck,
                             int32_t* status, hipStream_t s) {
    const int HC = c.L * c.R * c.H;
    if (HC == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_compact_kernel, dim3(HC), dim3(kThreads), 0, s, c, keep, budget,
                       keep_shared, pos_ids, pos_stride, ck, status);
    return hipGetLastError();
}

}  // namespace bkv
