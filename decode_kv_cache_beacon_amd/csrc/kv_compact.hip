// kv_compact.hip -- in-place, order-preserving compaction of a paged bf16 KV
// cache (the cache-compaction step every selector shares; Random Attention
// article, section "发现四").
//
// One workgroup per head-cache.  Survivor i moves from slot keep[i] >= i to
// slot i (move_rows: ascending chunks read into registers, a barrier, then
// written, so the in-place move is race-free without a second buffer).  The
// kernel first checks that the keep list is strictly ascending inside [0, N)
// and finds the first moved survivor; rows before it (the prompt at least)
// are never touched.
//
// With shared positions every head of a (layer, request) applies the one keep
// list of that (layer, request).

#include "compact_util.h"

namespace bkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_compact_kernel(CacheView c,
                                                              const int32_t* __restrict__ keep,
                                                              int B, int keep_shared,
                                                              int32_t* __restrict__ pos_ids,
                                                              int pos_stride, Check ck,
                                                              int32_t* status) {
    const int hc = blockIdx.x;
    const HeadIdx x = split_hc(c, hc);
    if (!request_ok(c, x.layer, x.req, hc, ck, status)) return;

    const int N = slot_count(c, hc, x.req);
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
    const int32_t* bt = table_row(c, hc, x.req);
    const int nb = (N + kBlock - 1) / kBlock;
    for (int i = threadIdx.x; i < nb; i += kThreads) s_bt[i] = bt[i];
    __syncthreads();

    int32_t* pos = pos_ids ? pos_ids + (size_t)hc * pos_stride : nullptr;
    move_rows<kThreads>(kbase, vbase, s_bt, c.H, x.head, kp, 0, i0, nk, pos);
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
