// random_score.hip -- the random selector's scores (Random Attention article,
// section "Random Attention: 不判断重要性, 只随机保留": per-head independent
// random retention; no cache content is read).
//
// Counter-based: the draw of slot n depends only on (seed, request id, pass
// index, layer, head, n), so the scorer needs no RNG state and a new pass
// index draws afresh.  With shared positions (same article, section "发现二":
// every head on one common set of positions) one row per (layer, request) is
// drawn, with the head field of the counter set to 0; for page retention one
// row per request, with the layer and head fields set to 0.  Philox4x64-10 as published by Salmon, Moraes, Dror and
// Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds of
// two 64x64->128-bit multiplies with a Weyl-sequence key schedule.  One thread
// evaluates one counter and scores the four slots 4g .. 4g+3.

#include "compact_util.h"

namespace bkv {
namespace {

constexpr int kThreads = 256;

struct U64x4 {
    uint64_t v[4];
};

__device__ __forceinline__ U64x4 philox4x64_10(U64x4 x, uint64_t k0, uint64_t k1) {
    constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull;
    constexpr uint64_t kMul1 = 0xCA5A826395121157ull;
    constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull;
    constexpr uint64_t kWeyl1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t lo0 = kMul0 * x.v[0], hi0 = __umul64hi(kMul0, x.v[0]);
        const uint64_t lo1 = kMul1 * x.v[2], hi1 = __umul64hi(kMul1, x.v[2]);
        U64x4 y;
        y.v[0] = hi1 ^ x.v[1] ^ k0;
        y.v[1] = lo1;
        y.v[2] = hi0 ^ x.v[3] ^ k1;
        y.v[3] = lo0;
        x = y;
        k0 += kWeyl0;
        k1 += kWeyl1;
    }
    return x;
}

__global__ __launch_bounds__(kThreads) void random_score_kernel(
    CacheView c, uint64_t seed, const uint64_t* __restrict__ req_ids,
    const int32_t* __restrict__ pass_idx, int rows, uint32_t* __restrict__ scores, int stride,
    Check ck, int32_t* status) {
    const int row = blockIdx.x;  // head-cache, (layer, request) or request
    const HeadIdx x = rows == BKV_ROWS_PER_REQUEST        ? HeadIdx{0, row, 0}
                      : rows == BKV_ROWS_PER_LAYER_REQUEST ? HeadIdx{row / c.R, row % c.R, 0}
                                                           : split_hc(c, row);
    const int hc = rows == BKV_ROWS_PER_HEAD ? row : -1;
    if (!request_ok(c, x.layer, x.req, hc, ck, status)) return;
    const int N = slot_count(c, hc, x.req);
    const int P = c.prompt_len[x.req];
    const int g = blockIdx.y * kThreads + threadIdx.x;  // counter word 0: slot group
    const int n0 = g * 4;
    if (n0 >= N || n0 + 4 <= P) return;

    U64x4 ctr;
    ctr.v[0] = (uint64_t)g;
    ctr.v[1] = (uint64_t)(uint32_t)pass_idx[x.req];
    ctr.v[2] = ((uint64_t)(uint32_t)x.layer << 32) | (uint64_t)(uint32_t)x.head;
    ctr.v[3] = req_ids[x.req];
    const U64x4 w = philox4x64_10(ctr, seed, 0);
    uint32_t* out = scores + (size_t)row * stride;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int n = n0 + k;
        if (n >= P && n < N) out[n - P] = (uint32_t)(w.v[k] >> 32);
    }
}

// Fused per-head pass: each workgroup draws its head-cache's candidate
// scores (written to the score buffer and kept in LDS as keys), selects the
// top B - P with the radix select, and compacts the head-cache in place --
// the same results as random_score_kernel, topk_select_kernel and
// kv_compact_kernel in turn, in one launch and without the keys or the keep
// list leaving the workgroup.  Dynamic LDS holds the stride candidate keys
// followed by the keep list.
__global__ __launch_bounds__(kThreads) void random_evict_kernel(
    CacheView c, uint64_t seed, const uint64_t* __restrict__ req_ids,
    const int32_t* __restrict__ pass_idx, uint32_t* __restrict__ scores, int stride, int B,
    int32_t* __restrict__ keep_out, int32_t* __restrict__ pos_ids, int pos_stride, Check ck,
    int32_t* status) {
    extern __shared__ uint32_t s_key[];  // [stride] keys, then the keep list
    __shared__ int s_bt[kMaxBlocksPerReq];
    __shared__ RadixScratch s_rs;
    __shared__ int s_wsum[kThreads / kWave];
    __shared__ int s_drop;

    const int hc = blockIdx.x;
    const HeadIdx x = split_hc(c, hc);
    if (!request_ok(c, x.layer, x.req, hc, ck, status)) return;
    const int N = slot_count(c, hc, x.req);
    const int P = c.prompt_len[x.req];
    const int tid = threadIdx.x;
    int32_t* keep_row = keep_out ? keep_out + (size_t)hc * B : nullptr;
    uint32_t* out = scores + (size_t)hc * stride;

    // draws of the candidates [P, N), one counter per four slots
    U64x4 ctr;
    ctr.v[1] = (uint64_t)(uint32_t)pass_idx[x.req];
    ctr.v[2] = ((uint64_t)(uint32_t)x.layer << 32) | (uint64_t)(uint32_t)x.head;
    ctr.v[3] = req_ids[x.req];
    for (int g = P / 4 + tid; 4 * g < N; g += kThreads) {
        ctr.v[0] = (uint64_t)g;
        const U64x4 w = philox4x64_10(ctr, seed, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int n = 4 * g + k;
            if (n >= P && n < N) {
                const uint32_t v = (uint32_t)(w.v[k] >> 32);
                out[n - P] = v;
                s_key[n - P] = v;
            }
        }
    }
    if (N <= B) {  // nothing to evict: every slot stays where it is
        if (keep_row)
            for (int i = tid; i < B; i += kThreads) keep_row[i] = (i < N) ? i : -1;
        return;
    }
    if (keep_row)
        for (int i = tid; i < P; i += kThreads) keep_row[i] = i;
    const int m = N - P, k = B - P;
    if (k == 0) return;  // only the prompt survives, and it does not move
    const int nb = (N + kBlock - 1) / kBlock;
    const int32_t* bt = table_row(c, hc, x.req);
    for (int i = tid; i < nb; i += kThreads) s_bt[i] = bt[i];
    // kept candidate r -> its slot, after the stride keys
    select_and_move<kThreads, 8>(c, x.layer, x.head, 1, P, B, m, s_key,
                                 reinterpret_cast<int*>(s_key + stride), &s_rs, s_wsum, &s_drop,
                                 s_bt, keep_row,
                                 pos_ids ? pos_ids + (size_t)hc * pos_stride : nullptr,
                                 pos_stride);
}

}  // namespace

hipError_t launch_random_evict(const CacheView& c, uint64_t seed, const uint64_t* req_ids,
                               const int32_t* pass_idx, uint32_t* scores, int stride, int budget,
                               int32_t* keep_out, int32_t* pos_ids, int pos_stride, Check ck,
                               int32_t* status, hipStream_t s) {
    const int HC = c.L * c.R * c.H;
    if (HC == 0) return hipSuccess;
    const size_t lds = (size_t)(stride + budget) * sizeof(uint32_t);
    if (lds > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)random_evict_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(random_evict_kernel, dim3(HC), dim3(kThreads), lds, s, c, seed, req_ids,
                       pass_idx, scores, stride, budget, keep_out, pos_ids, pos_stride, ck,
                       status);
    return hipGetLastError();
}

hipError_t launch_random_score(const CacheView& c, uint64_t seed, const uint64_t* req_ids,
                               const int32_t* pass_idx, int rows, uint32_t* scores, int stride,
                               Check ck, int32_t* status, hipStream_t s) {
    const int n_rows = rows == BKV_ROWS_PER_REQUEST        ? c.R
                       : rows == BKV_ROWS_PER_LAYER_REQUEST ? c.L * c.R
                                                            : c.L * c.R * c.H;
    if (n_rows == 0) return hipSuccess;
    const int max_slots = c.max_blocks * kBlock;
    const int groups = (max_slots + 3) / 4;
    const int gx = (groups + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(random_score_kernel, dim3(n_rows, gx), dim3(kThreads), 0, s, c, seed,
                       req_ids, pass_idx, rows, scores, stride, ck, status);
    return hipGetLastError();
}

}  // namespace bkv
