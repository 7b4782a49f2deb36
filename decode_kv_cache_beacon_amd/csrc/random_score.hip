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

#include "bkv_internal.h"

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
    if (!request_ok(c, x.layer, x.req, ck, status)) return;
    const int N = c.seq_len[x.req];
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

}  // namespace

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
