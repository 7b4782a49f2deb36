// topk_select.hip -- per-head top-B selection with full prompt protection
// (Random Attention article, section "Random Attention: 不判断重要性, 只随机保留":
// prompt KV always kept, generated KV reduced to a per-head top-K; the budget
// includes the prompt).
//
// One workgroup per head-cache.  The N - P candidate scores are staged in LDS
// as unsigned 32-bit keys (non-negative fp32 scores order exactly like their
// bit patterns).  An MSB-first radix select (four 8-bit digits, LDS histogram)
// finds the (B-P)-th largest key T and how many keys equal to T must be kept;
// equal keys are taken in slot order (earlier slot first).  Two block-wide
// prefix scans (over "== T" and over "kept") then emit the kept slots in
// ascending order, prompt first.  The selection is exact integer work, so the
// result is bit-reproducible.
//
// Shared positions (same article, section "发现二": all heads on one common
// set of positions): one workgroup per (layer, request) selects once for all
// its KV heads.  A candidate's key is the largest of its `score_heads`
// per-head keys (score_heads = 1 for one shared random draw), and the keep
// list is written once per (layer, request).

#include "select_util.h"

namespace bkv {
namespace {

// kThreads: 256 for the serving shapes (about a thousand candidates; 64 and
// 128 threads were slower), 1024 from kWideFrom candidates on, where one
// workgroup per CU is typical (one-shot passes over long caches).
constexpr int kWideFrom = 8192;

template <int kThreads>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(CacheView c,
                                                               const uint32_t* __restrict__ scores,
                                                               int is_f32, int stride,
                                                               int score_heads, int shared, int B,
                                                               int32_t* __restrict__ keep, Check ck,
                                                               int32_t* status) {
    extern __shared__ uint32_t s_key[];  // [stride]
    __shared__ RadixScratch s_rs;
    __shared__ int s_wsum[kThreads / kWave];

    const int unit = blockIdx.x;  // head-cache, or (layer, request) when shared
    const HeadIdx x = shared ? HeadIdx{unit / c.R, unit % c.R, 0} : split_hc(c, unit);
    const int hc = shared ? -1 : unit;
    if (!request_ok(c, x.layer, x.req, hc, ck, status)) return;
    const int N = slot_count(c, hc, x.req);
    const int P = c.prompt_len[x.req];
    int32_t* out = keep + (size_t)unit * B;
    const int tid = threadIdx.x;

    if (N <= B) {  // nothing to evict: keep every slot
        for (int i = tid; i < B; i += kThreads) out[i] = (i < N) ? i : -1;
        return;
    }
    const int m = N - P;  // candidates
    const int k = B - P;  // candidates to keep, 0 <= k < m
    for (int i = tid; i < P; i += kThreads) out[i] = i;
    if (k == 0) return;

    const uint32_t* src = scores + (size_t)unit * score_heads * stride;
    for (int i = tid; i < m; i += kThreads) {
        uint32_t v = 0;
        for (int h = 0; h < score_heads; ++h) {
            uint32_t w = src[(size_t)h * stride + i];
            if (is_f32 && (w >> 31)) w = 0;  // negative fp32 scores rank as 0
            v = max(v, w);
        }
        s_key[i] = v;
    }

    // MSB-first radix select of the k-th largest key; `need` copies of it are kept.
    int need;
    const uint32_t T = radix_select<kThreads>(s_key, m, k, &s_rs, &need);

    // kept candidates in slot order after the prompt (r < k always holds; the
    // bound is defensive)
    emit_selected<kThreads>(
        s_key, m, T, need, s_wsum,
        [&](int r, int i) {
            if (r < k) out[P + r] = P + i;
        },
        [](int) {});
}

}  // namespace

hipError_t launch_topk_select(const CacheView& c, const void* scores, int kind, int stride,
                              int score_heads, int shared, int budget, int32_t* keep, Check ck,
                              int32_t* status, hipStream_t s) {
    const int units = c.L * c.R * (shared ? 1 : c.H);
    if (units == 0) return hipSuccess;
    const size_t lds = (size_t)stride * sizeof(uint32_t);
    const bool wide = stride >= kWideFrom;
    const void* fn = wide ? (const void*)topk_select_kernel<1024>
                          : (const void*)topk_select_kernel<256>;
    if (lds > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds);
        if (e != hipSuccess) return e;
    }
    const auto* sc = static_cast<const uint32_t*>(scores);
    const int is_f32 = kind == BKV_SCORE_F32 ? 1 : 0;
    const int heads = shared ? score_heads : 1;
    if (wide)
        hipLaunchKernelGGL(topk_select_kernel<1024>, dim3(units), dim3(1024), lds, s, c, sc,
                           is_f32, stride, heads, shared, budget, keep, ck, status);
    else
        hipLaunchKernelGGL(topk_select_kernel<256>, dim3(units), dim3(256), lds, s, c, sc, is_f32,
                           stride, heads, shared, budget, keep, ck, status);
    return hipGetLastError();
}

}  // namespace bkv
