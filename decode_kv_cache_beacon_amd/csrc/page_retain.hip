// page_retain.hip -- page retention: the cache shrinks by whole 16-slot pages,
// chosen once per request for every layer and head, so the compaction becomes
// a rewrite of the request's block table and no K/V row moves.
//
// Random Attention article, section "发现二": keeping contiguous blocks of 1 to
// 64 tokens instead of scattered tokens leaves accuracy almost unchanged, and
// so does forcing every head onto one common set of positions.  With the
// block equal to the cache page and one selection per request, both hold at
// once and the selection maps straight onto the paged layout.
//
// Per head-cache (the same section measures the block shapes with every head
// selecting on its own, and credits that independence with a second layer of
// redundancy across heads): every head-cache selects its own pages from its
// own score row and writes its own page-table row, still with no K/V row
// moves; the cache then reads each head-cache through its row.
//
// One workgroup of 1024 threads per request (256 per head-cache):
//   1. stage the request's block-table row in LDS (before anything is written,
//      so the output row may alias the input);
//   2. page key = the largest candidate-slot score of the page over all the
//      request's score rows (every layer and head of per-head beacon scores,
//      or one shared random row), folded into LDS with an integer max.  With
//      per-head rows and a key buffer, one workgroup per (layer, request)
//      forms these keys first (page_keys_kernel), so the rows are read by
//      the whole chip rather than by one workgroup per request;
//   3. prompt pages and a partial last page are kept; the budget / 16 - forced
//      best remaining pages are found with the shared radix select (ties to
//      the earlier page);
//   4. one block-wide scan places each kept page's block at the front of the
//      new row (page order) and each dropped page's block in the released list.

#include "select_util.h"

namespace bkv {
namespace {

// kPerHead: workgroup u serves head-cache u (its own score row, its own
// page-table row and slot count, outputs at row u); otherwise request u (its
// score rows across every layer and head, or one per-request row).
// pkeys (per request, nullable): the candidate pages' keys already formed
// by page_keys_kernel, [R][max_blocks], read instead of the score rows.
template <int kThreads, bool kPerHead>
__global__ __launch_bounds__(kThreads) void page_retain_kernel(
    CacheView c, const uint32_t* __restrict__ scores, int is_f32, int stride, int per_request_row,
    int B, int32_t* __restrict__ keep_pages, int32_t* table_out, int32_t* len_out,
    int32_t* __restrict__ freed, const uint32_t* __restrict__ pkeys, Check ck, int32_t* status) {
    constexpr int kWaves = kThreads / kWave;
    constexpr int kMaxPagesPerThread = (kMaxBlocksPerReq + kThreads - 1) / kThreads;
    __shared__ int s_bt[kMaxBlocksPerReq];
    __shared__ uint32_t s_pkey[kMaxBlocksPerReq];
    __shared__ RadixScratch s_rs;
    __shared__ int s_wsum[kWaves];

    const int u = blockIdx.x;
    const HeadIdx x = kPerHead ? split_hc(c, u) : HeadIdx{0, u, 0};
    const int r = x.req;
    const int hc = kPerHead ? u : -1;
    const int tid = threadIdx.x;
    if (!request_ok(c, x.layer, r, hc, ck, status)) return;
    const int N = slot_count(c, hc, r);
    const int P = c.prompt_len[r];
    const int npages = (N + kBlock - 1) / kBlock;
    const int Bp = B / kBlock;
    const int32_t* bt = table_row(c, hc, r);
    for (int j = tid; j < npages; j += kThreads) {
        s_bt[j] = bt[j];
        s_pkey[j] = 0;
    }
    __syncthreads();  // every read of the block-table row and of seq_len is done

    const int pf = (P + kBlock - 1) / kBlock;  // pages [0, pf) hold prompt slots
    const bool last_partial = (N % kBlock) != 0 && npages - 1 >= pf;
    const int pe = npages - (last_partial ? 1 : 0);  // candidate pages [pf, pe)
    const bool evict = npages > Bp;
    const int k = evict ? Bp - pf - (last_partial ? 1 : 0) : 0;  // >= 0 (budget check)

    uint32_t T = 0;
    int need = 0;
    if (k > 0 && pkeys) {
        for (int j = pf + tid; j < pe; j += kThreads) s_pkey[j] = pkeys[(size_t)r * c.max_blocks + j];
        __syncthreads();
        T = radix_select<kThreads>(s_pkey + pf, pe - pf, k, &s_rs, &need);
    } else if (k > 0) {
        // candidate slots n in [pf*16, pe*16), at score column n - P
        const int i0 = pf * kBlock - P, i1 = pe * kBlock - P;
        const bool one_row = kPerHead || per_request_row;
        const int layers = one_row ? 1 : c.L;
        const int heads = one_row ? 1 : c.H;
        const size_t layer_step = one_row ? 0 : (size_t)c.R * c.H * stride;
        const size_t row0 = kPerHead ? (size_t)u : per_request_row ? (size_t)r : (size_t)r * c.H;
        const uint32_t* first_row = scores + row0 * stride;
        for (int i = i0 + tid; i < i1; i += kThreads) {
            uint32_t v = 0;
            for (int l = 0; l < layers; ++l) {
                const uint32_t* src = first_row + l * layer_step + i;
                for (int h = 0; h < heads; ++h) {
                    uint32_t w = src[(size_t)h * stride];
                    if (is_f32 && (w >> 31)) w = 0;  // negative fp32 scores rank as 0
                    v = max(v, w);
                }
            }
            atomicMax(&s_pkey[(P + i) / kBlock], v);
        }
        __syncthreads();
        T = radix_select<kThreads>(s_pkey + pf, pe - pf, k, &s_rs, &need);
    }

    // Each thread owns a contiguous run of pages (page order).
    const int seg = (npages + kThreads - 1) / kThreads;
    const int lo = min(tid * seg, npages), hi = min(lo + seg, npages);
    int eq = 0;
    if (k > 0)
        for (int j = max(lo, pf); j < min(hi, pe); ++j) eq += (s_pkey[j] == T);
    const int eq_before = block_exclusive_scan<kThreads>(eq, s_wsum);
    bool take[kMaxPagesPerThread];
    int kept = 0, e = eq_before;
#pragma unroll
    for (int u = 0; u < kMaxPagesPerThread; ++u) {
        const int j = lo + u;
        bool t = false;
        if (j < hi) {
            if (!evict || j < pf || j >= pe) {
                t = true;  // nothing to evict, a prompt page or the partial last page
            } else if (k > 0) {
                const uint32_t v = s_pkey[j];
                t = v > T || (v == T && e < need);
                e += (v == T);
            }
        }
        take[u] = t;
        kept += t;
    }
    const int kept_before = block_exclusive_scan<kThreads>(kept, s_wsum);
    const int n_kept = evict ? Bp : npages;

    int32_t* kp = keep_pages + (size_t)u * Bp;
    int32_t* row_out = table_out + (size_t)u * c.max_blocks;
    int32_t* fr = freed + (size_t)u * c.max_blocks;
    int kb = kept_before;
#pragma unroll
    for (int u = 0; u < kMaxPagesPerThread; ++u) {
        const int j = lo + u;
        if (j >= hi) break;
        if (take[u]) {
            if (kb < Bp) kp[kb] = j;  // kb < Bp whenever j is kept under eviction
            row_out[kb] = s_bt[j];
            ++kb;
        } else {
            fr[j - kb] = s_bt[j];
        }
    }
    for (int i = n_kept + tid; i < Bp; i += kThreads) kp[i] = -1;
    for (int i = n_kept + tid; i < npages; i += kThreads) row_out[i] = -1;
    for (int i = npages - n_kept + tid; i < c.max_blocks; i += kThreads) fr[i] = -1;
    if (tid == 0) {
        // every kept page is full except a partial last page, which is always kept
        const int tail = N % kBlock;
        len_out[u] = evict ? n_kept * kBlock - (tail ? kBlock - tail : 0) : N;
    }
}

constexpr int kKeyThreads = 256;

// The page keys of one request's score rows of one layer (workgroup (layer,
// request)): the largest score of each candidate page over the layer's H
// rows, folded into LDS and then into keys[r][page] with an integer max, so
// every CU reads a share of the rows instead of one workgroup per request.
__global__ __launch_bounds__(kKeyThreads) void page_keys_kernel(
    CacheView c, const uint32_t* __restrict__ scores, int is_f32, int stride, int B,
    uint32_t* __restrict__ keys, Check ck, int32_t* status) {
    __shared__ uint32_t s_k[kMaxBlocksPerReq];
    const int layer = blockIdx.x / c.R, r = blockIdx.x % c.R;
    const int tid = threadIdx.x;
    if (!request_ok(c, layer, r, -1, ck, status)) return;
    const int N = c.seq_len[r];
    const int P = c.prompt_len[r];
    const int npages = (N + kBlock - 1) / kBlock;
    const int pf = (P + kBlock - 1) / kBlock;
    const bool last_partial = (N % kBlock) != 0 && npages - 1 >= pf;
    const int pe = npages - (last_partial ? 1 : 0);
    if (npages <= B / kBlock || pe <= pf) return;  // nothing the selection reads
    for (int j = pf + tid; j < pe; j += kKeyThreads) s_k[j] = 0;
    __syncthreads();
    const int i0 = pf * kBlock - P, i1 = pe * kBlock - P;
    const uint32_t* rows = scores + ((size_t)layer * c.R + r) * c.H * stride;
    for (int i = i0 + tid; i < i1; i += kKeyThreads) {
        uint32_t v = 0;
        for (int h = 0; h < c.H; ++h) {
            uint32_t w = rows[(size_t)h * stride + i];
            if (is_f32 && (w >> 31)) w = 0;  // negative fp32 scores rank as 0
            v = max(v, w);
        }
        atomicMax(&s_k[(P + i) / kBlock], v);
    }
    __syncthreads();
    for (int j = pf + tid; j < pe; j += kKeyThreads)
        if (s_k[j]) atomicMax(&keys[(size_t)r * c.max_blocks + j], s_k[j]);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_page_retain(const CacheView& c, const void* scores, int kind, int stride,
                              int rows, int budget, int32_t* keep_pages, int32_t* block_table_out,
                              int32_t* seq_len_out, int32_t* freed, uint32_t* key_ws, Check ck,
                              int32_t* status, hipStream_t s) {
    if (c.R == 0) return hipSuccess;
    const uint32_t* sc = static_cast<const uint32_t*>(scores);
    const int is_f32 = kind == BKV_SCORE_F32 ? 1 : 0;
    // per-head rows and a key buffer: the keys by (layer, request) workgroups first
    const bool split = key_ws && rows == BKV_ROWS_PER_HEAD;
    if (split) {
        const size_t n = (size_t)c.R * c.max_blocks;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 1024)),
                           dim3(256), 0, s, key_ws, n);
        hipLaunchKernelGGL(page_keys_kernel, dim3((unsigned)(c.L * c.R)), dim3(kKeyThreads), 0, s,
                           c, sc, is_f32, stride, budget, key_ws, ck, status);
    }
    hipLaunchKernelGGL((page_retain_kernel<1024, false>), dim3(c.R), dim3(1024), 0, s, c, sc,
                       is_f32, stride, rows == BKV_ROWS_PER_REQUEST ? 1 : 0, budget, keep_pages,
                       block_table_out, seq_len_out, freed, split ? key_ws : nullptr, ck, status);
    return hipGetLastError();
}

hipError_t launch_page_retain_heads(const CacheView& c, const void* scores, int kind, int stride,
                                    int budget, int32_t* keep_pages, int32_t* head_table_out,
                                    int32_t* head_len_out, int32_t* dropped, Check ck,
                                    int32_t* status, hipStream_t s) {
    const unsigned HC = (unsigned)(c.L * c.R * c.H);
    if (HC == 0) return hipSuccess;
    hipLaunchKernelGGL((page_retain_kernel<256, true>), dim3(HC), dim3(256), 0, s, c,
                       static_cast<const uint32_t*>(scores), kind == BKV_SCORE_F32 ? 1 : 0,
                       stride, 0, budget, keep_pages, head_table_out, head_len_out, dropped,
                       nullptr, ck, status);
    return hipGetLastError();
}

}  // namespace bkv
