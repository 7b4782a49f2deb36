// select_util.h -- block-level scans and the MSB-first radix select shared by
// the selection kernels (per-slot top-B and per-page retention).  Every
// function here is called by all threads of the block and synchronises.
#pragma once

#include "bkv_internal.h"

namespace bkv {

__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum of one int per thread over the whole block, in thread
// order.  s_wsum needs one entry per wave.
template <int kThreads>
__device__ int block_exclusive_scan(int v, int* s_wsum) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int incl = wave_inclusive_scan(v);
    if (lane == kWave - 1) s_wsum[w] = incl;
    __syncthreads();
    int off = 0;
    for (int j = 0; j < w; ++j) off += s_wsum[j];
    __syncthreads();  // s_wsum may be reused by the next scan
    return off + incl - v;
}

// Shared-memory scratch of radix_select.
struct RadixScratch {
    int hist[256];
    uint32_t prefix;
    int need;
};

// The k-th largest (1 <= k <= m) of the m unsigned keys key[0..m): four 8-bit
// digits, most significant first, each counted in an LDS histogram and located
// by a wave scan over the digits in descending order.  Returns the key T and
// sets *need_out to how many keys equal to T rank inside the top k.
template <int kThreads>
__device__ uint32_t radix_select(const uint32_t* key, int m, int k, RadixScratch* rs,
                                 int* need_out) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    int need = k;  // rank still to locate inside the keys matching `prefix`
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kThreads) rs->hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < m; i += kThreads) {
            const uint32_t v = key[i];
            if ((v & mask) == prefix) atomicAdd(&rs->hist[(v >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns digits 255-4l .. 252-4l (descending)
            int cnt[4], local = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                cnt[j] = rs->hist[255 - 4 * tid - j];
                local += cnt[j];
            }
            const int incl = wave_inclusive_scan(local);
            const int excl = incl - local;  // keys with a larger digit
            if (excl < need && need <= incl) {
                int rem = need - excl, above = excl, digit = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (rem <= cnt[j]) {
                        digit = 255 - 4 * tid - j;
                        break;
                    }
                    rem -= cnt[j];
                    above += cnt[j];
                }
                rs->prefix = prefix | ((uint32_t)digit << shift);
                rs->need = need - above;
            }
        }
        __syncthreads();
        prefix = rs->prefix;
        need = rs->need;
        mask |= 0xFFu << shift;
    }
    *need_out = need;
    return prefix;
}

// After radix_select: walks the m candidates in slot order and calls
// take(r, i) for the r-th kept candidate i (keys above T, and the first
// `need` keys equal to T) and drop(i) for every other one.  Each thread owns
// one contiguous run of candidates; two block-wide scans give each run its
// number of earlier keys equal to T and of earlier kept keys.
template <int kThreads, typename Take, typename Drop>
__device__ void emit_selected(const uint32_t* key, int m, uint32_t T, int need, int* s_wsum,
                              Take take, Drop drop) {
    const int seg = (m + kThreads - 1) / kThreads;
    const int lo = min((int)threadIdx.x * seg, m), hi = min(lo + seg, m);
    int eq = 0;
    for (int i = lo; i < hi; ++i) eq += (key[i] == T);
    const int eq_before = block_exclusive_scan<kThreads>(eq, s_wsum);
    int kept = 0, e = eq_before;
    for (int i = lo; i < hi; ++i) {
        const uint32_t v = key[i];
        kept += v > T || (v == T && e < need);
        e += (v == T);
    }
    int r = block_exclusive_scan<kThreads>(kept, s_wsum);
    e = eq_before;
    for (int i = lo; i < hi; ++i) {
        const uint32_t v = key[i];
        const bool t = v > T || (v == T && e < need);
        e += (v == T);
        if (t)
            take(r++, i);
        else
            drop(i);
    }
}

}  // namespace bkv
