// compact_util.h -- the order-preserving in-place row move shared by the
// compaction kernel and the fused kernels, and the fused kernels' common
// selection-and-move tail.  Called by all threads of the block; they
// synchronise.
#pragma once

#include "select_util.h"

namespace bkv {

// Moves survivor i of one head-cache from slot keep(i) >= i to slot i, for
// every i in [i0, nk), K and V rows together (and pos ids when `pos` is not
// null).  keep(i) = kp[i - kp_off] must be strictly ascending in i; s_bt is
// the request's block-table row, staged in LDS.
//
// Because the list is ascending, every source slot of a later chunk lies
// beyond every destination slot of the current one: the block walks the
// survivors in ascending chunks, reads a whole chunk (K, V, pos) into
// registers, waits at a barrier and only then writes it, so the move needs no
// second buffer.  16 lanes move one 256-byte row with 16-byte accesses (each
// wave instruction moves four whole rows, 1 KiB); rows are touched once, so
// the accesses are non-temporal.
template <int kThreads, int kRounds = 8>
__device__ void move_rows(uint64_t kbase, uint64_t vbase, const int* s_bt, int H, int head,
                          const int32_t* kp, int kp_off, int i0, int nk, int32_t* pos) {
    constexpr int kPieces = kRowBytes / 16;                 // 16-byte pieces per row
    constexpr int kRowsPerRound = kThreads / kPieces;       // rows per instruction round
    constexpr int kRowsPerIter = kRowsPerRound * kRounds;   // rows per barrier
    const int piece = (threadIdx.x % kPieces) * 16;
    const int rsub = threadIdx.x / kPieces;
    const bool pos_lane = pos && piece == 0;

    for (int base = i0; base < nk; base += kRowsPerIter) {
        u32x4 kr[kRounds], vr[kRounds];
        int pr[kRounds];
        // Branch-free load phase: rows past the end re-read the last survivor
        // (always in bounds) and are simply not stored.
        int src[kRounds];
#pragma unroll
        for (int u = 0; u < kRounds; ++u)
            src[u] = kp[min(base + rsub + u * kRowsPerRound, nk - 1) - kp_off];
#pragma unroll
        for (int u = 0; u < kRounds; ++u) {
            const int s = src[u];
            const uint64_t off = row_offset(s_bt[s >> 4], H, head, s & 15) + piece;
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
                const uint64_t off = row_offset(s_bt[i >> 4], H, head, i & 15) + piece;
                store16_nt(kbase + off, kr[u]);
                store16_nt(vbase + off, vr[u]);
                if (pos_lane) pos[i] = pr[u];
            }
        }
    }
}

// The tail of the fused kernels.  The m = N - P candidate keys of one
// selection are staged in s_key (the writes of every thread issued before the
// call: radix_select opens with a barrier), and the request has N > B and
// B > P.  Selects the top B - P keys (ties to the earlier slot), writes the
// kept candidates' slots in order to s_keep and to keep_row (nullable, after
// the prompt entries the caller has written), and moves the survivors of the
// n heads head0 .. head0 + n - 1 of `layer` in place (pos0: the first head's
// pos ids row, nullable).  Survivors before the first dropped candidate keep
// their slots.
template <int kThreads, int kRounds>
__device__ void select_and_move(const CacheView& c, int layer, int head0, int n, int P, int B,
                                int m, const uint32_t* s_key, int* s_keep, RadixScratch* rs,
                                int* s_wsum, int* s_drop, const int* s_bt, int32_t* keep_row,
                                int32_t* pos0, int pos_stride) {
    if (threadIdx.x == 0) *s_drop = m;
    int need;
    const uint32_t T = radix_select<kThreads>(s_key, m, B - P, rs, &need);
    emit_selected<kThreads>(
        s_key, m, T, need, s_wsum,
        [&](int r, int i) {
            s_keep[r] = P + i;
            if (keep_row) keep_row[P + r] = P + i;
        },
        [&](int i) { atomicMin(s_drop, i); });
    __syncthreads();
    const int i0 = P + *s_drop;
    for (int h = 0; h < n; ++h)
        move_rows<kThreads, kRounds>(c.k_pools[layer], c.v_pools[layer], s_bt, c.H, head0 + h,
                                     s_keep, P, i0, B,
                                     pos0 ? pos0 + (size_t)h * pos_stride : nullptr);
}

}  // namespace bkv
