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
// How (one 8-wave workgroup per head-cache, gfx950):
//   - The beacon.key logits are a [K x 128] x [128 x N] contraction: bf16 MFMA
//     v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Beacons are the A
//     operand (rows, kept in registers for the whole head), 32 keys form the B
//     operand (columns), so each lane owns one key column and 16 beacon rows of
//     a 32x32 result.  Rows are split between two groups of four waves; wave
//     (group g, phase q) consumes key tiles q, q+4, q+8, ...
//   - Key tiles (32 keys = 8 KiB) stream through a 16-tile LDS ring filled by
//     direct-to-LDS DMA (global_load_lds_dwordx4): each load instruction moves
//     1 KiB of whole key rows, the ring is refilled three iterations ahead, and
//     each tile serves both row groups.  A row's 16-byte chunks are
//     XOR-swizzled by the row index so that the fragment reads are free of
//     bank conflicts.  The four waves of group 1 issue all the DMA, so their
//     vmcnt counts ring loads only; one barrier per iteration hands the tiles
//     over.
//   - Phase 1 (log-sum-exp per beacon): per lane and row a running sum of
//     exp2(acc * log2(e)/sqrt(d) - M) with one reference M per wave taken from
//     the wave's first tile; lanes, then waves, are merged in LDS.  If any live
//     row's sum overflows or underflows (logit spread beyond the fp32 exponent
//     range) the head is redone exactly with direct loads: an all-key maximum
//     per row first, then the sums against that maximum.
//   - Phase 2 (score): the keys stream through the ring again (the re-read is
//     served by L2/MALL) and the MFMA accumulator starts from C = -lse_j (in
//     accumulator units), so the subtraction is free; each lane takes the max
//     over its rows, the two row groups are merged through LDS one iteration
//     later, and one exp2 per key gives sigma(n).
// Scaling by 1/sqrt(d) happens in fp32 after accumulation; the bf16 beacons
// are never pre-scaled.

#include "bkv_internal.h"

namespace bkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kCs = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
constexpr int kWaves = 8;
constexpr int kQ = 4;                              // tile phases = waves per row group
constexpr int kTileKeys = 32;
constexpr int kTileBytes = kTileKeys * kRowBytes;  // 8 KiB
constexpr int kDepth = 3;                          // ring refilled this many iterations ahead
constexpr int kRingIters = kDepth + 1;
constexpr int kRingTiles = kQ * kRingIters;        // 16 tiles = 128 KiB
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
// s_nop covers the wait state the hardware needs between writing M0 and an
// LDS DMA that reads it.  M0 is reserved by the compiler, which sets it right
// before each of its own uses; nothing else in this kernel reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint64_t g, uint32_t m0) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
}
#pragma clang diagnostic pop

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Sum (or max) over the 32 lanes of one lane half.
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

template <int MBW>
__global__ __launch_bounds__(kWaves * kWave) void beacon_score_kernel(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    int window, float bonus, float* __restrict__ scores, int stride, float* __restrict__ lse_out,
    Check ck, int32_t* status) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kRingTiles * kTileBytes];
    __shared__ int s_bt[kMaxBlocksPerReq];
    __shared__ float s_part[kWaves][BKV_MAX_BEACONS];
    __shared__ float s_M[kWaves];
    __shared__ float s_lse2[BKV_MAX_BEACONS];
    __shared__ float s_ref[BKV_MAX_BEACONS];
    __shared__ int s_live[BKV_MAX_BEACONS];
    __shared__ float s_pmax[2][kQ][32];
    __shared__ int s_rescue;

    const int hc = blockIdx.x;
    const HeadIdx x = split_hc(c, hc);
    if (!request_ok(c, x.layer, x.req, ck, status)) return;
    const int N = c.seq_len[x.req];
    const int P = c.prompt_len[x.req];

    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int hh = lane >> 5;
    const int col = lane & 31;
    const int group = w / kQ;
    const int q = w % kQ;
    const bool loader = group == 1;
    const int Kp = (K + 31) & ~31;
    const int MB = Kp / 32;
    const int mb0 = group * MBW;
    const bool computes = mb0 < MB;

    const int nb = (N + kBlock - 1) / kBlock;
    const int32_t* bt = c.block_table + (size_t)x.req * c.max_blocks;
    for (int i = tid; i < nb; i += blockDim.x) s_bt[i] = bt[i];
    for (int j = tid; j < Kp; j += blockDim.x)
        s_live[j] = (j < K) && counts[(size_t)hc * K + j] > 0;
    if (tid == 0) s_rescue = 0;
    __syncthreads();

    if (N == 0) {  // empty cache: nothing to score, every live lse is log(0)
        for (int j = tid; j < K; j += blockDim.x)
            if (lse_out)
                lse_out[(size_t)hc * K + j] = s_live[j] ? -INFINITY : __int_as_float(0x7fc00000);
        return;
    }

    const uint64_t kpool = c.k_pools[x.layer];
    const int ntiles = (N + kTileKeys - 1) / kTileKeys;
    const int iters = (ntiles + kQ - 1) / kQ;
    // last iteration in which this wave's phase has a tile (-1 if none)
    const int jlast = (q < ntiles) ? (ntiles - 1 - q) / kQ : -1;

    // DMA of key tile t into ring slot `slot` (issued by a group-1 wave).  Lane
    // l of instruction i fills LDS bytes [1024 i + 16 l, +16) of the slot: row
    // r = 4i + l/16, chunk position p = l%16, which holds global chunk
    // p ^ (r & 15) of key 32t + r (key N-1 past the end).
    const uint32_t ring0 = lds_addr(s_ring);
    auto issue_tile = [&](int t, int slot) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(ring0 + slot * kTileBytes);
#pragma unroll
        for (int i = 0; i < kDmaPerTile; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int ch = (lane & 15) ^ (r & 15);
            const int n = min(kTileKeys * t + r, N - 1);
            const uint64_t g = kpool + row_offset(s_bt[n >> 4], c.H, x.head, n & 15) + 16 * ch;
            dma16(g, dst + 1024 * i);
        }
    };
    auto slot_of = [&](int it) { return (it % kRingIters) * kQ + q; };
    auto prologue = [&]() {
        if (loader)
            for (int j = 0; j < kDepth && j <= jlast; ++j) issue_tile(kQ * j + q, slot_of(j));
    };
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
    // hand-over of iteration `it`: the loaders wait for their DMA of it, all
    // waves pass the barrier (iteration it-1's reads are then done), and the
    // slot read in it-1 is refilled with iteration it + kDepth
    auto begin_iter = [&](int it) {
        if (loader) wait_ring(min(kDepth - 1, jlast - it));
        ring_barrier();
        if (loader && it + kDepth <= jlast) issue_tile(kQ * (it + kDepth) + q, slot_of(it + kDepth));
    };

    prologue();  // the first tiles are in flight while the beacons are prepared

    // A fragments: beacon row 32*(mb0+m) + col, bf16 (RNE) of the fp32 state.
    bf16x8_t A[MBW][8];
    uint32_t live_bits[MBW];
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
        const int j = 32 * (mb0 + m) + col;
        const bool lv = (mb0 + m < MB) && s_live[j];
        const float* br = beacons + ((size_t)hc * K + (lv ? j : 0)) * kHeadDim + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            u32x4 pk = {0u, 0u, 0u, 0u};
            if (lv) {
                const float4 lo = *reinterpret_cast<const float4*>(br + 16 * s);
                const float4 hi = *reinterpret_cast<const float4*>(br + 16 * s + 4);
                pk.x = (uint32_t)to_bf16_rne(lo.x) | ((uint32_t)to_bf16_rne(lo.y) << 16);
                pk.y = (uint32_t)to_bf16_rne(lo.z) | ((uint32_t)to_bf16_rne(lo.w) << 16);
                pk.z = (uint32_t)to_bf16_rne(hi.x) | ((uint32_t)to_bf16_rne(hi.y) << 16);
                pk.w = (uint32_t)to_bf16_rne(hi.z) | ((uint32_t)to_bf16_rne(hi.w) << 16);
            }
            A[m][s] = as_bf16x8(pk);
        }
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
        begin_iter(it);
        if (!computes || it > jlast) continue;
        const int tt = kQ * it + q;
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
    // lanes -> waves -> rows (no ring load is in flight from here on)
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
        if (mb0 + m >= MB) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float v = half_sum(sum[m][i]);
            if (col == 0) s_part[w][32 * (mb0 + m) + acc_row(i, hh)] = v;
        }
    }
    if (lane == 0) s_M[w] = (jlast >= 0 && computes) ? Mw : -INFINITY;
    __syncthreads();
    for (int j = tid; j < Kp; j += blockDim.x) {
        const int g = (j / 32) / MBW;
        float Mg = -INFINITY;
        for (int k2 = 0; k2 < kQ; ++k2) Mg = fmaxf(Mg, s_M[g * kQ + k2]);
        float total = 0.f;
        for (int k2 = 0; k2 < kQ; ++k2) {
            const float Mk = s_M[g * kQ + k2];
            if (Mk != -INFINITY) total += s_part[g * kQ + k2][j] * exp2f(Mk - Mg);
        }
        const bool lv = s_live[j];
        const bool ok = total >= 0x1p-100f && total < INFINITY;
        if (lv && !ok) s_rescue = 1;
        s_lse2[j] = lv ? Mg + log2f(total) : INFINITY;
    }
    __syncthreads();

    if (s_rescue) {
        // Exact fallback with direct loads: per-row maximum over all keys
        // first, then the sums against it (every term <= 1, the maximum == 1).
#pragma unroll
        for (int m = 0; m < MBW; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) sum[m][i] = -INFINITY;
        if (computes) {
            for (int tt = q; tt < ntiles; tt += kQ) {
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
                if (col == 0) s_part[w][32 * (mb0 + m) + acc_row(i, hh)] = v;
            }
        }
        __syncthreads();
        for (int j = tid; j < Kp; j += blockDim.x) {
            const int g = (j / 32) / MBW;
            float R = -INFINITY;
            for (int k2 = 0; k2 < kQ; ++k2) R = fmaxf(R, s_part[g * kQ + k2][j]);
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
            for (int tt = q; tt < ntiles; tt += kQ) {
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
                if (col == 0) s_part[w][32 * (mb0 + m) + acc_row(i, hh)] = v;
            }
        }
        __syncthreads();
        for (int j = tid; j < Kp; j += blockDim.x) {
            const int g = (j / 32) / MBW;
            float total = 0.f;
            for (int k2 = 0; k2 < kQ; ++k2) total += s_part[g * kQ + k2][j];
            s_lse2[j] = s_live[j] ? s_ref[j] + log2f(total) : INFINITY;
        }
        __syncthreads();
    }

    // written by group 0, which issues no ring loads
    if (lse_out && group == 0) {
        for (int j = tid; j < K; j += kQ * kWave)
            lse_out[(size_t)hc * K + j] = s_live[j] ? s_lse2[j] * kLn2 : __int_as_float(0x7fc00000);
    }
    prologue();  // phase 2 streams the keys again

    // ---------------- phase 2: sigma(n) = exp(max_j s_jn - lse_j) ----------------
    f32x16_t Cf[MBW];
#pragma unroll
    for (int m = 0; m < MBW; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float l2 = (mb0 + m < MB) ? s_lse2[32 * (mb0 + m) + acc_row(i, hh)] : INFINITY;
            Cf[m][i] = -l2 / kCs;
        }
    float* out = scores + (size_t)hc * stride;
    // Group 0 finishes a tile one iteration late, once group 1's partial
    // maximum for it has passed the next barrier.
    auto finalize = [&](int it, float mx) {
        const int tt = kQ * it + q;
        const int n = kTileKeys * tt + col;
        if (it <= jlast && hh == 0 && n >= P && n < N) {
            mx = fmaxf(mx, s_pmax[it & 1][q][col]);
            const float sigma = __builtin_amdgcn_exp2f(mx * kCs);
            out[n - P] = sigma + ((n >= N - window) ? bonus : 0.f);
        }
    };
    float mx_prev = -INFINITY;
    for (int it = 0; it < iters; ++it) {
        begin_iter(it);
        if (group == 0 && it > 0) finalize(it - 1, mx_prev);
        float mx = -INFINITY;
        if (it <= jlast && computes) {
            Tile t;
            read_tile(t, slot_of(it));
#pragma unroll
            for (int m = 0; m < MBW; ++m) {
                if (mb0 + m >= MB) continue;
                const f32x16_t acc = logits(A[m], t, Cf[m]);
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
        }
        if (group == 1 && hh == 0) s_pmax[it & 1][q][col] = mx;
        mx_prev = mx;
    }
    ring_barrier();
    if (group == 0) finalize(iters - 1, mx_prev);
}

}  // namespace

hipError_t launch_beacon_score(const CacheView& c, const float* beacons, const int32_t* counts,
                               int K, int window, float bonus, float* scores, int stride,
                               float* lse, Check ck, int32_t* status, hipStream_t s) {
    const int HC = c.L * c.R * c.H;
    if (HC == 0) return hipSuccess;
    // row blocks per wave: 1 for K <= 64, 2 for K <= 128, 4 for K <= 256
    if (K <= 64) {
        hipLaunchKernelGGL(beacon_score_kernel<1>, dim3(HC), dim3(kWaves * kWave), 0, s, c,
                           beacons, counts, K, window, bonus, scores, stride, lse, ck, status);
    } else if (K <= 128) {
        hipLaunchKernelGGL(beacon_score_kernel<2>, dim3(HC), dim3(kWaves * kWave), 0, s, c,
                           beacons, counts, K, window, bonus, scores, stride, lse, ck, status);
    } else {
        hipLaunchKernelGGL(beacon_score_kernel<4>, dim3(HC), dim3(kWaves * kWave), 0, s, c,
                           beacons, counts, K, window, bonus, scores, stride, lse, ck, status);
    }
    return hipGetLastError();
}

}  // namespace bkv
