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
// How (one workgroup per head-cache, gfx950):
//   - The beacon.key logits are a [K x 128] x [128 x N] contraction: bf16 MFMA
//     v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Beacons are the A
//     operand (rows), 32 keys form the B operand (columns), so each lane owns
//     one key column and 16 beacon rows of the 32x32 result.
//   - A wave keeps the bf16 A fragments of its row blocks in registers for the
//     whole head.  Beyond 32 beacons the rows are split between two groups of
//     four waves (8 waves, two per SIMD, so one wave's MFMA work overlaps
//     another's exp/VALU work); within a group the 4 waves take every 4th key
//     tile.  Each lane loads its B fragment straight from the paged pool:
//     8 x 16 bytes of one 256-byte key row (rows are found through the block
//     table, staged in LDS), and the next tile is in flight while the current
//     one is consumed.
//   - Phase 1 (log-sum-exp per beacon): per lane and row a running sum of
//     exp2(acc * log2(e)/sqrt(d) - M) with one reference M per wave taken from
//     the wave's first tile; lanes, then waves, are merged in LDS.  If any live
//     row's sum overflows or underflows (logit spread beyond the fp32 exponent
//     range) the head is redone exactly: an all-key maximum per row first, then
//     the sums against that maximum.
//   - Phase 2 (score): the keys are read again (expected to hit L2/MALL) and
//     the MFMA accumulator starts from C = -lse_j (in accumulator units), so
//     the subtraction is free; the lane takes the max over its rows, the two
//     lane halves are merged, and one exp2 per key gives sigma(n).
// Scaling by 1/sqrt(d) happens in fp32 after accumulation; the bf16 beacons
// are never pre-scaled.

#include "bkv_internal.h"

namespace bkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kCs = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
constexpr int kTileWaves = 4;                                        // waves sharing a row group

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within its 32-row block) of accumulator element i for lane half hh.
__device__ __forceinline__ int acc_row(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

struct Tile {
    bf16x8_t b[8];
};

// B fragment of key n: d in [16s + 8hh, 16s + 8hh + 8) for k-step s.  Lanes
// past the last key re-read key N-1 (always in bounds); their results are
// masked by the caller.
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

template <int MBW, int kThreads>
__global__ __launch_bounds__(kThreads) void beacon_score_kernel(
    CacheView c, const float* __restrict__ beacons, const int32_t* __restrict__ counts, int K,
    int window, float bonus, float* __restrict__ scores, int stride, float* __restrict__ lse_out,
    Check ck, int32_t* status) {
    __shared__ int s_bt[kMaxBlocksPerReq];
    __shared__ float s_part[2 * kTileWaves][BKV_MAX_BEACONS];
    __shared__ float s_M[2 * kTileWaves];
    __shared__ float s_lse2[BKV_MAX_BEACONS];
    __shared__ float s_ref[BKV_MAX_BEACONS];
    __shared__ int s_live[BKV_MAX_BEACONS];
    __shared__ float s_pmax[kTileWaves][32];
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
    const int group = w / kTileWaves;
    const int q = w % kTileWaves;
    const int NG = blockDim.x / (kWave * kTileWaves);
    const int Kp = (K + 31) & ~31;
    const int MB = Kp / 32;
    const int mb0 = group * MBW;

    const int nb = (N + kBlock - 1) / kBlock;
    const int32_t* bt = c.block_table + (size_t)x.req * c.max_blocks;
    for (int i = tid; i < nb; i += blockDim.x) s_bt[i] = bt[i];
    for (int j = tid; j < Kp; j += blockDim.x)
        s_live[j] = (j < K) && counts[(size_t)hc * K + j] > 0;
    if (tid == 0) s_rescue = 0;
    __syncthreads();

    if (N == 0) {  // empty cache: nothing to score, every live lse is log(0)
        for (int j = tid; j < K; j += blockDim.x)
            if (lse_out) lse_out[(size_t)hc * K + j] = s_live[j] ? -INFINITY : __int_as_float(0x7fc00000);
        return;
    }

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
            for (int i = 0; i < 16; ++i) bits |= (uint32_t)(s_live[32 * (mb0 + m) + acc_row(i, hh)] != 0) << i;
        }
        live_bits[m] = bits;
    }

    const uint64_t kpool = c.k_pools[x.layer];
    const int ntiles = (N + 31) >> 5;
    const f32x16_t zero = {};
    // with four row blocks per wave the registers do not allow a second tile
    constexpr bool kPrefetch = MBW <= 2;

    // ---------------- phase 1: per-row log-sum-exp ----------------
    float Mw = -INFINITY;  // wave reference (log2 units)
    if (q < ntiles) {
        Tile t;
        const int n = 32 * q + col;
        load_key(t, kpool, s_bt, c.H, x.head, n, N, hh);
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
    float sum[MBW][16];
#pragma unroll
    for (int m = 0; m < MBW; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum[m][i] = 0.f;

    {
        auto consume = [&](const Tile& t, int tt) {
            const int n = 32 * tt + col;
            const bool full = 32 * tt + 32 <= N;
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
        };
        if (kPrefetch) {
            // two tiles alternate: one is consumed while the next is in flight
            Tile ta, tb;
            int tt = q;
            if (tt < ntiles) load_key(ta, kpool, s_bt, c.H, x.head, 32 * tt + col, N, hh);
            while (tt < ntiles) {
                if (tt + kTileWaves < ntiles)
                    load_key(tb, kpool, s_bt, c.H, x.head, 32 * (tt + kTileWaves) + col, N, hh);
                consume(ta, tt);
                tt += kTileWaves;
                if (tt >= ntiles) break;
                if (tt + kTileWaves < ntiles)
                    load_key(ta, kpool, s_bt, c.H, x.head, 32 * (tt + kTileWaves) + col, N, hh);
                consume(tb, tt);
                tt += kTileWaves;
            }
        } else {
            for (int tt = q; tt < ntiles; tt += kTileWaves) {
                Tile t;
                load_key(t, kpool, s_bt, c.H, x.head, 32 * tt + col, N, hh);
                consume(t, tt);
            }
        }
    }
    // lanes -> waves -> rows
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
        if (mb0 + m >= MB) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float v = half_sum(sum[m][i]);
            if (col == 0) s_part[w][32 * (mb0 + m) + acc_row(i, hh)] = v;
        }
    }
    if (lane == 0) s_M[w] = (q < ntiles) ? Mw : -INFINITY;
    __syncthreads();
    for (int j = tid; j < Kp; j += blockDim.x) {
        const int g = (j / 32) / MBW;
        float Mg = -INFINITY;
        for (int k2 = 0; k2 < kTileWaves; ++k2) Mg = fmaxf(Mg, s_M[g * kTileWaves + k2]);
        float total = 0.f;
        for (int k2 = 0; k2 < kTileWaves; ++k2) {
            const float Mk = s_M[g * kTileWaves + k2];
            if (Mk != -INFINITY) total += s_part[g * kTileWaves + k2][j] * exp2f(Mk - Mg);
        }
        const bool lv = s_live[j];
        const bool ok = total >= 0x1p-100f && total < INFINITY;
        if (lv && !ok) s_rescue = 1;
        s_lse2[j] = lv ? Mg + log2f(total) : INFINITY;
    }
    __syncthreads();

    if (s_rescue) {
        // Exact fallback: per-row maximum over all keys first, then the sums
        // against it (every term <= 1, the maximum term == 1).
#pragma unroll
        for (int m = 0; m < MBW; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) sum[m][i] = -INFINITY;
        for (int tt = q; tt < ntiles; tt += kTileWaves) {
            Tile t;
            const int n = 32 * tt + col;
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
            for (int k2 = 0; k2 < kTileWaves; ++k2) R = fmaxf(R, s_part[g * kTileWaves + k2][j]);
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
            for (int tt = q; tt < ntiles; tt += kTileWaves) {
                Tile t;
                const int n = 32 * tt + col;
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
            for (int k2 = 0; k2 < kTileWaves; ++k2) total += s_part[g * kTileWaves + k2][j];
            s_lse2[j] = s_live[j] ? s_ref[j] + log2f(total) : INFINITY;
        }
        __syncthreads();
    }

    if (lse_out) {
        for (int j = tid; j < K; j += blockDim.x)
            lse_out[(size_t)hc * K + j] = s_live[j] ? s_lse2[j] * kLn2 : __int_as_float(0x7fc00000);
    }

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
    const int iters = (ntiles + kTileWaves - 1) / kTileWaves;
    // one step of the score loop: tile tt of this wave (if any), merged across
    // the row groups; every wave runs the same number of steps (barriers)
    auto step = [&](int it, const Tile& cur, Tile& nxt) {
        const int tt = q + kTileWaves * it;
        const int n = 32 * tt + col;
        float mx = -INFINITY;
        if (tt < ntiles) {
            if (kPrefetch && tt + kTileWaves < ntiles)
                load_key(nxt, kpool, s_bt, c.H, x.head, n + 32 * kTileWaves, N, hh);
#pragma unroll
            for (int m = 0; m < MBW; ++m) {
                if (mb0 + m >= MB) continue;
                const f32x16_t acc = logits(A[m], cur, Cf[m]);
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
        }
        if (NG > 1) {  // merge the two row groups through LDS
            if (group == 1 && hh == 0) s_pmax[q][col] = mx;
            __syncthreads();
            if (group == 0) mx = fmaxf(mx, s_pmax[q][col]);
            __syncthreads();
        }
        if (group == 0 && hh == 0 && tt < ntiles && n >= P && n < N) {
            const float sigma = __builtin_amdgcn_exp2f(mx * kCs);
            out[n - P] = sigma + ((n >= N - window) ? bonus : 0.f);
        }
    };
    if (kPrefetch) {
        Tile ta, tb;
        if (q < ntiles) load_key(ta, kpool, s_bt, c.H, x.head, 32 * q + col, N, hh);
        for (int it = 0; it < iters; it += 2) {
            step(it, ta, tb);
            if (it + 1 < iters) step(it + 1, tb, ta);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
            Tile t;
            const int tt = q + kTileWaves * it;
            if (tt < ntiles) load_key(t, kpool, s_bt, c.H, x.head, 32 * tt + col, N, hh);
            step(it, t, t);
        }
    }
}

}  // namespace

hipError_t launch_beacon_score(const CacheView& c, const float* beacons, const int32_t* counts,
                               int K, int window, float bonus, float* scores, int stride,
                               float* lse, Check ck, int32_t* status, hipStream_t s) {
    const int HC = c.L * c.R * c.H;
    if (HC == 0) return hipSuccess;
    // Two row groups of four waves (8 waves, 2 per SIMD) whenever K > 32, so
    // that one wave's MFMA work overlaps another's exp/VALU work.
    if (K <= 32) {
        hipLaunchKernelGGL((beacon_score_kernel<1, 256>), dim3(HC), dim3(256), 0, s, c, beacons,
                           counts, K, window, bonus, scores, stride, lse, ck, status);
    } else if (K <= 64) {
        hipLaunchKernelGGL((beacon_score_kernel<1, 512>), dim3(HC), dim3(512), 0, s, c, beacons,
                           counts, K, window, bonus, scores, stride, lse, ck, status);
    } else if (K <= 128) {
        hipLaunchKernelGGL((beacon_score_kernel<2, 512>), dim3(HC), dim3(512), 0, s, c, beacons,
                           counts, K, window, bonus, scores, stride, lse, ck, status);
    } else {
        hipLaunchKernelGGL((beacon_score_kernel<4, 512>), dim3(HC), dim3(512), 0, s, c, beacons,
                           counts, K, window, bonus, scores, stride, lse, ck, status);
    }
    return hipGetLastError();
}

}  // namespace bkv
