// decode_attention.hip -- single-query decode attention over the compacted
// paged cache: the step every selector hands its cache to (Random Attention
// article, section "发现四": the selectors share the attention kernels and the
// paging).  For each head-cache (layer, request, KV head) and each of its G
// query heads:
//     s_n = scale * (q . k_n),   out = sum_n softmax(s)_n v_n,   n < N.
// Keys were stored with their positions already applied, so slot order and
// the per-head slot/position mismatch left by compaction play no part.
//
// Layout (gfx950, HBM-bound: every K and V byte is read once):
//   - One wave per head-cache, four per workgroup.  A wave instruction moves
//     four consecutive slots: lane row r (16 lanes) holds slot base + 4i + r,
//     lane c of the row the 16 bytes [16c, 16c + 16) of its 256-byte K and V
//     rows.  Four slots are always inside one page, so each instruction reads
//     1 KiB of contiguous pool memory.
//   - q . k: each lane takes v_dot2_f32_bf16 over its eight dimensions for
//     every query head (q stays packed bf16 in registers), then a DPP sum over
//     the 16 lanes of the row gives every lane of the row the full dot.
//   - Online softmax per lane row over its own slots, one page (16 slots) per
//     step: the row's running maximum and sum are rescaled once per step, and
//     the same lanes that hold a V chunk hold its weight, so p . v needs no
//     exchange.  The next page's K and V are in flight during the step.
//   - The four rows of the wave are merged at the end with lane swaps.

#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kRows = 4;  // slots per wave instruction
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNoMax = -1.0e30f;  // finite start of a running maximum

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int kCtrl>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(
                   __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives it.
__device__ __forceinline__ float row16_sum(float x) {
    x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
    x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
    x = dpp_add<0x141>(x);  // row_half_mirror
    x = dpp_add<0x140>(x);  // row_mirror
    return x;
}

// The vector elements are copied to scalars before the bit cast: a bit cast
// applied to the element expression q[j] itself reads element 0 every time.
__device__ __forceinline__ float dot8(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t qw = q[j], kw = k[j];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw),
                                              __builtin_bit_cast(bf16x2_t, kw), acc, false);
    }
    return acc;
}

template <int GP>  // query heads per KV head, rounded up (1, 2, 4 or 8)
__global__ __launch_bounds__(kThreads) void decode_attention_kernel(
    CacheView c, const uint16_t* __restrict__ q, int G, float scale, float* __restrict__ out,
    int HC, int32_t* status) {
    __shared__ int s_bt[kWavesPerBlock][kMaxBlocksPerReq];

    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int hc = blockIdx.x * kWavesPerBlock + w;
    if (hc >= HC) return;  // the whole wave leaves; nothing below waits on other waves
    const HeadIdx x = split_hc(c, hc);
    // the workgroup's four waves may serve different requests: checks per wave
    if (!request_ok<true>(c, x.layer, x.req, hc, Check{-1, -1, 1, 0}, status)) return;
    const int N = slot_count(c, hc, x.req);
    const int rr = lane >> 4;          // slot within an instruction
    const int cc = lane & 15;          // 16-byte chunk of the row
    float* o = out + (size_t)hc * G * kHeadDim;

    // the head-cache's block-table row, in this wave's part of LDS
    int* bt = s_bt[w];
    const int32_t* btg = table_row(c, hc, x.req);
    for (int i = lane; i < (N + kBlock - 1) / kBlock; i += kWave) bt[i] = btg[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    u32x4 qp[GP];  // this lane's eight dimensions of every query head, packed bf16
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        qp[g] = u32x4{0u, 0u, 0u, 0u};
        if (g < G)
            qp[g] = load16((uint64_t)(q + ((size_t)hc * G + g) * kHeadDim + 8 * cc));
    }
    const float cs = scale * kLog2e;  // logits in log2 units

    float m[GP], l[GP], acc[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        m[g] = kNoMax;
        l[g] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
    }

    const uint64_t kbase = c.k_pools[x.layer];
    const uint64_t vbase = c.v_pools[x.layer];
    // K and V of one page (16 slots: kRows per instruction, four instructions).
    // Slots past N re-read slot N - 1 (in bounds) and are masked.
    auto load_page = [&](int base, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = min(base + kRows * i + rr, N - 1);
            const uint64_t off = row_offset(bt[n >> 4], c.H, x.head, n & 15) + 16 * cc;
            kr[i] = load16_nt(kbase + off);
            vr[i] = load16_nt(vbase + off);
        }
    };

    u32x4 kc[4], vc[4], kn[4], vn[4];
    if (N > 0) load_page(0, kc, vc);
    for (int base = 0; base < N; base += kBlock) {
        if (base + kBlock < N) load_page(base + kBlock, kn, vn);
        float s[4][GP];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = base + kRows * i + rr < N;
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                const float d = row16_sum(dot8(qp[g], kc[i], 0.f));
                s[i][g] = valid ? d * cs : -INFINITY;
            }
        }
        float vf[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vf[i][2 * j] = bf16_lo(vc[i][j]);
                vf[i][2 * j + 1] = bf16_hi(vc[i][j]);
            }
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float mb = fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]));
            const float mn = fmaxf(m[g], mb);
            const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
            m[g] = mn;
            float lg = l[g] * alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[g][j] *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(s[i][g] - mn);  // masked: exp2(-inf) = 0
                lg += p;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[g][j] = __builtin_fmaf(p, vf[i][j], acc[g][j]);
            }
            l[g] = lg;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kc[i] = kn[i];
            vc[i] = vn[i];
        }
    }

    // merge the four lane rows: common maximum, rescaled sums and accumulators
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        if (g >= G) break;
        float M = fmaxf(m[g], __shfl_xor(m[g], 16, kWave));
        M = fmaxf(M, __shfl_xor(M, 32, kWave));
        const float wgt = __builtin_amdgcn_exp2f(m[g] - M);
        float lt = l[g] * wgt;
        lt += __shfl_xor(lt, 16, kWave);
        lt += __shfl_xor(lt, 32, kWave);
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;  // N == 0 gives 0
        float r8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float a = acc[g][j] * wgt;
            a += __shfl_xor(a, 16, kWave);
            a += __shfl_xor(a, 32, kWave);
            r8[j] = a * inv;
        }
        if (rr == 0) {
            float4* dst = (float4*)(o + (size_t)g * kHeadDim + 8 * cc);
            dst[0] = make_float4(r8[0], r8[1], r8[2], r8[3]);
            dst[1] = make_float4(r8[4], r8[5], r8[6], r8[7]);
        }
    }
}

template <int GP>
hipError_t launch_g(const CacheView& c, const uint16_t* q, int G, float scale, float* out,
                    int32_t* status, hipStream_t s) {
    const int HC = c.L * c.R * c.H;
    const int blocks = (HC + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(decode_attention_kernel<GP>, dim3(blocks), dim3(kThreads), 0, s, c, q, G,
                       scale, out, HC, status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attention(const CacheView& c, const uint16_t* q, int G, float scale,
                                   float* out, int32_t* status, hipStream_t s) {
    if ((int64_t)c.L * c.R * c.H == 0) return hipSuccess;
    if (G <= 1) return launch_g<1>(c, q, G, scale, out, status, s);
    if (G <= 2) return launch_g<2>(c, q, G, scale, out, status, s);
    if (G <= 4) return launch_g<4>(c, q, G, scale, out, status, s);
    return launch_g<8>(c, q, G, scale, out, status, s);
}

}  // namespace bkv
