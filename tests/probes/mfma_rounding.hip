// mfma_rounding.hip -- test-only kernel: one wave runs one
// v_mfma_f32_32x32x16_bf16 on fragments the host chooses, so a test can bound
// how far each fp32 result lies from the exact value.  The beacon maintenance
// kernel's error bound assumes every such result is within 8u (u = 2^-24) of
// the sum of the magnitudes it adds.  Lane l supplies its A and B fragments
// (8 bf16 bit patterns each, a[l*8 + e], b[l*8 + e]) and its 16 accumulator
// inputs c[l*16 + i]; d[l*16 + i] receives the outputs.  One block of 64
// threads; every access is lane * 8 + e or lane * 16 + i of caller buffers of
// 512 (a, b) and 1024 (c, d) elements.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void mfma_rounding_kernel(const uint16_t* a, const uint16_t* b,
                                                           const float* c, float* d) {
    const int l = threadIdx.x;
    u16x8 av, bv;
    for (int e = 0; e < 8; ++e) {
        av[e] = a[l * 8 + e];
        bv[e] = b[l * 8 + e];
    }
    f32x16_t acc;
    for (int i = 0; i < 16; ++i) acc[i] = c[l * 16 + i];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
    for (int i = 0; i < 16; ++i) d[l * 16 + i] = acc[i];
}

extern "C" int mfma_rounding_run(const void* a, const void* b, const void* c, void* d,
                                 void* stream) {
    if (!a || !b || !c || !d) return 1;
    hipLaunchKernelGGL(mfma_rounding_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const uint16_t*)a, (const uint16_t*)b, (const float*)c, (float*)d);
    return (int)hipGetLastError();
}
