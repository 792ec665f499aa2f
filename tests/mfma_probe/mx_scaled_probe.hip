// Numerics probe of the block-scaled MFMA the MXFP4 decode uses for QK
// (v_mfma_scale_f32_16x16x128_f8f6f4, fp4 A with e8m0 scales per 32 k, e4m3 B
// with e8m0 scales), for the GPU test that characterises its accumulation.
// Test infrastructure only: the decode library does not use this file.
//
// One wave per 16 x 16 tile: A is 16 rows (tokens) of 128 fp4 values (64
// bytes, element 2i in the low nibble) with 4 scale bytes each, B is 16 rows
// (query rows) of 128 e4m3 bytes with 4 scale bytes each. The 128-deep
// reduction is computed four ways:
//   0  one instruction over all four 32-element blocks;
//   1  four instructions, each with only block j's A values (the others
//      zero), accumulating in the instruction's fp32 C operand;
//   2  the same four instructions with C = 0, their results added in fp32;
//   3  two instructions over blocks {0, 1} and {2, 3}, accumulating in C.
// out[((tile * 4 + variant) * 16 + token) * 16 + row].
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void mx_probe_kernel(const uint8_t* A, const uint8_t* As, const uint8_t* Bq,
                                                      const uint8_t* Bs, float* out, int ntiles) {
    const int t = blockIdx.x;
    if (t >= ntiles) return;
    const int lane = threadIdx.x, m = lane & 15, g = lane >> 4;
    // A lane (m, g): token m, k = 32g + [0, 32) (16 bytes); its scale byte is block g's
    const uint32_t* a4 = reinterpret_cast<const uint32_t*>(A + (size_t)t * 16 * 64 + m * 64 + 16 * g);
    const int sa = As[(size_t)t * 16 * 4 + m * 4 + g];
    // B lane (n = m, g): bytes k = 16g + [0, 16), then k = 64 + 16g + [0, 16); scale of block g
    const uint8_t* b = Bq + (size_t)t * 16 * 128 + m * 128;
    const uint32_t* blo = reinterpret_cast<const uint32_t*>(b + 16 * g);
    const uint32_t* bhi = reinterpret_cast<const uint32_t*>(b + 64 + 16 * g);
    const int sb = Bs[(size_t)t * 16 * 4 + m * 4 + g];
    const i32x8 av = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
    const i32x8 bv = {(int)blo[0], (int)blo[1], (int)blo[2], (int)blo[3],
                      (int)bhi[0], (int)bhi[1], (int)bhi[2], (int)bhi[3]};
    const i32x8 none = {0, 0, 0, 0, 0, 0, 0, 0};
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 r[4];
    r[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 0, 0, sa, 0, sb);
    f32x4 c1 = z, s2 = z, c3 = z;
    for (int j = 0; j < 4; ++j) {
        const i32x8 aj = g == j ? av : none;
        c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aj, bv, c1, 4, 0, 0, sa, 0, sb);
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aj, bv, z, 4, 0, 0, sa, 0, sb);
        for (int e = 0; e < 4; ++e) s2[e] += p[e];
    }
    for (int h = 0; h < 2; ++h) {
        const i32x8 ah = (g >> 1) == h ? av : none;
        c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, bv, c3, 4, 0, 0, sa, 0, sb);
    }
    r[1] = c1;
    r[2] = s2;
    r[3] = c3;
    // C lane (n = m, g) element e is S[token 4g + e][row n]
    for (int v = 0; v < 4; ++v)
        for (int e = 0; e < 4; ++e) out[(((size_t)t * 4 + v) * 16 + (4 * g + e)) * 16 + m] = r[v][e];
}

// Device pointers; returns a hipError_t value (0 on success). Enqueued on `stream`.
extern "C" int mx_probe_run(const void* A, const void* As, const void* Bq, const void* Bs, void* out, int ntiles,
                            void* stream) {
    if (ntiles <= 0) return 0;
    hipLaunchKernelGGL(mx_probe_kernel, dim3(ntiles), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(As),
                       static_cast<const uint8_t*>(Bq), static_cast<const uint8_t*>(Bs), static_cast<float*>(out),
                       ntiles);
    return (int)hipGetLastError();
}
