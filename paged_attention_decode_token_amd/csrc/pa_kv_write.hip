// MXFP4 KV-cache write for gfx950: quantize new bf16 K and V rows to e2m1
// data with one e8m0 scale per 32 elements along head_dim, and store them in
// the paged caches the MXFP4 decode reads (ROCm/aiter PR #7056, "Summary":
// data [blocks][Hkv][page][D/2], scales [blocks][Hkv][page][D/32], written by a
// separate KV-write kernel).
//
// Encoding of one 32-element block (OCP Microscaling v1.0, conversion of
// scalars to an MX block, with e2m1's largest exponent 2):
//   E = floor(log2 max|v|) - 2, clamped to [-126, 127] (scale bytes 1..254,
//   the range the decode supports; an all-zero block gets byte 1);
//   element = v / 2^E rounded to nearest-even e2m1, saturating at +-6, with the
//   sign bit of v (so small negatives give -0);
//   a block holding NaN or an infinity gets scale byte 0xFF and zero data.
//
// HBM-bound: per (token, KV head) it reads 4D bytes (K and V in bf16) and
// writes 2 (D/2 + D/32) bytes. One lane takes one 16-byte chunk (8 elements) of
// K and the same chunk of V, so each load instruction of a wave reads 1 KB of
// consecutive input; four consecutive lanes hold one 32-element block, and
// their maximum is combined with two quad-permute DPP moves.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

#define KW_DEV __device__ __forceinline__

// Largest |bf16| bit pattern of the block: integer order of (bits & 0x7FFF)
// is the order of magnitudes, with infinity (0x7F80) and NaN (above) on top.
KW_DEV uint32_t block_abs_max(const uint4 w) {
    uint32_t m = 0;
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = max(m, ws[i] & 0x7FFFu);
        m = max(m, (ws[i] >> 16) & 0x7FFFu);
    }
    // quad_perm [1, 0, 3, 2] then [2, 3, 0, 1]: every lane of the quad ends
    // with the maximum of all four
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, true));
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, true));
    return m;
}

// e2m1 code of one bf16 element already scaled: the number of rounding
// thresholds |x| has passed. Between two neighbours the midpoint goes to the
// even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2,
// 3.5 -> 4, 5 -> 4; everything above 5 saturates at 6 (code 7).
KW_DEV uint32_t e2m1_code(uint32_t bf16_bits, float inv_scale) {
    const float a = fabsf(__builtin_bit_cast(float, (bf16_bits & 0x7FFFu) << 16) * inv_scale);
    const uint32_t q = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return q | ((bf16_bits >> 12) & 0x8u);
}

// Encode this lane's 8 elements of its block: 32 bits of packed codes
// (element 2k in the low nibble of byte k) and the block's scale byte.
KW_DEV void encode_chunk(const uint4 w, uint32_t* packed, uint32_t* scale_byte) {
    const uint32_t m = block_abs_max(w);
    if (m >= 0x7F80u) {
        *packed = 0;
        *scale_byte = 0xFFu;
        return;
    }
    const uint32_t ef = m >> 7;                   // bf16 exponent field of the block maximum
    const uint32_t byte = ef > 3u ? ef - 2u : 1u;  // E + 127 with E = (ef - 127) - 2, at least 1
    const float inv = __builtin_bit_cast(float, (254u - byte) << 23);  // 2^-E, a normal float
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t p = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p |= e2m1_code(ws[i] & 0xFFFFu, inv) << (8 * i);
        p |= e2m1_code(ws[i] >> 16, inv) << (8 * i + 4);
    }
    *packed = p;
    *scale_byte = byte;
}

typedef uint32_t kw_u32x4 __attribute__((ext_vector_type(4)));

KW_DEV uint4 load_stream(const uint16_t* p) {
    const kw_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const kw_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// U chunks of K and of V per lane, 256 * U consecutive chunks per workgroup.
template <int D, int U>
__global__ __launch_bounds__(256) void pa_kv_write_mxfp4_kernel(const KvWriteArgs a) {
    constexpr uint32_t CPR = D / 8;  // 16-byte chunks per (token, head) row
    const uint32_t base = blockIdx.x * (256u * U) + threadIdx.x;
    uint4 kw[U], vw[U];
    int32_t slot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t c = base + 256u * u;
        slot[u] = -1;
        kw[u] = make_uint4(0, 0, 0, 0);
        vw[u] = make_uint4(0, 0, 0, 0);
        if (c < a.chunks) {
            const uint32_t n = (c / CPR) / (uint32_t)a.num_kv_heads;
            slot[u] = a.slots[n];
            kw[u] = load_stream(a.key + (size_t)c * 8);
            vw[u] = load_stream(a.value + (size_t)c * 8);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // every lane of a quad shares its block, so all four take the same path
        uint32_t kp, ksb, vp, vsb;
        encode_chunk(kw[u], &kp, &ksb);
        encode_chunk(vw[u], &vp, &vsb);
        const uint32_t c = base + 256u * u;
        const int32_t s = slot[u];
        if (c < a.chunks && s >= 0 && s < a.num_slots) {
            const uint32_t r = c / CPR, cc = c % CPR;
            const uint32_t h = r % (uint32_t)a.num_kv_heads;
            const uint32_t page = (uint32_t)s / (uint32_t)a.page_size;
            const uint32_t prow = (uint32_t)s - page * (uint32_t)a.page_size;
            const size_t row = ((size_t)page * a.num_kv_heads + h) * a.page_size + prow;
            *reinterpret_cast<uint32_t*>(a.key_cache + row * (D / 2) + cc * 4) = kp;
            *reinterpret_cast<uint32_t*>(a.value_cache + row * (D / 2) + cc * 4) = vp;
            if ((cc & 3u) == 0) {
                a.key_scale[row * (D / 32) + cc / 4] = (uint8_t)ksb;
                a.value_scale[row * (D / 32) + cc / 4] = (uint8_t)vsb;
            }
        }
    }
}

constexpr int kWriteUnroll = 2;

template <int D>
hipError_t launch_d(const KvWriteArgs& a, hipStream_t stream) {
    const uint32_t per_wg = 256u * kWriteUnroll;
    const uint32_t grid = (a.chunks + per_wg - 1) / per_wg;
    hipLaunchKernelGGL((pa_kv_write_mxfp4_kernel<D, kWriteUnroll>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write_mxfp4(int head_dim, const KvWriteArgs& a, hipStream_t stream) {
    if (a.chunks == 0) return hipSuccess;
    switch (head_dim) {
        case 64: return launch_d<64>(a, stream);
        case 128: return launch_d<128>(a, stream);
        case 256: return launch_d<256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
