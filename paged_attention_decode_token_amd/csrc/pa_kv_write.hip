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
// K and the same chunk of V; four consecutive lanes hold one 32-element block,
// and their maximum is combined with two quad-permute DPP moves. The e2m1
// rounding is the hardware's scaled conversion, one instruction per two
// elements. Measured on MI355X for this traffic (4.3 GB read, 1.1 GB written
// per call), streaming reads alone reach 7.0 TB/s, with linear writes 6.5 TB/s,
// and with the writes scattered over pages as 64-byte half lines 5.7 TB/s,
// which is why each wave writes whole runs of one head's rows. The data stores
// are nontemporal (16 x 131072 tokens, 4 heads, cold: 961 -> 944 us per call);
// the scale stores, which share lines between neighbouring waves, are not.
// Waves that each take four token groups, their loads issued together,
// measured slower (1005 us): many short waves hide the latency better.
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

typedef __bf16 kw_bf16x2 __attribute__((ext_vector_type(2)));

// Encode this lane's 8 elements of its block: 32 bits of packed codes
// (element 2k in the low nibble of byte k) and the block's scale byte.
// v_cvt_scalef32_pk_fp4_bf16 converts two bf16 values to e2m1 as v / scale,
// rounded to nearest even and saturated at +-6, with the sign kept (so small
// negatives give -0); measured on gfx950 to match that definition for every
// finite bf16 bit pattern, subnormals included, at scales 2^-126 .. 2^125.
// Each call fills one byte of the result, low nibble first.
KW_DEV void encode_chunk(const uint4 w, uint32_t* packed, uint32_t* scale_byte) {
    const uint32_t m = block_abs_max(w);
    const uint32_t ef = m >> 7;                   // bf16 exponent field of the block maximum
    const uint32_t byte = ef > 3u ? ef - 2u : 1u;  // E + 127 with E = (ef - 127) - 2, at least 1
    const float scale = __builtin_bit_cast(float, byte << 23);  // 2^E, a normal float
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(kw_bf16x2, w.x), scale, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(kw_bf16x2, w.y), scale, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(kw_bf16x2, w.z), scale, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(kw_bf16x2, w.w), scale, 3);
    const bool nonfinite = m >= 0x7F80u;  // NaN or an infinity in the block
    *packed = nonfinite ? 0u : p;
    *scale_byte = nonfinite ? 0xFFu : byte;
}

typedef uint32_t kw_u32x4 __attribute__((ext_vector_type(4)));

KW_DEV uint4 load_stream(const uint16_t* p) {
    const kw_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const kw_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr uint32_t kXcds = 8;  // accelerator complex dies of an MI355X

// x / d for a divisor the whole launch shares: a shift when d is a power of two
// (shift >= 0, the usual head counts and page sizes), else a division.
KW_DEV uint32_t div_by(uint32_t x, int32_t d, int32_t shift) {
    return shift >= 0 ? x >> shift : x / (uint32_t)d;
}

// Gather the scale bytes of one token row's blocks (held by the lanes with
// chunk % 4 == 0) into the row's first lane of each 16-lane group, so that one
// store writes up to four of them. Returns the packed bytes (valid in lanes
// whose chunk % 16 == 0, or % 8 == 0 when a row has only two blocks).
template <uint32_t CPR>
KW_DEV uint32_t gather_scales(uint32_t b) {
    if constexpr (CPR >= 16) {
        const uint32_t b4 = (uint32_t)__shfl_down((int)b, 4, 16), b8 = (uint32_t)__shfl_down((int)b, 8, 16),
                       b12 = (uint32_t)__shfl_down((int)b, 12, 16);
        return b | (b4 << 8) | (b8 << 16) | (b12 << 24);
    } else {
        return b | ((uint32_t)__shfl_down((int)b, 4, 8) << 8);
    }
}

// One wave takes TPW = 64 / CPR consecutive tokens of one KV head: lane l holds
// chunk l % CPR of token l / CPR. Loads read whole 256-byte rows; in a prefill,
// where consecutive tokens land in consecutive rows of a page, the wave's data
// stores cover TPW * D / 2 contiguous bytes. Wave task q = (token group q / Hkv,
// head q % Hkv); four per workgroup.
template <int D>
__global__ __launch_bounds__(256) void pa_kv_write_mxfp4_kernel(const KvWriteArgs a) {
    constexpr uint32_t CPR = D / 8;     // 16-byte chunks per (token, head) row
    constexpr uint32_t TPW = 64 / CPR;  // tokens per wave
    const uint32_t lane = threadIdx.x & 63u;
    // Workgroups are dispatched round-robin over the 8 XCDs, each with its own
    // L2. Give every XCD a contiguous range of the work (the grid is a multiple
    // of 8), so that the neighbouring workgroups whose stores share a 128-byte
    // line -- a scale line holds 128 / (D / 32) tokens -- meet in one L2 instead
    // of writing back partial lines from eight.
    const uint32_t per_xcd = gridDim.x / kXcds;
    const uint32_t wg = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const uint32_t q = wg * 4u + (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t H = (uint32_t)a.num_kv_heads;
    const uint32_t tg = div_by(q, a.num_kv_heads, a.heads_shift), h = q - tg * H;
    const uint32_t t = tg * TPW + lane / CPR, cc = lane % CPR;
    const bool live = q < a.wave_tasks && t < (uint32_t)a.num_tokens;
    uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
    int32_t s = -1;
    if (live) {
        const size_t c = ((size_t)t * H + h) * CPR + cc;
        s = a.slots[t];
        kw = load_stream(a.key + c * 8);
        vw = load_stream(a.value + c * 8);
    }
    // every lane of a quad shares its block, so all four take the same path
    uint32_t kp, ksb, vp, vsb;
    encode_chunk(kw, &kp, &ksb);
    encode_chunk(vw, &vp, &vsb);
    ksb = gather_scales<CPR>(ksb);
    vsb = gather_scales<CPR>(vsb);
    if (live && s >= 0 && s < a.num_slots) {
        const uint32_t page = div_by((uint32_t)s, a.page_size, a.page_shift);
        const uint32_t prow = (uint32_t)s - page * (uint32_t)a.page_size;
        const size_t row = ((size_t)page * H + h) * a.page_size + prow;
        __builtin_nontemporal_store(kp, reinterpret_cast<uint32_t*>(a.key_cache + row * (D / 2) + cc * 4));
        __builtin_nontemporal_store(vp, reinterpret_cast<uint32_t*>(a.value_cache + row * (D / 2) + cc * 4));
        if constexpr (CPR >= 16) {
            if ((cc & 15u) == 0) {
                *reinterpret_cast<uint32_t*>(a.key_scale + row * (D / 32) + cc / 4) = ksb;
                *reinterpret_cast<uint32_t*>(a.value_scale + row * (D / 32) + cc / 4) = vsb;
            }
        } else {
            if (cc == 0) {
                *reinterpret_cast<uint16_t*>(a.key_scale + row * (D / 32)) = (uint16_t)ksb;
                *reinterpret_cast<uint16_t*>(a.value_scale + row * (D / 32)) = (uint16_t)vsb;
            }
        }
    }
}

template <int D>
hipError_t launch_d(const KvWriteArgs& a, hipStream_t stream) {
    const uint32_t wgs = (a.wave_tasks + 3u) / 4u;
    const uint32_t grid = (wgs + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((pa_kv_write_mxfp4_kernel<D>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write_mxfp4(int head_dim, const KvWriteArgs& a, hipStream_t stream) {
    if (a.wave_tasks == 0) return hipSuccess;
    switch (head_dim) {
        case 64: return launch_d<64>(a, stream);
        case 128: return launch_d<128>(a, stream);
        case 256: return launch_d<256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
