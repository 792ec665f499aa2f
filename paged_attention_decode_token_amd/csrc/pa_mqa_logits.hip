// MXFP4 paged MQA logits for gfx950: the sparse indexer's per-token scores
// (ROCm/aiter PR #5761, "Unify gfx950+gfx1250 MXFP4 paged MQA-logits": per
// query row, scores over the positions of its window [local_start, local_end)
// of the sequence row_to_batch names, one K head shared by every query head,
// K read through the block table; nothing outside the window is written).
//
//   out[r][t] = sum_h w[r][h] * relu(qhat[r][h] . khat[t]),  relu(x) = x < 0 ? 0 : x
//
// with q and K in MXFP4 (e2m1, one e8m0 scale per 32 elements), head_dim 128.
// relu keeps a NaN, so a NaN scale reaches the positions that read it.
//
// Built with the MFMA results in ordinary VGPRs (-amdgpu-mfma-vgpr-form): the
// accumulator-register form costs one copy per result element here.
//
// Work: a workgroup is one wave, which takes 192 positions of one row as twelve
// 16-token tiles. Measured cold on the 16 x 131072 decode: workgroups of one
// wave beat four (37.2 -> 36.3 us at 8 tiles) and eight (38.5 us); with one
// wave, 12 tiles (128 VGPRs, 4 waves per SIMD) 35.3 us, 16 tiles 35.3, 8 tiles
// 36.0, 4 tiles 41.3, 24 tiles 37.5 and 32 tiles 39.7 (2 waves per SIMD); the
// two-rows-per-sequence batch is fastest at 12 (19.6 us against 19.9 at 16).
// Double-buffered waves measured slower. Per tile and group of
// 16 heads, one
// v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 on both sides gives
// S[head][token]: A = the row's q (16 heads, loaded once per wave), B = the
// tile's 16 K rows. Lane layouts, measured on gfx950: A lane (m, g) nibble i
// is k = 32g + i of row m, B lane (n, g) nibble i is k = 32g + i of column n
// (element 2i in the low nibble), and each lane's scale byte applies to its own
// 32 elements; C lane (n, g) holds rows 4g .. 4g + 3 of column n. A lane then
// weights and sums its four heads of every group, and two lane swaps add the
// four lane groups. The wave's 128 scores leave in two whole-line stores of 64
// lanes, after the last tile.
//
// HBM-bound: per (row, position) one K row (64 data + 4 scale bytes) is read
// and one fp32 score written; the row's q, scales and weights (4.4 KB at 64
// heads) are read once per wave and stay in L2. K data is loaded and the
// scores stored nontemporally, the scores as whole lines (16 rows x 131072
// positions, 64 heads, cold: 39.7 -> 37.3 us per call; two rows per sequence
// over 32768 positions 21.7 -> 20.9 us). Nontemporal stores of 64-byte pieces
// did not merge in L2 and wrote 1.26x the score bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef int mq_i32x8 __attribute__((ext_vector_type(8)));
typedef float mq_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mq_u32x4 __attribute__((ext_vector_type(4)));

#define MQ_DEV __device__ __forceinline__

constexpr int kMqTiles = 12;             // 16-token tiles per wave
constexpr int kMqWave = 16 * kMqTiles;   // positions per wave
constexpr int kMqWaves = 1;              // waves per workgroup
constexpr int kMqChunk = kMqWaves * kMqWave;  // positions per workgroup
static_assert(kMqChunk == kMqChunkPositions, "the host sizes the grid by kMqChunkPositions");
constexpr uint32_t kMqXcds = 8;  // accelerator complex dies of an MI355X

MQ_DEV uint32_t mq_div(uint32_t x, int32_t d, int32_t shift) {
    return shift >= 0 ? x >> shift : x / (uint32_t)d;
}

// relu on the bits: the integer max with 0 keeps every non-negative float and
// turns negatives and -0 into +0 (one v_max_i32).
MQ_DEV float mq_relu(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// HT groups of 16 heads; head_dim 128 (one MFMA per group and tile). A wave
// owns kMqTiles 16-token tiles: it reads the block-table columns they span
// once (one per lane) and hands each tile its page id by a lane shuffle, then
// issues every tile's K load before the first MFMA, so no load waits on another.
template <int HT>
__global__ __launch_bounds__(64 * kMqWaves) void pa_mqa_logits_mxfp4_kernel(const MqaArgs a) {
    // Blocks are dispatched round-robin over the 8 XCDs; give each XCD a
    // contiguous range of (chunk, row) work items, rows fastest, so the rows
    // that share a chunk's K rows meet in one L2. The grid is a multiple of 8.
    const uint32_t per_xcd = gridDim.x / kMqXcds;
    const uint32_t item = (blockIdx.x % kMqXcds) * per_xcd + blockIdx.x / kMqXcds;
    if (item >= a.items) return;
    const int r = (int)(item % (uint32_t)a.num_rows);
    const int chunk = (int)(item / (uint32_t)a.num_rows);
    const int b = a.row_to_batch[r];
    if (b < 0 || b >= a.num_seqs) return;
    const int t0 = max(a.local_starts[r], 0);
    const int t1 = min(a.local_ends[r], a.max_pos);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int ws = chunk * kMqChunk + kMqWave * wave;  // this wave's first position
    if (ws >= t1 || ws + kMqWave <= t0) return;        // the whole wave, uniformly

    const int n = lane & 15, g = lane >> 4;
    const int H = HT * 16;

    // the row's q fragments (head 16i + n, block g) and the weights of the
    // heads this lane's accumulator rows hold (16i + 4g + 0..3), issued first:
    // they depend on the row only, and overlap the block-table read
    mq_u32x4 qd[HT];
    uint32_t qs[HT];
    mq_f32x4 w[HT];
#pragma unroll
    for (int i = 0; i < HT; ++i) {
        const size_t qrow = (size_t)r * H + 16 * i + n;
        qd[i] = *reinterpret_cast<const mq_u32x4*>(a.q + qrow * 64 + 16 * g);
        qs[i] = a.q_scale[qrow * 4 + g];
        w[i] = *reinterpret_cast<const mq_f32x4*>(a.weights + (size_t)r * H + 16 * i + 4 * g);
    }
    // page ids of the columns the wave's positions span (at most
    // kMqWave / 16 + 1 of them): lane l holds column cb + l, clamped into the
    // table, its entry clamped into the pool
    const uint32_t cb = mq_div((uint32_t)ws, a.page_size, a.page_shift);
    const int32_t* btab = a.block_tables + (size_t)b * a.max_blocks_per_seq;
    const uint32_t mycol = min(cb + (uint32_t)lane, (uint32_t)(a.max_blocks_per_seq - 1));
    const int mypage = min(max(btab[mycol], 0), a.num_blocks - 1);

    mq_u32x4 kd[kMqTiles];
    uint32_t ks[kMqTiles];
#pragma unroll
    for (int j = 0; j < kMqTiles; ++j) {
        // positions past the window (at most to the end of the wave's range)
        // are computed and not stored
        const uint32_t t = (uint32_t)(ws + 16 * j + n);
        const uint32_t colt = mq_div(t, a.page_size, a.page_shift);
        const uint32_t slot = t - colt * (uint32_t)a.page_size;
        const int page = __shfl(mypage, (int)(colt - cb));  // colt - cb <= kMqWave / 16 < 64
        const size_t krow = (size_t)page * a.page_size + slot;
        // nontemporal: each instruction reads 16 whole K rows (1 KB, whole
        // lines), used by this wave only (the scale bytes of a page share lines
        // between tiles and stay ordinary loads)
        kd[j] = __builtin_nontemporal_load(reinterpret_cast<const mq_u32x4*>(a.k_cache + krow * 64 + 16 * g));
        ks[j] = a.k_scale[krow * 4 + g];
    }
    // NaN reaches a score only through an e8m0 NaN scale (0xFF; e2m1 has no
    // NaN): a q scale makes every score of the row NaN, a K scale every score
    // of its token. Both are read off the scale bytes, so relu may turn a NaN
    // into 0. Scores are assumed to stay within fp32 range.
    bool qbad = false;
#pragma unroll
    for (int i = 0; i < HT; ++i) qbad |= qs[i] == 0xFFu;
    const bool row_nan = __any(qbad);
    const float qnan = __builtin_nanf("");
    float* orow = a.out + (size_t)r * a.out_stride;
    // every lane group ends a tile with the same sum (the two lane swaps add
    // the same pairs, in either order), so lane (n, g) keeps the score of token
    // n of tile 4 h + g in keep[h]: lane l then holds position ws + 64 h + l,
    // and each 64 positions of the wave's scores leave in one store of 256 bytes
    static_assert(kMqTiles % 4 == 0, "whole stores of 64 positions");
    constexpr int KH = kMqTiles / 4;
    float keep[KH];
#pragma unroll
    for (int h = 0; h < KH; ++h) keep[h] = 0.f;

#pragma unroll
    for (int j = 0; j < kMqTiles; ++j) {
        const mq_i32x8 kb = {(int)kd[j].x, (int)kd[j].y, (int)kd[j].z, (int)kd[j].w, 0, 0, 0, 0};
        mq_f32x4 s[HT];
#pragma unroll
        for (int i = 0; i < HT; ++i) {
            const mq_i32x8 qa = {(int)qd[i].x, (int)qd[i].y, (int)qd[i].z, (int)qd[i].w, 0, 0, 0, 0};
            const mq_f32x4 z = {0.f, 0.f, 0.f, 0.f};
            s[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, kb, z, 4, 4, 0, (int)qs[i], 0, (int)ks[j]);
        }
        float acc = ks[j] == 0xFFu ? qnan : 0.f;
#pragma unroll
        for (int i = 0; i < HT; ++i) {
            acc += w[i].x * mq_relu(s[i].x);
            acc += w[i].y * mq_relu(s[i].y);
            acc += w[i].z * mq_relu(s[i].z);
            acc += w[i].w * mq_relu(s[i].w);
        }
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        if (row_nan) acc = qnan;
        if ((j & 3) == g) keep[j >> 2] = acc;
    }
#pragma unroll
    for (int h = 0; h < KH; ++h) {
        const int t = ws + 64 * h + lane;
        if (t >= t0 && t < t1) __builtin_nontemporal_store(keep[h], orow + t);  // written once, read later
    }
}

template <int HT>
hipError_t launch_h(const MqaArgs& a, hipStream_t stream) {
    const uint32_t grid = (a.items + kMqXcds - 1) / kMqXcds * kMqXcds;
    hipLaunchKernelGGL((pa_mqa_logits_mxfp4_kernel<HT>), dim3(grid), dim3(64 * kMqWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mqa_logits_mxfp4(int num_heads, const MqaArgs& a, hipStream_t stream) {
    if (a.items == 0) return hipSuccess;
    switch (num_heads) {
        case 16: return launch_h<1>(a, stream);
        case 32: return launch_h<2>(a, stream);
        case 64: return launch_h<4>(a, stream);
        case 128: return launch_h<8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
