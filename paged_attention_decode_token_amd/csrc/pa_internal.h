// Internal interface between the host side (pa_api.cpp) and the kernels
// (pa_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum KvKind { KV_BF16 = 0, KV_FP8 = 1, KV_MXFP4 = 2 };
enum ScaleKind { SC_NONE = 0, SC_TENSOR = 1, SC_TOKEN = 2 };

// Tokens per planning tile: the unit of work per sequence (ROCm/aiter PR #7092,
// "Root cause": ceil(context_len / 256) tiles per sequence).
constexpr int kTileTokens = 256;
// Threads per workgroup of the tile kernel: four 64-wide waves, each owning
// 64 tokens of every tile (PR #7056, "Behavior and intent").
constexpr int kTileThreads = 256;

struct TileArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* ks;  // per-tensor fp32[1], per-token fp32 table, or MXFP4 e8m0 bytes
    const void* vs;
    const int32_t* block_tables;
    const int32_t* context_lens;
    void* out;                 // bf16 [B][qlen][Hq][D]
    const int32_t* tasks;      // int32 x 4 per task, one per workgroup
    const int32_t* seq_parts;  // int32 x 2 per (sequence, KV head): partitions, first partial unit
    float* part_ml;            // [units][rows][2]: running max (base 2), sum of weights
    float* part_o;             // [units][rows][D]: weighted sum of V (times the per-tensor V scale)
    int32_t num_seqs, qlen, num_kv_heads, q_per_kv, rows, max_blocks, num_blocks;
    float scale_log2;  // softmax_scale * log2(e)
    int32_t plan_free;  // 1: tasks follow from the block index, the task list and seq_parts are unused:
                        // uniform_parts tasks per (sequence, KV head), each part_tiles tiles
                        // (the last open-ended); with more than one, partition p of
                        // (sequence b, KV head h) writes partial unit (b Hkv + h) uniform_parts + p
    int32_t uniform_parts;  // plan_free: partitions per sequence (0 or 1: direct output)
    int32_t part_tiles;     // plan_free with uniform_parts > 1: tiles per partition
    int32_t causal;     // 1: query token i attends to t < L - qlen + i + 1
    int32_t window;     // > 0: and to t >= (that end) - window
};

struct KernelKey {
    int kv, scale, vt, head_dim, page, ntiles_n, q_fp8, mx_scaled;
    int win;  // causal rows (qlen > 1) or a sliding window
};

// MXFP4 KV-cache write: one 16-byte chunk (8 elements) of K and of V per lane,
// one wave per (group of 64 / (D / 8) tokens, KV head).
struct KvWriteArgs {
    const uint16_t* key;    // bf16 [tokens][Hkv][D]
    const uint16_t* value;
    const int32_t* slots;   // [tokens]
    uint8_t* key_cache;     // [blocks][Hkv][page][D/2]
    uint8_t* value_cache;
    uint8_t* key_scale;     // [blocks][Hkv][page][D/32]
    uint8_t* value_scale;
    uint32_t wave_tasks;    // ceil(tokens / (64 / (D / 8))) * Hkv
    int32_t num_tokens, num_kv_heads, page_size, num_slots;
    int32_t heads_shift, page_shift;  // log2 of Hkv / page_size when a power of two, else -1
};

// Launch the KV write for head_dim 64, 128 or 256 (hipErrorInvalidValue otherwise).
hipError_t launch_kv_write_mxfp4(int head_dim, const KvWriteArgs& args, hipStream_t stream);

// MXFP4 paged MQA logits (head_dim 128): one workgroup per (chunk of
// kMqChunkPositions positions, row) work item.
constexpr int kMqChunkPositions = 192;
struct MqaArgs {
    const uint8_t* q;        // [rows][H][64]
    const uint8_t* q_scale;  // [rows][H][4]
    const float* weights;    // [rows][H]
    const uint8_t* k_cache;  // [blocks][page][64]
    const uint8_t* k_scale;  // [blocks][page][4]
    const int32_t* block_tables;
    const int32_t* row_to_batch;
    const int32_t* local_starts;
    const int32_t* local_ends;
    float* out;              // [rows][out_stride]
    uint32_t items;          // rows * chunks
    int32_t num_rows, page_size, page_shift, num_blocks, num_seqs, max_blocks_per_seq, out_stride;
    int32_t max_pos;         // min(max_blocks_per_seq * page_size, out_stride)
};

// Launch the MQA-logits kernel for 16, 32, 64 or 128 heads (hipErrorInvalidValue otherwise).
hipError_t launch_mqa_logits_mxfp4(int num_heads, const MqaArgs& args, hipStream_t stream);

// Launch the tile kernel for `key` (returns hipErrorInvalidValue for a key with
// no compiled instance).
hipError_t launch_tile(const KernelKey& key, const TileArgs& args, int num_tasks, hipStream_t stream);

// Launch the cross-partition log-sum-exp merge for every output row.
hipError_t launch_merge(const TileArgs& args, int head_dim, hipStream_t stream);

// Whether an instance exists for `key`.
bool have_tile_kernel(const KernelKey& key);

// Tile-kernel workgroups of `key` that fit on one compute unit at once.
int tile_blocks_per_cu(const KernelKey& key);

}  // namespace pa
