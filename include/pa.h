/*
 * pa.h -- C ABI of the paged-attention decode library (libpa.so, gfx950 / MI355X).
 *
 * One decode step of attention over a paged KV cache: for every sequence b,
 * query token i < qlen and query head h, read K/V through the page block
 * table up to context_lens[b], score Q against K, softmax, multiply by V, and
 * merge the per-partition partial results (ROCm/aiter PR #7092 "pa_decode:
 * zero V rows past the context before PV", sections "Root cause" and "Fix";
 * ROCm/aiter PR #7056 "pa_decode: MXFP4 K/V in the shared PA tile kernel",
 * sections "Summary" and "Behavior and intent").
 *
 *   kvh       = h / q_per_kv                                (heads grouped contiguously)
 *   s_t       = softmax_scale * dot(qhat, K_t)              for t < L = context_lens[b]
 *   out[b,i,h]= sum_t softmax(s)_t * V_t                    (bf16, round to nearest even)
 *   L = 0     -> out row = 0
 *
 * Rows no sequence owns (block 0 pinned pages, the tail of a sequence's last
 * page, anything at or past L, and with a sliding window anything before every
 * query row's window) never influence out: their scores are -inf, and on the
 * masked tiles their V bytes and per-token scales are zeroed before the P*V
 * product (PR #7092, section "Fix"). NaN/Inf there is harmless.
 *
 * Everything is plain C: pointers, sizes and enums. PyTorch (or any caller)
 * owns the device tensors; the library owns only what pa_plan allocates.
 *
 * Error behaviour: every entry point returns a pa_status; on failure,
 * pa_last_error() gives a thread-local message. No entry point aborts or
 * throws across the ABI.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. PA_ERR_INVALID_ARG: malformed input (NULL, misaligned,
 * inconsistent sizes). PA_ERR_UNSUPPORTED: well-formed but outside what the
 * kernels implement (e.g. MXFP4 with page size 64, head_dim 64, not gfx950).
 * PA_ERR_HIP: a HIP runtime call failed. PA_ERR_OOM: device allocation failed. */
typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,
    PA_ERR_UNSUPPORTED = 2,
    PA_ERR_HIP = 3,
    PA_ERR_OOM = 4
} pa_status;

/* KV cache element formats.
 * PA_KV_BF16      : bfloat16.
 * PA_KV_FP8_E4M3  : OCP e4m3fn bytes (bias 7, max 448, S.1111.111 = NaN), with
 *                   per-tensor or per-token fp32 scales (PR #7092, "Tests").
 * PA_KV_MXFP4     : OCP MX e2m1 pairs (element 2i in the low nibble) plus one
 *                   e8m0 scale byte per 32 elements along head_dim (PR #7056,
 *                   "Summary"). */
typedef enum pa_kv_dtype { PA_KV_BF16 = 0, PA_KV_FP8_E4M3 = 1, PA_KV_MXFP4 = 2 } pa_kv_dtype;

typedef enum pa_scale_mode {
    PA_SCALE_NONE = 0,       /* bf16 and MXFP4 (MXFP4 carries its own block scales) */
    PA_SCALE_PER_TENSOR = 1, /* fp8: k_scale, v_scale = device fp32[1] each          */
    PA_SCALE_PER_TOKEN = 2   /* fp8: k_scale, v_scale = device fp32 [num_blocks][Hkv][page_size] */
} pa_scale_mode;

/* V layout. PLAIN: [num_blocks][Hkv][page_size][head_dim] (token-major, like K).
 * TRANSPOSED ("trans_v", PR #7092 "Tests"): [num_blocks][Hkv][head_dim][page_size]. */
typedef enum pa_v_layout { PA_V_PLAIN = 0, PA_V_TRANSPOSED = 1 } pa_v_layout;

/* Query format. PA_Q_FP8_E4M3 is accepted only with an MXFP4 cache, where it is
 * used as stored with unit scale (PR #7056, "Summary"). A bf16 query with an
 * MXFP4 cache is quantized to e4m3 per (sequence, query token, head) row with
 * a power-of-two scale 2^e, e the smallest integer with max|q| <= 448 * 2^e. */
typedef enum pa_q_dtype { PA_Q_BF16 = 0, PA_Q_FP8_E4M3 = 1 } pa_q_dtype;

/* Problem descriptor. All sizes are element counts unless stated.
 *   num_seqs            B, sequences in the batch (>= 0)
 *   qlen                query tokens per sequence (1..4 typical). rows = qlen * q_per_kv
 *                       query rows share a KV head: at most 64, and at most 32
 *                       with head_dim 256 (64 rows at head_dim 256 would need 256
 *                       accumulator registers per lane for O alone); ROCm/aiter
 *                       PR #7092, "Tests": its unowned-row matrix has a 64-row
 *                       case (qlen 4, GQA 16, head_dim 128)
 *   num_kv_heads        Hkv
 *   q_per_kv            G, query heads per KV head (Hq = Hkv * G)
 *   head_dim            D: 128 or 256 (MXFP4: 128)
 *   page_size           tokens per page: 16, 64 or 128 (MXFP4: 128)
 *   num_blocks          pages in the pool (>= 1; block 0 always exists)
 *   max_blocks_per_seq  width of block_tables
 *   max_context_len     upper bound of context_lens (used when no host lengths are given)
 *   kv_dtype, scale_mode, v_layout, q_dtype   see the enums (MXFP4: PLAIN only)
 *   softmax_scale       0 -> 1/sqrt(head_dim)
 *   max_partitions      0 -> 64; upper bound of partitions per sequence
 *   task_budget         0 -> automatic: the tiles-per-task target with the lowest
 *                       estimated completion time when tasks run longest first
 *                       on the resident workgroup slots; > 0: about this many tasks
 *   mxfp4_scaled_qk     MXFP4 only. 0 (default): K is widened exactly to bf16 and
 *                       QK runs on the bf16 MFMA with fp32 accumulation. 1: QK
 *                       runs on the block-scaled fp4 x fp8 MFMA
 *                       (v_mfma_scale_f32_16x16x128_f8f6f4): fp4 K with its e8m0
 *                       block scales times the e4m3 query with its row scale
 *                       (PR #7056, "Behavior and intent"), about 1 percent faster
 *                       at 131072 tokens. On gfx950 that instruction keeps one
 *                       32-element block's sum to about 2^-14 of the block's
 *                       largest product (2^-12.6 with the query scaled up to
 *                       448), however the reduction is split across
 *                       instructions; where two top logits nearly tie, an output
 *                       element can then move by more than 2e-2 * max(1, |o|).
 *   causal              0 (default): every query token attends to all of [0, L).
 *                       1: the qlen query tokens are the last qlen positions of
 *                       the sequence (their K/V already in the cache, as in
 *                       multi-token verification); token i attends to
 *                       t < e_i = L - qlen + i + 1 ([P1] "Tests": qlen 1-4
 *                       probes; the causal select of the later tile commit).
 *   window              0 (default): no sliding window. W > 0: token i attends
 *                       only to t >= e_i - W as well (the W positions ending at
 *                       its own). Let s_lo = max(0, e_0 - W), the start of the
 *                       earliest row's window (e_0 = L - qlen + 1 when causal,
 *                       else L). Tokens before s_lo are seen by no row and are
 *                       treated like tokens at or past L: block-table columns
 *                       j < floor(s_lo / page_size) (pages wholly before s_lo)
 *                       are never read, and tokens of the page holding s_lo
 *                       that lie before it may hold anything (NaN, Inf,
 *                       garbage, including their per-token scales): their
 *                       scores are -inf and their V bytes and V scales are
 *                       zeroed before P*V. Tokens in [s_lo, L) must hold the
 *                       sequence's data even where some rows do not see them.
 *                       A row whose range is empty is written as 0. Not offered
 *                       with MXFP4 ([P2] "Summary": sliding window is refused
 *                       there).
 */
typedef struct pa_problem {
    int32_t num_seqs;
    int32_t qlen;
    int32_t num_kv_heads;
    int32_t q_per_kv;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t kv_dtype;
    int32_t scale_mode;
    int32_t v_layout;
    int32_t q_dtype;
    float softmax_scale;
    int32_t max_partitions;
    int32_t task_budget;
    int32_t mxfp4_scaled_qk;
    int32_t causal;
    int32_t window;
} pa_problem;

/* Opaque plan: validated problem, task list and partition workspace. */
typedef struct pa_plan pa_plan_t;

/* A HIP stream (hipStream_t); NULL means the default stream. */
typedef void* pa_stream_t;

/*
 * pa_plan -- validate the problem, probe the device once per process (refuses
 * anything but gfx950 with PA_ERR_UNSUPPORTED), cut every sequence into
 * 256-token tiles and the tiles into partitions (PR #7092, "Root cause": only
 * ceil(L/256) tiles per sequence exist; PR #7056, "Bandwidth": tile kernel plus
 * partition reducer), and allocate the device workspace (task list, partition
 * partials). The task list is copied to the device on `stream`.
 *
 * host_context_lens: optional host int32[num_seqs]. With it, partitions follow
 * the real lengths (the device lengths passed to pa_decode must then be equal
 * or shorter; with a window, a sequence's first partition starts at the device
 * window's first tile, so a shorter device length still covers its window).
 * Without it, every sequence is split as if it had max_context_len tokens and
 * the kernels clamp to the device lengths.
 *
 * Ownership: *plan_out belongs to the caller; release it with pa_plan_destroy.
 * Refusals: see pa_status. A host length above max_blocks_per_seq * page_size
 * or above max_context_len is PA_ERR_INVALID_ARG.
 */
pa_status pa_plan(const pa_problem* problem, const int32_t* host_context_lens, pa_stream_t stream,
                  pa_plan_t** plan_out);

/*
 * pa_decode -- enqueue the decode on `stream`: the tile kernel, then (when a
 * sequence has more than one partition) the log-sum-exp merge kernel. It
 * neither allocates nor synchronizes. Calls that share a plan must be
 * stream-ordered, since the plan owns the partition workspace.
 *
 * All pointers are caller-owned device memory, 16-byte aligned:
 *   query         [B][qlen][Hq][D]    bf16, or e4m3 bytes (PA_Q_FP8_E4M3)
 *   key_cache     [num_blocks][Hkv][page][D] bf16 / e4m3; MXFP4: uint8 [..][page][D/2]
 *   value_cache   like key_cache; TRANSPOSED: [num_blocks][Hkv][D][page]
 *   k_scale, v_scale  NULL (bf16); fp32[1] (per-tensor); fp32 [num_blocks][Hkv][page]
 *                 (per-token); MXFP4: uint8 e8m0 [num_blocks][Hkv][page][D/32]
 *   block_tables  int32 [B][max_blocks_per_seq]
 *   context_lens  int32 [B]
 *   out           bf16 [B][qlen][Hq][D]; every element is written
 *
 * Device-side guarantees: block_tables columns >= ceil(L/page) are never read;
 * tiles past ceil(L/256) are never read; tokens >= L never affect out; with a
 * window, columns and tokens before s_lo (see pa_problem.window) are treated
 * the same way; page ids
 * outside [0, num_blocks) and lengths outside [0, max_blocks_per_seq * page]
 * are clamped so that no access leaves the caller's buffers (the output of
 * such a sequence is then unspecified).
 */
pa_status pa_decode(const pa_plan_t* plan, const void* query, const void* key_cache, const void* value_cache,
                    const void* k_scale, const void* v_scale, const int32_t* block_tables,
                    const int32_t* context_lens, void* out, pa_stream_t stream);

/*
 * pa_decode_direct -- plan-free decode: one task per (sequence, KV head),
 * derived from the workgroup index, over every tile of the sequence up to the
 * device context length; each task normalizes and stores its output rows
 * itself, so there is no plan, no partition reduce, no workspace and no host
 * copy of the lengths (ROCm/aiter PR #7056, "Bandwidth": the plan-free mode
 * whose tasks follow from the block index, and the direct output of a plan
 * with one partition). The result is bitwise equal to pa_decode with a plan of
 * max_partitions == 1 for the same problem. Context-0 rows are written as 0.
 *
 * Suited to batches with many short sequences: a long sequence is one
 * workgroup's serial work here, where pa_plan would split it.
 *
 * Arguments, layouts and device-side guarantees are those of pa_decode; the
 * problem descriptor's max_partitions and task_budget are ignored. Validates
 * the problem and probes the device on every call (the probe is cached per
 * process), allocates nothing and does not synchronize.
 */
pa_status pa_decode_direct(const pa_problem* problem, const void* query, const void* key_cache,
                           const void* value_cache, const void* k_scale, const void* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, void* out, pa_stream_t stream);

/*
 * pa_decode_static -- pa_decode_direct's arguments, and a decode that
 * allocates nothing and needs no plan: for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Every sequence is split into the same number P of partitions of the tiles
 * max_context_len (capped by max_blocks_per_seq * page_size, and with a window
 * by the tiles its rows' windows can span) implies; partition p of a sequence
 * covers its tiles [p * T, (p + 1) * T) counted from its window's first tile
 * (the last partition also covers any tiles beyond), so device lengths may be
 * anything up to the table's reach. The partials go to a static device buffer
 * of PA_STATIC_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends), and the log-sum-exp merge kernel combines them; with P = 1
 * each task writes its rows directly, exactly as pa_decode_direct does.
 *
 *   max_partitions 0   P is chosen for about one round of resident
 *                      workgroups and lowered until the partials fit the buffer.
 *   max_partitions > 0 P = min(max_partitions, tiles); if its partials
 *                      (num_seqs * P * num_kv_heads * qlen * q_per_kv *
 *                      (head_dim + 2) * 4 bytes, plus alignment) exceed the
 *                      buffer, PA_ERR_UNSUPPORTED, before any device work.
 *
 * Every partial a call reads is written by the same call, so nothing needs
 * clearing between calls; the buffer keeps the last call's partials. All
 * calls on one GPU share the buffer: calls that overlap on a GPU (different
 * streams, or threads without ordering) race and give undefined output, so
 * keep them stream-ordered. Layouts, refusals and device-side guarantees are
 * pa_decode's; task_budget is ignored. Nothing is allocated or synchronized;
 * the first call on a device looks up the buffer's address there.
 */
#define PA_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

pa_status pa_decode_static(const pa_problem* problem, const void* query, const void* key_cache,
                           const void* value_cache, const void* k_scale, const void* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, void* out, pa_stream_t stream);

/*
 * pa_write_kv_mxfp4 -- the MXFP4 KV-cache write: quantize num_tokens new K and V
 * rows and store them in the paged MXFP4 caches that pa_decode reads (ROCm/aiter
 * PR #7056, "Summary": the MXFP4 pages come from a separate KV-write kernel, as
 * e2m1 data with one e8m0 scale per 32 elements along head_dim).
 *
 * Each 32-element block of a row is encoded with the OCP Microscaling v1.0
 * conversion: E = floor(log2 max|v|) - 2 (e2m1's largest exponent is 2), scale
 * byte E + 127, elements v / 2^E rounded to nearest even in e2m1 and saturated
 * to +-6; element 2k in the low nibble of byte k. E is clamped to [-126, 127], so
 * every finite block gets a scale byte in 1..254 (an all-zero block gets 1). A
 * block holding NaN or an infinity gets scale byte 0xFF (the e8m0 NaN) and zero
 * data.
 *
 *   key, value          bf16 [num_tokens][num_kv_heads][head_dim], contiguous,
 *                       16-byte aligned, device memory.
 *   slot_mapping        int32 [num_tokens], device: token n goes to page
 *                       slot / page_size, row slot % page_size of every KV head.
 *                       Slots outside [0, num_blocks * page_size) (e.g. -1 for
 *                       padding) write nothing. A slot may appear at most once
 *                       per call; with duplicates the row's content is unspecified.
 *   key_cache, value_cache   uint8 [num_blocks][num_kv_heads][page_size][head_dim / 2]
 *   key_scale, value_scale   uint8 [num_blocks][num_kv_heads][page_size][head_dim / 32]
 *                       device memory, caches and scale tables 16-byte aligned;
 *                       rows no token maps to are not touched.
 *
 * head_dim must be 64, 128 or 256 (pa_decode reads MXFP4 at 128), page_size >= 1,
 * num_blocks * page_size < 2^31 and num_tokens * num_kv_heads * head_dim < 2^34.
 * Enqueued on `stream`; nothing is allocated or synchronized. num_tokens == 0 is
 * a no-op.
 */
typedef struct pa_kv_write_problem {
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_blocks;
} pa_kv_write_problem;

pa_status pa_write_kv_mxfp4(const pa_kv_write_problem* problem, const void* key, const void* value,
                            const int32_t* slot_mapping, void* key_cache, void* value_cache, void* key_scale,
                            void* value_scale, pa_stream_t stream);

/*
 * pa_mqa_logits_mxfp4 -- the sparse indexer's scores over a paged MXFP4 index-K
 * cache (ROCm/aiter PR #5761, "Unify gfx950+gfx1250 MXFP4 paged MQA-logits":
 * per query row, scores over the positions of its own window of the sequence
 * row_to_batch names, one K head shared by all query heads, K read through that
 * sequence's block table, nothing written outside the window):
 *
 *   out[r * out_stride + t] = sum_h weights[r][h] * relu(qhat[r][h] . khat_b(t))
 *   for t in [max(local_starts[r], 0), min(local_ends[r], W * page_size, out_stride))
 *
 * with b = row_to_batch[r], khat_b(t) the K row at page block_tables[b][t / page_size],
 * slot t % page_size, qhat and khat MXFP4 values (e2m1 times the e8m0 scale of
 * their 32-element block), and relu(x) = (x < 0 ? 0 : x), which keeps a NaN. The
 * pages give the op's inputs and contract but not the formula; this is the
 * published sparse-indexer score. Rows with b outside [0, num_seqs), and empty
 * windows, write nothing; every other position of out keeps its content.
 *
 *   q             uint8 [num_rows][num_heads][head_dim / 2]  e2m1, element 2i low nibble
 *   q_scale       uint8 [num_rows][num_heads][head_dim / 32] e8m0
 *   weights       fp32  [num_rows][num_heads]
 *   k_cache       uint8 [num_blocks][page_size][head_dim / 2]
 *   k_scale       uint8 [num_blocks][page_size][head_dim / 32]
 *   block_tables  int32 [num_seqs][max_blocks_per_seq] (W)
 *   row_to_batch, local_starts, local_ends   int32 [num_rows]
 *   out           fp32  [num_rows][out_stride]
 * All device memory; q, weights and k_cache 16-byte aligned, the rest 4-byte.
 * head_dim must be 128, num_heads 16, 32, 64 or 128, page_size a multiple of 16.
 * Block-table entries are clamped into [0, num_blocks), so a bad table cannot
 * fault. The result is fp32; each score is a sum of num_heads weighted products,
 * rounded in fp32. A NaN score comes only from an e8m0 NaN scale byte (0xFF) in
 * the row's q or the position's K row, and such a score is NaN exactly as relu
 * keeps it; scores whose partial sums leave the fp32 range are not specified.
 * Enqueued on `stream`; nothing is allocated or synchronized.
 */
typedef struct pa_mqa_problem {
    int32_t num_rows;
    int32_t num_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_blocks;
    int32_t num_seqs;
    int32_t max_blocks_per_seq;
    int32_t out_stride;
} pa_mqa_problem;

pa_status pa_mqa_logits_mxfp4(const pa_mqa_problem* problem, const void* q, const void* q_scale,
                              const float* weights, const void* k_cache, const void* k_scale,
                              const int32_t* block_tables, const int32_t* row_to_batch,
                              const int32_t* local_starts, const int32_t* local_ends, float* out,
                              pa_stream_t stream);

/* Release a plan and its device workspace (NULL-safe). Synchronizes the device. */
void pa_plan_destroy(pa_plan_t* plan);

/* Device bytes owned by the plan (task list + partition partials). */
size_t pa_plan_workspace_bytes(const pa_plan_t* plan);

/* Plan summary for logging and tests. */
typedef struct pa_plan_info {
    int32_t num_tasks;        /* workgroups of the tile kernel, one task each */
    int32_t max_parts;        /* largest partition count of any (sequence, KV head) */
    int32_t total_parts;      /* partitions that write partials ((sequence, KV head)s with > 1 partition) */
    int32_t tiles_per_task;   /* target tiles per task the planner chose */
    int32_t merge_needed;     /* 1 if pa_decode launches the merge kernel */
    int32_t num_cus;          /* compute units the plan was sized for */
    int32_t slots;            /* tile workgroups resident at once (compute units x occupancy) */
} pa_plan_info;

pa_status pa_plan_get_info(const pa_plan_t* plan, pa_plan_info* info);

/*
 * Host-only planner, for inspection and tests (no device needed): plans as
 * pa_plan would for a device with num_cus compute units holding
 * blocks_per_cu tile workgroups each. Fills
 * tasks_out (int32 x 4 per task, longest first: b, kvh | part << 16,
 * tile_begin, tile_end) and seq_parts_out (int32 x 2 per (sequence, KV head),
 * at b * num_kv_heads + kvh: partitions, first partial unit or -1). Capacities
 * are in records; *num_tasks receives the count (when the capacity is too
 * small, nothing is written and PA_ERR_INVALID_ARG returns with *num_tasks set
 * to the required capacity). Any output may be NULL.
 */
pa_status pa_plan_host(const pa_problem* problem, const int32_t* host_context_lens, int32_t num_cus,
                       int32_t blocks_per_cu, int32_t* tasks_out, int32_t task_capacity, int32_t* num_tasks,
                       int32_t* seq_parts_out, pa_plan_info* info);

/*
 * Per-kernel timing for measurement. With timing on, pa_decode records HIP
 * events around each kernel it launches on the caller's stream (no
 * allocation: the events are created here). pa_plan_read_timing waits for the
 * recorded events, returns the summed durations in milliseconds and the number
 * of calls, and clears the record. Not thread-safe; intended for benchmarks.
 */
pa_status pa_plan_set_timing(pa_plan_t* plan, int32_t enable, int32_t max_calls);
pa_status pa_plan_read_timing(pa_plan_t* plan, double* tile_ms, double* merge_ms, int32_t* calls);

/* Thread-local message of the last failure on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
