// Host side of libpa: C ABI, validation, device probe, planner and launches.
//
// The planner follows the work decomposition of ROCm/aiter PR #7092 ("Root
// cause": a sequence has ceil(context_len / 256) tiles and no others) and the
// partitioned plan of PR #7056 ("Microbench", "Bandwidth": tile kernel plus a
// partition reducer, a default task budget of about two workgroups per
// compute unit). Tiles of one (sequence, KV head) are cut into contiguous
// partitions; each partition is one workgroup; tasks are launched longest
// first so the ragged tail of the grid is short.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <functional>
#include <numeric>
#include <queue>
#include <string>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_err;

pa_status fail(pa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

struct DeviceInfo {
    int device = -1;
    int num_cus = 0;
    bool gfx950 = false;
    std::string arch;
};

std::mutex g_dev_mu;
std::vector<DeviceInfo> g_devs;  // probed once per device per process

pa_status probe_device(DeviceInfo* out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lk(g_dev_mu);
    for (const DeviceInfo& d : g_devs)
        if (d.device == dev) {
            *out = d;
            return PA_OK;
        }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    DeviceInfo d;
    d.device = dev;
    d.num_cus = prop.multiProcessorCount;
    d.arch = prop.gcnArchName;
    d.gfx950 = d.arch.compare(0, 6, "gfx950") == 0;
    g_devs.push_back(d);
    *out = d;
    return PA_OK;
}

int rows_of(const pa_problem& p) { return p.qlen * p.q_per_kv; }

pa_status validate(const pa_problem* p) {
    if (!p) return fail(PA_ERR_INVALID_ARG, "problem is NULL");
    if (p->num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs < 0");
    if (p->qlen < 1 || p->num_kv_heads < 1 || p->q_per_kv < 1)
        return fail(PA_ERR_INVALID_ARG, "qlen, num_kv_heads and q_per_kv must be >= 1");
    if (p->num_kv_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "num_kv_heads > 65535");
    if (p->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1 (block 0 always exists)");
    if (p->max_blocks_per_seq < 0 || p->max_context_len < 0)
        return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq and max_context_len must be >= 0");
    if (p->kv_dtype < PA_KV_BF16 || p->kv_dtype > PA_KV_MXFP4) return fail(PA_ERR_INVALID_ARG, "unknown kv_dtype");
    if (p->scale_mode < PA_SCALE_NONE || p->scale_mode > PA_SCALE_PER_TOKEN)
        return fail(PA_ERR_INVALID_ARG, "unknown scale_mode");
    if (p->v_layout != PA_V_PLAIN && p->v_layout != PA_V_TRANSPOSED) return fail(PA_ERR_INVALID_ARG, "unknown v_layout");
    if (p->q_dtype != PA_Q_BF16 && p->q_dtype != PA_Q_FP8_E4M3) return fail(PA_ERR_INVALID_ARG, "unknown q_dtype");
    if (!(std::isfinite(p->softmax_scale))) return fail(PA_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (p->mxfp4_scaled_qk != 0 && p->mxfp4_scaled_qk != 1)
        return fail(PA_ERR_INVALID_ARG, "mxfp4_scaled_qk must be 0 or 1");
    if (p->causal != 0 && p->causal != 1) return fail(PA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (p->window < 0) return fail(PA_ERR_INVALID_ARG, "window must be >= 0");
    if (p->max_partitions < 0 || p->task_budget < 0)
        return fail(PA_ERR_INVALID_ARG, "max_partitions and task_budget must be >= 0");
    if (p->max_partitions > 64) return fail(PA_ERR_UNSUPPORTED, "max_partitions %d (supported: <= 64)", p->max_partitions);
    if (p->page_size != 16 && p->page_size != 64 && p->page_size != 128)
        return fail(PA_ERR_UNSUPPORTED, "page_size %d (supported: 16, 64, 128)", p->page_size);
    if (p->head_dim != 128 && p->head_dim != 256)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 128, 256)", p->head_dim);
    if (rows_of(*p) > 64)
        return fail(PA_ERR_UNSUPPORTED, "qlen * q_per_kv = %d query rows per KV head (supported: <= 64)", rows_of(*p));
    // 33-64 rows take four 16-row N tiles, whose fp32 accumulators alone need
    // head_dim / 16 * 4 * 4 registers per lane: 128 at head_dim 128, 256 at 256,
    // which leaves no room for K, the scores and the softmax state
    if (rows_of(*p) > 32 && p->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED,
                    "qlen * q_per_kv = %d query rows per KV head with head_dim %d (more than 32 rows: head_dim 128 only)",
                    rows_of(*p), p->head_dim);
    if ((long long)p->max_blocks_per_seq * p->page_size > (1LL << 30))
        return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq * page_size exceeds 2^30 tokens");
    if (p->kv_dtype == PA_KV_BF16) {
        if (p->scale_mode != PA_SCALE_NONE) return fail(PA_ERR_INVALID_ARG, "bf16 KV takes no scales (scale_mode NONE)");
        if (p->q_dtype != PA_Q_BF16) return fail(PA_ERR_UNSUPPORTED, "bf16 KV needs a bf16 query");
    } else if (p->kv_dtype == PA_KV_FP8_E4M3) {
        if (p->scale_mode == PA_SCALE_NONE)
            return fail(PA_ERR_INVALID_ARG, "fp8 KV needs per-tensor or per-token scales");
        if (p->q_dtype != PA_Q_BF16) return fail(PA_ERR_UNSUPPORTED, "fp8 KV needs a bf16 query");
    } else {
        // MXFP4 (PR #7056, "Summary": head_dim 128, block size 128, query_length 1,
        // up to 16 query heads per KV head; no transposed V)
        if (p->scale_mode != PA_SCALE_NONE)
            return fail(PA_ERR_INVALID_ARG, "MXFP4 carries its own e8m0 block scales (scale_mode NONE)");
        if (p->page_size != 128) return fail(PA_ERR_UNSUPPORTED, "MXFP4 needs page_size 128");
        if (p->head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "MXFP4 needs head_dim 128");
        if (p->qlen != 1) return fail(PA_ERR_UNSUPPORTED, "MXFP4 needs qlen 1");
        if (p->q_per_kv > 16) return fail(PA_ERR_UNSUPPORTED, "MXFP4 supports up to 16 query heads per KV head");
        if (p->v_layout != PA_V_PLAIN) return fail(PA_ERR_UNSUPPORTED, "MXFP4 needs the plain V layout");
        if (p->window != 0) return fail(PA_ERR_UNSUPPORTED, "MXFP4 has no sliding window");
    }
    return PA_OK;
}

pa::KernelKey key_of(const pa_problem& p) {
    pa::KernelKey k;
    k.kv = p.kv_dtype == PA_KV_BF16 ? pa::KV_BF16 : (p.kv_dtype == PA_KV_FP8_E4M3 ? pa::KV_FP8 : pa::KV_MXFP4);
    k.scale = p.scale_mode == PA_SCALE_NONE ? pa::SC_NONE : (p.scale_mode == PA_SCALE_PER_TENSOR ? pa::SC_TENSOR : pa::SC_TOKEN);
    k.vt = p.v_layout == PA_V_TRANSPOSED ? 1 : 0;
    k.head_dim = p.head_dim;
    k.page = p.page_size;
    k.ntiles_n = rows_of(p) <= 16 ? 1 : (rows_of(p) <= 32 ? 2 : 4);
    k.q_fp8 = p.q_dtype == PA_Q_FP8_E4M3 ? 1 : 0;
    k.mx_scaled = (p.kv_dtype == PA_KV_MXFP4 && p.mxfp4_scaled_qk) ? 1 : 0;
    // 1: a sliding window; 2: causal rows without one (qlen 1: causal is the
    // plain decode), served by the windowed instances where no causal-only
    // instance is compiled
    k.win = p.window > 0 ? 1 : ((p.causal && p.qlen > 1) ? 2 : 0);
    if (k.win == 2 && !pa::have_tile_kernel(k)) k.win = 1;
    return k;
}

struct Plan {
    std::vector<int32_t> tasks;      // 4 per task, one task per workgroup
    std::vector<int32_t> seq_parts;  // 2 per (sequence, KV head): partitions, first partial unit or -1
    pa_plan_info info{};
};

// Task sizes (tiles) of every (sequence, KV head) when each sequence is cut
// into partitions of about `tpt` tiles (at most max_parts, at least one).
static void partition_counts(const std::vector<int>& tiles, int tpt, int max_parts, std::vector<int>* parts) {
    parts->resize(tiles.size());
    for (size_t b = 0; b < tiles.size(); ++b)
        (*parts)[b] = std::max(1, std::min(max_parts, (tiles[b] + tpt - 1) / tpt));
}

// Estimated completion time (seconds) of a task set launched longest first on
// `slots` workgroup slots. Running workgroups share the memory system: each
// streams at min(kWgBytesPerS, kHbmBytesPerS / running). A workgroup on its own
// is bound by its latency, about one 256-token tile per kTileS (its four waves
// keep one slice of K or V in flight each), and by what one compute unit
// streams, about 25 GB/s (6.4 TB/s over 256 CUs): a bf16 tile of 128 KB takes
// 5.2 us at that rate, an fp8 transposed-V tile of 64 KB 2.8 us, an MXFP4 tile
// of 35 KB 2 us on its own (measured on the workloads of the benchmark). A task
// costs its KV bytes plus a fixed start/epilogue time; any split sequence adds
// the merge launch.
static double plan_cost(const std::vector<int>& tiles, const std::vector<int>& parts, int H, int slots,
                        double tile_bytes, double partial_bytes, bool half_rows, long* ntasks_out) {
    // sustained HBM read rate of the tile kernel; transposed V rows are read
    // half by one wave and half by the next, which streams slower (5.3-5.8
    // TB/s for that pattern against 6.1-6.9 for whole rows, measured)
    const double kHbmBytesPerS = half_rows ? 5.9e12 : 6.4e12;
    const double kCuBytesPerS = 2.5e10;   // one compute unit
    const double kTileS = 2.8e-6;         // one workgroup, one tile, latency-bound
    const double kWgBytesPerS = std::min(kCuBytesPerS, tile_bytes / kTileS);
    const double kTaskS = 1.0e-6;         // start + four-wave merge + store of one task
    const double kMergeS = 8.0e-6;        // merge kernel (about 4.5 us) and the gap between the launches
    std::vector<double> bytes;
    bool split = false;
    double merge_bytes = 0.0;
    for (size_t b = 0; b < tiles.size(); ++b) {
        const int P = parts[b];
        split |= P > 1;
        const double pb = P > 1 ? partial_bytes : 0.0;  // written by the task, read by the merge
        merge_bytes += pb * P * H;
        for (int q = 0; q < P; ++q) {
            const long sz = (long)(q + 1) * tiles[b] / P - (long)q * tiles[b] / P;
            for (int h = 0; h < H; ++h) bytes.push_back(sz * tile_bytes + pb + kTaskS * kWgBytesPerS);
        }
    }
    *ntasks_out = (long)bytes.size();
    std::sort(bytes.begin(), bytes.end(), std::greater<double>());
    // processor sharing: every running task advances at the same rate, so the
    // next to finish is the one with the least bytes left
    std::priority_queue<double, std::vector<double>, std::greater<double>> run;
    size_t next = 0;
    double consumed = 0.0, t = 0.0;
    while (next < bytes.size() && (int)run.size() < slots) run.push(bytes[next++]);
    while (!run.empty()) {
        const double rate = std::min(kWgBytesPerS, kHbmBytesPerS / (double)run.size());
        const double x = run.top() - consumed;
        t += x / rate;
        consumed = run.top();
        run.pop();
        if (next < bytes.size()) run.push(consumed + bytes[next++]);
    }
    return t + (split ? kMergeS + merge_bytes / kHbmBytesPerS : 0.0);
}

// KV bytes of one 256-token tile of one KV head.
static double tile_bytes_of(const pa_problem& p) {
    const double D = p.head_dim;
    double per_token;
    if (p.kv_dtype == PA_KV_BF16)
        per_token = 4 * D;
    else if (p.kv_dtype == PA_KV_FP8_E4M3)
        per_token = 2 * D + (p.scale_mode == PA_SCALE_PER_TOKEN ? 8 : 0);
    else
        per_token = 2 * (D / 2 + D / 32);
    return per_token * pa::kTileTokens;
}

// Cut every (sequence, KV head) into partitions of contiguous tiles.
pa_status build_plan(const pa_problem& p, const int32_t* lens, int num_cus, int blocks_per_cu, Plan* out) {
    const int B = p.num_seqs, H = p.num_kv_heads;
    const int max_parts = p.max_partitions > 0 ? p.max_partitions : 64;
    const int slots = std::max(1, num_cus * std::max(1, blocks_per_cu));
    const long cap_tokens = (long)p.max_blocks_per_seq * p.page_size;
    std::vector<int> tiles(B), first(B, 0);  // tiles to read per sequence, from tile first[b] on
    for (int b = 0; b < B; ++b) {
        long L = lens ? lens[b] : p.max_context_len;
        if (lens) {
            if (L < 0) return fail(PA_ERR_INVALID_ARG, "context_lens[%d] = %ld < 0", b, L);
            if (L > cap_tokens)
                return fail(PA_ERR_INVALID_ARG, "context_lens[%d] = %ld exceeds max_blocks_per_seq * page_size = %ld", b,
                            L, cap_tokens);
            if (L > p.max_context_len)
                return fail(PA_ERR_INVALID_ARG, "context_lens[%d] = %ld exceeds max_context_len = %d", b, L,
                            p.max_context_len);
        } else {
            L = std::min(L, cap_tokens);
        }
        tiles[b] = (int)((L + pa::kTileTokens - 1) / pa::kTileTokens);
        if (lens && p.window > 0) {
            // tiles before the first query token's window are never read
            const long e0 = p.causal ? L - p.qlen + 1 : L;
            const long s0 = std::max(0L, e0 - p.window);
            first[b] = (int)std::min<long>(s0 / pa::kTileTokens, tiles[b]);
            tiles[b] -= first[b];
        }
    }
    long work = 0;
    int tmax = 0;
    for (int b = 0; b < B; ++b) {
        work += (long)tiles[b] * H;
        tmax = std::max(tmax, tiles[b]);
    }
    int tpt;
    std::vector<int> parts;
    if (p.task_budget > 0) {
        tpt = (int)std::max<long>(1, (work + p.task_budget - 1) / p.task_budget);
        partition_counts(tiles, tpt, max_parts, &parts);
    } else {
        // pick the tiles-per-task target with the lowest estimated completion time
        tpt = std::max(1, tmax);
        partition_counts(tiles, tpt, max_parts, &parts);
        long nt = 0;
        const double tb = tile_bytes_of(p);
        const double pbytes = (double)rows_of(p) * (p.head_dim + 2) * 4.0;  // one task's partial (O, m, l)
        const bool half_rows = p.v_layout == PA_V_TRANSPOSED;
        double best = plan_cost(tiles, parts, H, slots, tb, pbytes, half_rows, &nt);
        std::vector<int> cand;
        for (int t = tmax - 1; t >= 1; --t) {
            partition_counts(tiles, t, max_parts, &cand);
            if (cand == parts) continue;
            double c = plan_cost(tiles, cand, H, slots, tb, pbytes, half_rows, &nt);
            if (nt > 8L * slots) break;
            if (c < best * 0.995) {
                best = c;
                tpt = t;
                parts = cand;
            }
        }
    }
    out->tasks.clear();
    out->seq_parts.assign(2 * (size_t)B * H, 0);
    int units = 0, maxp = 0;
    {
        for (int b = 0; b < B; ++b) {
            const int P = parts[b];
            maxp = std::max(maxp, P);
            for (int kvh = 0; kvh < H; ++kvh) {
                const size_t pr = (size_t)b * H + kvh;
                out->seq_parts[2 * pr] = P;
                out->seq_parts[2 * pr + 1] = P > 1 ? units : -1;
                if (P > 1) units += P;
                for (int part = 0; part < P; ++part) {
                    const int t0 = (int)((long)part * tiles[b] / P), t1 = (int)((long)(part + 1) * tiles[b] / P);
                    out->tasks.insert(out->tasks.end(), {b, kvh | (part << 16), first[b] + t0, first[b] + t1});
                }
            }
        }
        // longest first; ties in (sequence, partition, head) order, so that the
        // KV heads of one partition are neighbours
        const size_t n = out->tasks.size() / 4;
        const auto& t = out->tasks;
        std::vector<size_t> order(n);
        std::iota(order.begin(), order.end(), 0);
        std::sort(order.begin(), order.end(), [&](size_t x, size_t y) {
            const int32_t sx = t[4 * x + 3] - t[4 * x + 2], sy = t[4 * y + 3] - t[4 * y + 2];
            if (sx != sy) return sx > sy;
            if (t[4 * x] != t[4 * y]) return t[4 * x] < t[4 * y];
            const int32_t px = t[4 * x + 1] >> 16, py = t[4 * y + 1] >> 16;
            if (px != py) return px < py;
            return (t[4 * x + 1] & 0xFFFF) < (t[4 * y + 1] & 0xFFFF);
        });
        // Per-token scales of 16-token pages: the scale rows of KV heads 2k and
        // 2k + 1 of a page share one 128-byte line ([block][head][16] fp32). The
        // two heads' tasks of a partition (neighbours above, same length) are
        // placed 8 launch slots apart, which the hardware dispatches to the same
        // XCD, so the line comes from HBM once and the second read finds it in
        // that XCD's L2. Within each run of 16 tasks, slot 16m + 8s + x takes
        // task 2 (8m + x) + s; the runs stay in longest-first order.
        const bool pair_heads = p.scale_mode == PA_SCALE_PER_TOKEN && p.page_size * 4 < 128 && H % 2 == 0;
        std::vector<size_t> slot_task(n);
        for (size_t i = 0; i < n; ++i) slot_task[i] = i;
        if (pair_heads)
            for (size_t i = 0; i < n / 16 * 16; ++i) {
                const size_t m = i / 16, s8 = (i / 8) % 2, x = i % 8;
                slot_task[i] = 2 * (8 * m + x) + s8;
            }
        std::vector<int32_t> sorted(out->tasks.size());
        for (size_t i = 0; i < n; ++i)
            for (int k = 0; k < 4; ++k) sorted[4 * i + k] = t[4 * order[slot_task[i]] + k];
        out->tasks.swap(sorted);
    }
    const size_t n = out->tasks.size() / 4;
    if (n > 0x7FFFFFFF / 4) return fail(PA_ERR_UNSUPPORTED, "too many tasks");
    out->info.num_tasks = (int32_t)n;
    out->info.max_parts = maxp;
    out->info.total_parts = units;
    out->info.tiles_per_task = tpt;
    out->info.merge_needed = units > 0 ? 1 : 0;
    out->info.num_cus = num_cus;
    out->info.slots = slots;
    return PA_OK;
}

}  // namespace

struct pa_plan {
    pa_problem prob{};
    pa::KernelKey key{};
    pa_plan_info info{};
    int device = -1;
    int32_t* d_tasks = nullptr;
    int32_t* d_seq_parts = nullptr;
    float* d_part_ml = nullptr;
    float* d_part_o = nullptr;
    size_t ws_bytes = 0;
    // timing
    bool timing = false;
    int max_calls = 0;
    mutable int ncalls = 0;
    std::vector<hipEvent_t> ev;  // 3 per call
};

extern "C" {

const char* pa_last_error(void) { return g_err.c_str(); }

const char* pa_version(void) { return "pa_decode gfx950 0.1"; }

pa_status pa_plan_host(const pa_problem* problem, const int32_t* host_context_lens, int32_t num_cus,
                       int32_t blocks_per_cu, int32_t* tasks_out, int32_t task_capacity, int32_t* num_tasks,
                       int32_t* seq_parts_out, pa_plan_info* info) {
    pa_status st = validate(problem);
    if (st != PA_OK) return st;
    if (num_cus < 1 || blocks_per_cu < 1) return fail(PA_ERR_INVALID_ARG, "num_cus and blocks_per_cu must be >= 1");
    Plan plan;
    st = build_plan(*problem, host_context_lens, num_cus, blocks_per_cu, &plan);
    if (st != PA_OK) return st;
    if (num_tasks) *num_tasks = plan.info.num_tasks;
    if (info) *info = plan.info;
    if (tasks_out) {
        if (task_capacity < plan.info.num_tasks) return fail(PA_ERR_INVALID_ARG, "task capacity too small");
        std::memcpy(tasks_out, plan.tasks.data(), plan.tasks.size() * sizeof(int32_t));
    }
    if (seq_parts_out) std::memcpy(seq_parts_out, plan.seq_parts.data(), plan.seq_parts.size() * sizeof(int32_t));
    return PA_OK;
}

pa_status pa_plan(const pa_problem* problem, const int32_t* host_context_lens, pa_stream_t stream,
                  pa_plan_t** plan_out) {
    if (!plan_out) return fail(PA_ERR_INVALID_ARG, "plan_out is NULL");
    *plan_out = nullptr;
    pa_status st = validate(problem);
    if (st != PA_OK) return st;
    DeviceInfo dev;
    st = probe_device(&dev);
    if (st != PA_OK) return st;
    if (!dev.gfx950) return fail(PA_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev.device, dev.arch.c_str());
    const pa::KernelKey key = key_of(*problem);
    if (!pa::have_tile_kernel(key)) return fail(PA_ERR_UNSUPPORTED, "no kernel instance for this problem");
    Plan plan;
    st = build_plan(*problem, host_context_lens, dev.num_cus, pa::tile_blocks_per_cu(key), &plan);
    if (st != PA_OK) return st;

    pa_plan_t* p = new (std::nothrow) pa_plan_t();
    if (!p) return fail(PA_ERR_OOM, "host allocation failed");
    p->prob = *problem;
    p->key = key;
    p->info = plan.info;
    p->device = dev.device;
    const size_t rows = (size_t)rows_of(*problem);
    const size_t nslots = (size_t)plan.info.total_parts * rows;
    const size_t tasks_b = std::max<size_t>(16, plan.tasks.size() * sizeof(int32_t));
    const size_t seq_b = std::max<size_t>(16, plan.seq_parts.size() * sizeof(int32_t));
    const size_t ml_b = std::max<size_t>(16, nslots * 2 * sizeof(float));
    const size_t o_b = std::max<size_t>(16, nslots * problem->head_dim * sizeof(float));
    hipError_t e;
    if ((e = hipMalloc(&p->d_tasks, tasks_b)) != hipSuccess || (e = hipMalloc(&p->d_seq_parts, seq_b)) != hipSuccess ||
        (e = hipMalloc(&p->d_part_ml, ml_b)) != hipSuccess || (e = hipMalloc(&p->d_part_o, o_b)) != hipSuccess) {
        pa_plan_destroy(p);
        return fail(PA_ERR_OOM, "workspace allocation failed: %s", hipGetErrorString(e));
    }
    p->ws_bytes = tasks_b + seq_b + ml_b + o_b;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!plan.tasks.empty() &&
        (e = hipMemcpyAsync(p->d_tasks, plan.tasks.data(), plan.tasks.size() * sizeof(int32_t), hipMemcpyHostToDevice, s)) !=
            hipSuccess) {
        pa_plan_destroy(p);
        return fail(PA_ERR_HIP, "task upload failed: %s", hipGetErrorString(e));
    }
    if (!plan.seq_parts.empty() &&
        (e = hipMemcpyAsync(p->d_seq_parts, plan.seq_parts.data(), plan.seq_parts.size() * sizeof(int32_t),
                            hipMemcpyHostToDevice, s)) != hipSuccess) {
        pa_plan_destroy(p);
        return fail(PA_ERR_HIP, "partition table upload failed: %s", hipGetErrorString(e));
    }
    // the host vectors die with this call: make the uploads complete first
    if ((e = hipStreamSynchronize(s)) != hipSuccess) {
        pa_plan_destroy(p);
        return fail(PA_ERR_HIP, "plan upload sync failed: %s", hipGetErrorString(e));
    }
    if (std::getenv("PA_LOG"))
        std::fprintf(stderr, "[pa] plan: %d tasks on %d slots, %d tiles/task target, max %d partitions, %d partial units, %zu B workspace\n",
                     plan.info.num_tasks, plan.info.slots, plan.info.tiles_per_task, plan.info.max_parts,
                     plan.info.total_parts, p->ws_bytes);
    *plan_out = p;
    return PA_OK;
}

void pa_plan_destroy(pa_plan_t* p) {
    if (!p) return;
    if (p->d_tasks || p->d_seq_parts || p->d_part_ml || p->d_part_o || !p->ev.empty()) (void)hipDeviceSynchronize();
    if (p->d_tasks) (void)hipFree(p->d_tasks);
    if (p->d_seq_parts) (void)hipFree(p->d_seq_parts);
    if (p->d_part_ml) (void)hipFree(p->d_part_ml);
    if (p->d_part_o) (void)hipFree(p->d_part_o);
    for (hipEvent_t e : p->ev) (void)hipEventDestroy(e);
    delete p;
}

size_t pa_plan_workspace_bytes(const pa_plan_t* p) { return p ? p->ws_bytes : 0; }

pa_status pa_plan_get_info(const pa_plan_t* p, pa_plan_info* info) {
    if (!p || !info) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    *info = p->info;
    return PA_OK;
}

static bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

// Pointer checks shared by the planned and the plan-free decode.
static pa_status check_pointers(const pa_problem& p, const void* query, const void* key_cache,
                                const void* value_cache, const void* k_scale, const void* v_scale,
                                const int32_t* block_tables, const int32_t* context_lens, const void* out) {
    if (!query || !key_cache || !value_cache || !block_tables || !context_lens || !out)
        return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
    if (misaligned(query) || misaligned(key_cache) || misaligned(value_cache) || misaligned(out))
        return fail(PA_ERR_INVALID_ARG, "query, caches and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return fail(PA_ERR_INVALID_ARG, "block_tables and context_lens must be 4-byte aligned");
    const bool need_scales = p.kv_dtype == PA_KV_MXFP4 || p.scale_mode != PA_SCALE_NONE;
    if (need_scales && (!k_scale || !v_scale)) return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale are required");
    if (need_scales && (misaligned(k_scale) || misaligned(v_scale)) &&
        !(p.scale_mode == PA_SCALE_PER_TENSOR && !((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3u)))
        return fail(PA_ERR_INVALID_ARG, "scale tables must be 16-byte aligned (per-tensor scales: 4-byte)");
    return PA_OK;
}

pa_status pa_decode(const pa_plan_t* plan, const void* query, const void* key_cache, const void* value_cache,
                    const void* k_scale, const void* v_scale, const int32_t* block_tables,
                    const int32_t* context_lens, void* out, pa_stream_t stream) {
    if (!plan) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
    const pa_problem& p = plan->prob;
    if (p.num_seqs == 0) return PA_OK;
    pa_status st = check_pointers(p, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, out);
    if (st != PA_OK) return st;
    hipError_t e = hipSetDevice(plan->device);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipSetDevice failed: %s", hipGetErrorString(e));

    pa::TileArgs a{};
    a.q = query;
    a.k = key_cache;
    a.v = value_cache;
    a.ks = k_scale;
    a.vs = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.tasks = plan->d_tasks;
    a.seq_parts = plan->d_seq_parts;
    a.part_ml = plan->d_part_ml;
    a.part_o = plan->d_part_o;
    a.num_seqs = p.num_seqs;
    a.qlen = p.qlen;
    a.num_kv_heads = p.num_kv_heads;
    a.q_per_kv = p.q_per_kv;
    a.rows = rows_of(p);
    a.max_blocks = p.max_blocks_per_seq;
    a.num_blocks = p.num_blocks;
    const double sm = p.softmax_scale != 0.f ? (double)p.softmax_scale : 1.0 / std::sqrt((double)p.head_dim);
    a.scale_log2 = (float)(sm * 1.4426950408889634);
    a.causal = p.causal;
    a.window = p.window;
    a.plan_free = 0;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    pa_plan_t* mp = const_cast<pa_plan_t*>(plan);
    const bool rec = mp->timing && mp->ncalls < mp->max_calls;
    hipEvent_t* ev = rec ? &mp->ev[3 * (size_t)mp->ncalls] : nullptr;
    if (rec && (e = hipEventRecord(ev[0], s)) != hipSuccess) return fail(PA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
    e = pa::launch_tile(plan->key, a, plan->info.num_tasks, s);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "tile kernel launch failed: %s", hipGetErrorString(e));
    if (rec && (e = hipEventRecord(ev[1], s)) != hipSuccess) return fail(PA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
    if (plan->info.merge_needed) {
        e = pa::launch_merge(a, p.head_dim, s);
        if (e != hipSuccess) return fail(PA_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString(e));
    }
    if (rec) {
        if ((e = hipEventRecord(ev[2], s)) != hipSuccess) return fail(PA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
        mp->ncalls++;
    }
    return PA_OK;
}

pa_status pa_decode_direct(const pa_problem* problem, const void* query, const void* key_cache,
                           const void* value_cache, const void* k_scale, const void* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, void* out, pa_stream_t stream) {
    pa_status st = validate(problem);
    if (st != PA_OK) return st;
    const pa_problem& p = *problem;
    if (p.num_seqs == 0) return PA_OK;
    if ((long)p.num_seqs * p.num_kv_heads > 0x7FFFFFFFL)
        return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_kv_heads exceeds the grid");
    st = check_pointers(p, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, out);
    if (st != PA_OK) return st;
    DeviceInfo dev;
    st = probe_device(&dev);
    if (st != PA_OK) return st;
    if (!dev.gfx950) return fail(PA_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev.device, dev.arch.c_str());
    const pa::KernelKey key = key_of(p);
    if (!pa::have_tile_kernel(key)) return fail(PA_ERR_UNSUPPORTED, "no kernel instance for this problem");
    hipError_t e = hipSetDevice(dev.device);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipSetDevice failed: %s", hipGetErrorString(e));

    pa::TileArgs a{};
    a.q = query;
    a.k = key_cache;
    a.v = value_cache;
    a.ks = k_scale;
    a.vs = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.tasks = nullptr;
    a.seq_parts = nullptr;
    a.part_ml = nullptr;
    a.part_o = nullptr;
    a.num_seqs = p.num_seqs;
    a.qlen = p.qlen;
    a.num_kv_heads = p.num_kv_heads;
    a.q_per_kv = p.q_per_kv;
    a.rows = rows_of(p);
    a.max_blocks = p.max_blocks_per_seq;
    a.num_blocks = p.num_blocks;
    const double sm = p.softmax_scale != 0.f ? (double)p.softmax_scale : 1.0 / std::sqrt((double)p.head_dim);
    a.scale_log2 = (float)(sm * 1.4426950408889634);
    a.causal = p.causal;
    a.window = p.window;
    a.plan_free = 1;
    a.uniform_parts = 1;
    e = pa::launch_tile(key, a, p.num_seqs * p.num_kv_heads, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "tile kernel launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

}  // extern "C"

// ------------------------------------------------------ allocation-free decode
//
// pa_decode_static keeps its partition partials in this array: one copy per
// device, loaded with the library's code object and held until the process
// ends. Host code never passes the array's name to a kernel or a copy (on the
// host it is a stand-in, not a device address); the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static constexpr size_t kStaticScratchBytes = PA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device `dev`.
pa_status static_scratch(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return PA_OK;
}

// Partial bytes of P partitions per sequence: (m, l) of every slot row, then
// O, 256-byte aligned.
size_t static_partial_bytes(const pa_problem& p, long P, size_t* o_off) {
    const size_t n = (size_t)p.num_seqs * (size_t)P * (size_t)p.num_kv_heads * (size_t)rows_of(p);
    const size_t ml = (n * 2 * sizeof(float) + 255) & ~size_t(255);
    *o_off = ml;
    return ml + n * (size_t)p.head_dim * sizeof(float);
}

// Tiles a sequence can span: the table's reach and max_context_len, and with a
// window the tiles its rows' windows cover (at most W + qlen - 1 tokens).
int static_tiles(const pa_problem& p) {
    long reach = std::min<long>(p.max_context_len, (long)p.max_blocks_per_seq * p.page_size);
    long tiles = (reach + pa::kTileTokens - 1) / pa::kTileTokens;
    if (p.window > 0)
        tiles = std::min<long>(tiles, ((long)p.window + p.qlen - 1 + pa::kTileTokens - 1) / pa::kTileTokens + 1);
    return (int)std::max<long>(1, tiles);
}

}  // namespace

extern "C" {

pa_status pa_decode_static(const pa_problem* problem, const void* query, const void* key_cache,
                           const void* value_cache, const void* k_scale, const void* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, void* out, pa_stream_t stream) {
    pa_status st = validate(problem);
    if (st != PA_OK) return st;
    const pa_problem& p = *problem;
    if (p.num_seqs == 0) return PA_OK;
    st = check_pointers(p, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, out);
    if (st != PA_OK) return st;
    const int tiles = static_tiles(p);
    const long pairs = (long)p.num_seqs * p.num_kv_heads;
    size_t o_off = 0;
    int P = 0;
    if (p.max_partitions > 0) {
        P = std::min(p.max_partitions, tiles);
        const size_t need = static_partial_bytes(p, P, &o_off);
        if (P > 1 && need > kStaticScratchBytes)
            return fail(PA_ERR_UNSUPPORTED,
                        "%d partitions need %zu bytes of partials; the static scratch holds %zu (max_partitions 0 "
                        "picks a count that fits)",
                        P, need, kStaticScratchBytes);
    }
    DeviceInfo dev;
    st = probe_device(&dev);
    if (st != PA_OK) return st;
    if (!dev.gfx950) return fail(PA_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev.device, dev.arch.c_str());
    const pa::KernelKey key = key_of(p);
    if (!pa::have_tile_kernel(key)) return fail(PA_ERR_UNSUPPORTED, "no kernel instance for this problem");
    if (P == 0) {
        // about one round of resident workgroups, as many partials as fit
        const long slots = (long)dev.num_cus * pa::tile_blocks_per_cu(key);
        P = (int)std::min<long>(std::min(64, tiles), std::max<long>(1, (slots + pairs - 1) / pairs));
        while (P > 1 && static_partial_bytes(p, P, &o_off) > kStaticScratchBytes) --P;
    }
    const int part_tiles = (tiles + P - 1) / P;
    P = (tiles + part_tiles - 1) / part_tiles;  // no partition left without tiles
    if (pairs * P > 0x7FFFFFFFL) return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_kv_heads * partitions exceeds the grid");
    void* base = nullptr;
    if (P > 1) {
        st = static_scratch(dev.device, &base);
        if (st != PA_OK) return st;
        static_partial_bytes(p, P, &o_off);
    }

    pa::TileArgs a{};
    a.q = query;
    a.k = key_cache;
    a.v = value_cache;
    a.ks = k_scale;
    a.vs = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.part_ml = static_cast<float*>(base);
    a.part_o = base ? reinterpret_cast<float*>(static_cast<char*>(base) + o_off) : nullptr;
    a.num_seqs = p.num_seqs;
    a.qlen = p.qlen;
    a.num_kv_heads = p.num_kv_heads;
    a.q_per_kv = p.q_per_kv;
    a.rows = rows_of(p);
    a.max_blocks = p.max_blocks_per_seq;
    a.num_blocks = p.num_blocks;
    const double sm = p.softmax_scale != 0.f ? (double)p.softmax_scale : 1.0 / std::sqrt((double)p.head_dim);
    a.scale_log2 = (float)(sm * 1.4426950408889634);
    a.causal = p.causal;
    a.window = p.window;
    a.plan_free = 1;
    a.uniform_parts = P;
    a.part_tiles = part_tiles;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = pa::launch_tile(key, a, (int)(pairs * P), s);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "tile kernel launch failed: %s", hipGetErrorString(e));
    if (P > 1) {
        e = pa::launch_merge(a, p.head_dim, s);
        if (e != hipSuccess) return fail(PA_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString(e));
    }
    return PA_OK;
}

pa_status pa_write_kv_mxfp4(const pa_kv_write_problem* problem, const void* key, const void* value,
                            const int32_t* slot_mapping, void* key_cache, void* value_cache, void* key_scale,
                            void* value_scale, pa_stream_t stream) {
    if (!problem) return fail(PA_ERR_INVALID_ARG, "problem is NULL");
    const pa_kv_write_problem& p = *problem;
    if (p.num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
    if (p.num_kv_heads < 1 || p.page_size < 1 || p.num_blocks < 1)
        return fail(PA_ERR_INVALID_ARG, "num_kv_heads, page_size and num_blocks must be >= 1");
    if (p.head_dim != 64 && p.head_dim != 128 && p.head_dim != 256)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128, 256)", p.head_dim);
    if ((long long)p.num_blocks * p.page_size > 0x7FFFFFFFLL)
        return fail(PA_ERR_UNSUPPORTED, "num_blocks * page_size exceeds 2^31 - 1 slots");
    const long long elems = (long long)p.num_tokens * p.num_kv_heads * p.head_dim;
    if (elems >= (1LL << 34)) return fail(PA_ERR_UNSUPPORTED, "num_tokens * num_kv_heads * head_dim exceeds 2^34");
    if (p.num_tokens == 0) return PA_OK;
    if (!key || !value || !slot_mapping || !key_cache || !value_cache || !key_scale || !value_scale)
        return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
    if (misaligned(key) || misaligned(value) || misaligned(key_cache) || misaligned(value_cache) ||
        misaligned(key_scale) || misaligned(value_scale))
        return fail(PA_ERR_INVALID_ARG, "key, value, the caches and the scale tables must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(slot_mapping) & 3u)
        return fail(PA_ERR_INVALID_ARG, "slot_mapping must be 4-byte aligned");
    DeviceInfo dev;
    pa_status st = probe_device(&dev);
    if (st != PA_OK) return st;
    if (!dev.gfx950) return fail(PA_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev.device, dev.arch.c_str());
    pa::KvWriteArgs a{};
    a.key = static_cast<const uint16_t*>(key);
    a.value = static_cast<const uint16_t*>(value);
    a.slots = slot_mapping;
    a.key_cache = static_cast<uint8_t*>(key_cache);
    a.value_cache = static_cast<uint8_t*>(value_cache);
    a.key_scale = static_cast<uint8_t*>(key_scale);
    a.value_scale = static_cast<uint8_t*>(value_scale);
    const long long tpw = 64 / (p.head_dim / 8);  // tokens per wave
    a.wave_tasks = (uint32_t)(((long long)p.num_tokens + tpw - 1) / tpw * p.num_kv_heads);
    a.num_tokens = p.num_tokens;
    a.num_kv_heads = p.num_kv_heads;
    a.page_size = p.page_size;
    a.num_slots = p.num_blocks * p.page_size;
    const auto log2_exact = [](int32_t v) {
        return (v & (v - 1)) == 0 ? __builtin_ctz((unsigned)v) : -1;
    };
    a.heads_shift = log2_exact(p.num_kv_heads);
    a.page_shift = log2_exact(p.page_size);
    hipError_t e = pa::launch_kv_write_mxfp4(p.head_dim, a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "KV write launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

pa_status pa_mqa_logits_mxfp4(const pa_mqa_problem* problem, const void* q, const void* q_scale,
                              const float* weights, const void* k_cache, const void* k_scale,
                              const int32_t* block_tables, const int32_t* row_to_batch,
                              const int32_t* local_starts, const int32_t* local_ends, float* out,
                              pa_stream_t stream) {
    if (!problem) return fail(PA_ERR_INVALID_ARG, "problem is NULL");
    const pa_mqa_problem& p = *problem;
    if (p.num_rows < 0 || p.num_seqs < 0 || p.out_stride < 0)
        return fail(PA_ERR_INVALID_ARG, "num_rows, num_seqs and out_stride must be >= 0");
    if (p.num_blocks < 1 || p.max_blocks_per_seq < 1 || p.page_size < 1)
        return fail(PA_ERR_INVALID_ARG, "num_blocks, max_blocks_per_seq and page_size must be >= 1");
    if (p.head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 128)", p.head_dim);
    if (p.num_heads != 16 && p.num_heads != 32 && p.num_heads != 64 && p.num_heads != 128)
        return fail(PA_ERR_UNSUPPORTED, "num_heads %d (supported: 16, 32, 64, 128)", p.num_heads);
    if (p.page_size % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "page_size %d is not a multiple of 16", p.page_size);
    const long long reach = (long long)p.max_blocks_per_seq * p.page_size;
    if (reach > 0x7FFFFFFFLL - 2 * pa::kMqChunkPositions || (long long)p.num_blocks * p.page_size > 0x7FFFFFFFLL ||
        p.out_stride > 0x7FFFFFFF - 2 * pa::kMqChunkPositions)
        return fail(PA_ERR_UNSUPPORTED, "a table, pool or output row beyond 2^31 positions");
    const long long max_pos = std::min(reach, (long long)p.out_stride);
    const long long chunks = (max_pos + pa::kMqChunkPositions - 1) / pa::kMqChunkPositions;
    // one workgroup per (chunk, row), the grid rounded up to a multiple of 8
    if ((long long)p.num_rows * chunks > (1LL << 31) - 8)
        return fail(PA_ERR_UNSUPPORTED, "num_rows * ceil(positions / %d) exceeds 2^31 - 8", pa::kMqChunkPositions);
    if (p.num_rows == 0 || max_pos == 0) return PA_OK;
    if (!q || !q_scale || !weights || !k_cache || !k_scale || !block_tables || !row_to_batch || !local_starts ||
        !local_ends || !out)
        return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
    if (misaligned(q) || misaligned(weights) || misaligned(k_cache))
        return fail(PA_ERR_INVALID_ARG, "q, weights and k_cache must be 16-byte aligned");
    const uintptr_t ors = reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
                          reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(row_to_batch) |
                          reinterpret_cast<uintptr_t>(local_starts) | reinterpret_cast<uintptr_t>(local_ends) |
                          reinterpret_cast<uintptr_t>(out);
    if (ors & 3u) return fail(PA_ERR_INVALID_ARG, "scale tables, index arrays and out must be 4-byte aligned");
    DeviceInfo dev;
    pa_status st = probe_device(&dev);
    if (st != PA_OK) return st;
    if (!dev.gfx950) return fail(PA_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev.device, dev.arch.c_str());
    pa::MqaArgs a{};
    a.q = static_cast<const uint8_t*>(q);
    a.q_scale = static_cast<const uint8_t*>(q_scale);
    a.weights = weights;
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.k_scale = static_cast<const uint8_t*>(k_scale);
    a.block_tables = block_tables;
    a.row_to_batch = row_to_batch;
    a.local_starts = local_starts;
    a.local_ends = local_ends;
    a.out = out;
    a.items = (uint32_t)((long long)p.num_rows * chunks);
    a.num_rows = p.num_rows;
    a.page_size = p.page_size;
    a.page_shift = (p.page_size & (p.page_size - 1)) == 0 ? __builtin_ctz((unsigned)p.page_size) : -1;
    a.num_blocks = p.num_blocks;
    a.num_seqs = p.num_seqs;
    a.max_blocks_per_seq = p.max_blocks_per_seq;
    a.out_stride = p.out_stride;
    a.max_pos = (int32_t)max_pos;
    hipError_t e = pa::launch_mqa_logits_mxfp4(p.num_heads, a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "MQA-logits launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

pa_status pa_plan_set_timing(pa_plan_t* p, int32_t enable, int32_t max_calls) {
    if (!p) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
    if (enable && max_calls < 1) return fail(PA_ERR_INVALID_ARG, "max_calls must be >= 1");
    p->ncalls = 0;
    p->timing = enable != 0;
    if (!enable) return PA_OK;
    hipError_t e = hipSetDevice(p->device);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipSetDevice failed: %s", hipGetErrorString(e));
    while ((int)p->ev.size() < 3 * max_calls) {
        hipEvent_t ev;
        if ((e = hipEventCreate(&ev)) != hipSuccess) return fail(PA_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        p->ev.push_back(ev);
    }
    p->max_calls = max_calls;
    return PA_OK;
}

pa_status pa_plan_read_timing(pa_plan_t* p, double* tile_ms, double* merge_ms, int32_t* calls) {
    if (!p) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
    double t = 0, m = 0;
    for (int i = 0; i < p->ncalls; ++i) {
        hipEvent_t* ev = &p->ev[3 * (size_t)i];
        hipError_t e = hipEventSynchronize(ev[2]);
        if (e != hipSuccess) return fail(PA_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
        float a = 0, b = 0;
        if ((e = hipEventElapsedTime(&a, ev[0], ev[1])) != hipSuccess ||
            (e = hipEventElapsedTime(&b, ev[1], ev[2])) != hipSuccess)
            return fail(PA_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
        t += a;
        m += b;
    }
    if (tile_ms) *tile_ms = t;
    if (merge_ms) *merge_ms = m;
    if (calls) *calls = p->ncalls;
    p->ncalls = 0;
    return PA_OK;
}

}  // extern "C"
