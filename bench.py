"""Benchmark of the paged-attention decode hot path on one MI355X.

One step = one pa_decode call over each page-size variant of the bf16
workload (batch 64, context lengths uniform in [1000, 8192], 8 KV heads x 8
query heads each, head_dim 128, qlen 1, pages of 64 and of 128 tokens), with
every input resident in HBM. The metric is the nominal KV payload (K and V
bytes of the owned tokens) per second.

Prints one JSON line. Besides the contract keys it carries:
  roofline      the tile kernel's achieved GB/s (algorithmic bytes per launch /
                average launch duration) against the 8 TB/s HBM peak, and the
                HBM traffic from rocprofv3 counters when a counter summary of
                the current kernel source is committed under profiles/. The
                launch durations come from HIP events that the library records
                around each tile launch on the launch stream, during a second
                pass of the same timed steps: every event record costs a few
                microseconds of queue time, so the steps that give `value` and
                `ms_per_step` run without them;
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded sample of
                the same workload (the oracle is test infrastructure and is
                used here only for that baseline).

With --all, every workload is also timed one call at a time with the cold-cache
protocol: a 1 GiB buffer is read before each call (the last-level cache is
256 MB; a read leaves clean lines, where a write would leave dirty lines for
the decode to write back), and the median of the per-call event times is
reported, for pa_decode with its plan and for the plan-free pa_decode_direct.
With --all or --kv-write, the MXFP4 KV-cache write (pa_write_kv_mxfp4) is timed
the same way on its two workloads: the pages of the long MXFP4 decode workload
written in one call, and the one-token-per-sequence write of a decode step.
With --all or --mqa, the MXFP4 paged MQA logits (pa_mqa_logits_mxfp4) is timed
the same way on its decode and two-row workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "KV-read HBM GB/s and % of peak; µs per pa_decode call per config"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("pa_kernels.hip", "pa_kv_write.hip", "pa_mqa_logits.hip", "pa_internal.h"):
        with open(os.path.join(ROOT, "paged_attention_decode_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_tag: str):
    """HBM bytes per launch from a committed counter summary of this kernel source, else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source") != kernel_source_hash():
        return None
    ent = d.get("kernels", {}).get(kernel_tag)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def kernel_tag_of(spec) -> str:
    """The tile kernel's template arguments as rocprofv3 prints them."""
    kv = {"bf16": 0, "fp8": 1, "mxfp4": 2}[spec.kv_dtype]
    sc = {"none": 0, "tensor": 1, "token": 2}[spec.scale_mode]
    vt = 1 if spec.v_layout == "trans" else 0
    rows = spec.qlen * spec.q_per_kv
    nt = 1 if rows <= 16 else (2 if rows <= 32 else 4)
    qf = 1 if spec.q_dtype == "fp8" else 0
    # a window: 1; causal rows without one: 2 for fp8 per-token caches (the
    # causal-only instances), 1 otherwise
    win = 1 if spec.window > 0 else (0 if not (spec.causal and spec.qlen > 1) else (2 if sc == 2 and kv == 1 else 1))
    return "Cfg<%d, %d, %d, %d, %d, %d, %d, 0, %d>" % (kv, sc, vt, spec.head_dim, spec.page_size, nt, qf, win)


def write_traffic(fetch_csv: str, write_csv: str, out_json: str):
    """Turn two rocprofv3 --pmc runs of `bench.py --calibrate-copy` (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch) into HBM bytes per tile launch.

    Each counter is scaled by what it reads for the 1 GiB copy kernel of the same
    run (torch.neg: 1 GiB read, 1 GiB written). Writes `out_json` keyed to the
    current kernel source and prints a markdown summary."""
    import csv
    from collections import defaultdict

    from paged_attention_decode_token_amd import inputs as I

    def per_kernel(path, counter):
        vals = defaultdict(list)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    def by_grid(path, counter, key):
        """{grid size: [values]} of the dispatches of the one kernel matching key."""
        vals = defaultdict(list)
        names = set()
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and key in r["Kernel_Name"]:
                    names.add(r["Kernel_Name"])
                    vals[int(r["Grid_Size"])].append(float(r["Counter_Value"]))
        return vals if len(names) == 1 else {}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def one(vals, key):
        hits = [v for k, v in vals.items() if key in k]
        if len(hits) != 1:
            raise SystemExit("expected one kernel matching %r in the counter CSV, found %d" % (key, len(hits)))
        return hits[0]

    gib_kib = float(1 << 20)
    f_copy, w_copy = one(fetch, "neg_kernel"), one(write, "neg_kernel")
    f_factor, w_factor = gib_kib / (sum(f_copy) / len(f_copy)), gib_kib / (sum(w_copy) / len(w_copy))
    kernels = {}
    lines = ["| workload | tile kernel | dispatches | HBM read B/launch | HBM write B/launch | algorithmic B | read / algorithmic |",
             "|---|---|---|---|---|---|---|"]
    for spec in (I.BF16_P64, I.BF16_P128, I.FP8TOK_Q1, I.FP8TOK_Q4, I.FP8TOK_Q4_CAUSAL, I.FP8_TRANS, I.MXFP4_LONG_Q8,
                 I.MXFP4_LONG_QBF):
        tag = kernel_tag_of(spec)
        if spec.kv_dtype != "bf16" and not any(tag in k for k in fetch):
            continue  # rows other than bf16 only when the run included them (--all --workloads ...)
        fv, wv = one(fetch, tag), one(write, tag)
        rd = sum(fv) / len(fv) * 1024 * f_factor
        wr = sum(wv) / len(wv) * 1024 * w_factor
        alg = I.make_case(spec).kv_bytes()
        kernels[spec.name] = {"kernel": tag, "dispatches": len(fv), "hbm_read_bytes_per_launch": round(rd),
                              "hbm_write_bytes_per_launch": round(wr), "hbm_bytes_per_launch": round(rd + wr),
                              "algorithmic_bytes": alg}
        lines.append("| %s | %s | %d | %.4g | %.4g | %.4g | %.4f |" % (spec.name, tag, len(fv), rd, wr, alg, rd / alg))
    # the MXFP4 cache write, when the run included it (bench.py --kv-write):
    # its prefill-sized workload is the launch with the largest grid
    fg, wg = by_grid(fetch_csv, "FETCH_SIZE", "pa_kv_write_mxfp4_kernel"), by_grid(write_csv, "WRITE_SIZE",
                                                                                  "pa_kv_write_mxfp4_kernel")
    if fg and wg:
        grid = max(fg)
        fv, wv = fg[grid], wg[grid]
        rd = sum(fv) / len(fv) * 1024 * f_factor
        wr = sum(wv) / len(wv) * 1024 * w_factor
        spec = I.MXFP4_WRITE_FILL
        alg = I.write_bytes(spec)
        alg_rd = I.write_bytes(spec, "read")
        kernels[spec.name] = {"kernel": "pa_kv_write_mxfp4_kernel<%d>" % spec.head_dim, "dispatches": len(fv),
                              "hbm_read_bytes_per_launch": round(rd), "hbm_write_bytes_per_launch": round(wr),
                              "hbm_bytes_per_launch": round(rd + wr), "algorithmic_bytes": alg,
                              "algorithmic_read_bytes": alg_rd}
        lines.append("| %s | %s | %d | %.4g | %.4g | %.4g | %.4f |" % (
            spec.name, kernels[spec.name]["kernel"], len(fv), rd, wr, alg, rd / alg_rd))
    # the MXFP4 MQA logits, when the run included it (bench.py --mqa): its
    # 16 x 131072-position decode workload is the launch with the largest grid
    fg, wg = by_grid(fetch_csv, "FETCH_SIZE", "pa_mqa_logits_mxfp4_kernel"), by_grid(write_csv, "WRITE_SIZE",
                                                                                    "pa_mqa_logits_mxfp4_kernel")
    if fg and wg:
        grid = max(fg)
        fv, wv = fg[grid], wg[grid]
        rd = sum(fv) / len(fv) * 1024 * f_factor
        wr = sum(wv) / len(wv) * 1024 * w_factor
        spec = I.MQA_DECODE_LONG
        case = I.make_mqa_case(spec)
        alg = case.bytes_moved()
        alg_rd = case.window_tokens() * (case.head_dim // 2 + case.head_dim // 32)
        kernels[spec.name] = {"kernel": "pa_mqa_logits_mxfp4_kernel<%d>" % (spec.num_heads // 16),
                              "dispatches": len(fv), "hbm_read_bytes_per_launch": round(rd),
                              "hbm_write_bytes_per_launch": round(wr), "hbm_bytes_per_launch": round(rd + wr),
                              "algorithmic_bytes": alg, "algorithmic_read_bytes": alg_rd}
        lines.append("| %s | %s | %d | %.4g | %.4g | %.4g | %.4f |" % (
            spec.name, kernels[spec.name]["kernel"], len(fv), rd, wr, alg, rd / alg_rd))
    doc = {"kernel_source": kernel_source_hash(), "fetch_factor": round(f_factor, 4),
           "write_factor": round(w_factor, 4), "kernels": kernels}
    with open(out_json, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print("Calibration (1 GiB torch.neg copy): FETCH_SIZE x %.4f, WRITE_SIZE x %.4f\n" % (f_factor, w_factor))
    print("\n".join(lines))


def read_bytes(case) -> int:
    """Algorithmic KV bytes of a call: K, V and scales of the tokens some query
    row attends to. That is [max(0, e_0 - window), L) per sequence with a
    window (e_0 = L - qlen + 1 when causal, else L), else all of [0, L)."""
    if not getattr(case, "window", 0):
        return case.kv_bytes()
    toks = 0
    for L in case.context_lens.tolist():
        e0 = max(0, L - case.qlen + 1) if case.causal else L
        toks += L - max(0, e0 - case.window)
    return toks * case.num_kv_heads * case.kv_bytes_per_token_head()


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo) and its logical CPU count."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return "%s (%d logical CPUs visible)" % (name, os.cpu_count() or 0)


def time_cpu_oracle(case, target_s=15.0):
    import oracle

    # one sequence first, then as many more as fit the time budget
    t0 = time.perf_counter()
    oracle.pa_decode(case, seqs=[0])
    dt = time.perf_counter() - t0
    n = max(1, min(case.num_seqs, int(target_s / max(dt, 1e-3))))
    seqs = list(range(n))
    reps = 0
    t0 = time.perf_counter()
    while True:  # whole passes over the sample until about target_s of CPU work
        oracle.pa_decode(case, seqs=seqs)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_s or reps >= 100:
            break
    nbytes = case.kv_bytes(seqs) * reps
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d of %d sequences of the page-64 variant, %d passes (%.0f MB of KV), %.1f s" % (
                n, case.num_seqs, reps, nbytes / 1e6, dt)}


# The workloads of the decode's five configurations, timed per call by default.
PER_CONFIG = [("cfg1", "TINY_BF16"), ("cfg2", "BF16_P64"), ("cfg2", "BF16_P128"), ("cfg3", "FP8TOK_Q1"),
              ("cfg3", "FP8TOK_Q4"), ("cfg4", "FP8_TRANS"), ("cfg5a", "MXFP4_SHORT_Q8"), ("cfg5a", "MXFP4_SHORT_QBF"),
              ("cfg5b", "MXFP4_LONG_Q8"), ("cfg5b", "MXFP4_LONG_QBF")]
# and the MXFP4 ones again with the opt-in block-scaled fp4 x fp8 QK MFMA
PER_CONFIG_SCALED_QK = ("MXFP4_SHORT_Q8", "MXFP4_SHORT_QBF", "MXFP4_LONG_Q8", "MXFP4_LONG_QBF")


def time_case(case, steps, warmup, flush, flush_out, extras=False, **problem_over):
    """Cold-cache timing of pa_decode on one case (inputs resident in HBM).

    Before each call a 1 GiB buffer is read (the last-level cache is 256 MB; a
    read leaves clean lines, where a write would leave dirty lines for the
    decode to write back); the median of the per-call event times is kept. The
    tile / merge split comes from the library's own events around each kernel,
    in a separate pass of the same cold calls; it is a mean, so a slow outlier
    call shows there and not in the median. With `extras`, also the differential
    figure (see time_all) and the plan-free pa_decode_direct's cold median."""
    import statistics

    import torch

    import paged_attention_decode_token_amd as pa

    d = pa.device_tensors(case)
    plan = pa.pa_plan(pa.problem_of(case, **problem_over), case.context_lens)
    out = torch.empty((case.num_seqs, case.qlen, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                      device="cuda")

    def call():
        pa.pa_decode(plan, d["query"], d["key_cache"], d["value_cache"], d["k_scale"], d["v_scale"],
                     d["block_tables"], d["context_lens"], out)

    def cold_median(fn):
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            torch.amax(flush, dim=0, out=flush_out)  # read-only sweep of the flush buffer
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3

    us = cold_median(call)
    plan.set_timing(True, steps)
    for _ in range(steps):
        torch.amax(flush, dim=0, out=flush_out)  # same cold start as the median's calls
        call()
    torch.cuda.synchronize()
    t_ms, m_ms, n = plan.read_timing()
    plan.set_timing(False)
    nbytes = read_bytes(case)
    inf = plan.info()
    gbps = nbytes / (us * 1e-6) / 1e9
    row = {"us_per_call": round(us, 2), "kv_bytes": nbytes, "kv_GBps": round(gbps, 1),
           "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBS, 1), "tile_us": round(t_ms / n * 1e3, 2),
           "merge_us": round(m_ms / n * 1e3, 2) if inf.merge_needed else 0.0,
           "tasks": inf.num_tasks, "slots": inf.slots, "partitions_max": inf.max_parts}
    if extras:
        # differential cold time: the event packets' cost is paid once per batch;
        # batches with and without the calls alternate, and the median of five
        # differences is kept (the flushes alone vary by about 1 % between batches)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        diffs = []
        for _ in range(5):
            a.record()
            for _ in range(steps):
                torch.amax(flush, dim=0, out=flush_out)
                call()
            b.record()
            torch.cuda.synchronize()
            t_calls = a.elapsed_time(b)
            a.record()
            for _ in range(steps):
                torch.amax(flush, dim=0, out=flush_out)
            b.record()
            torch.cuda.synchronize()
            diffs.append((t_calls - a.elapsed_time(b)) * 1e3 / steps)
        us_diff = statistics.median(diffs)
        prob = pa.problem_of(case, **problem_over)

        def call_direct():
            pa.pa_decode_direct(prob, d["query"], d["key_cache"], d["value_cache"], d["k_scale"], d["v_scale"],
                                d["block_tables"], d["context_lens"], out)

        us_direct = cold_median(call_direct)
        row.update({"us_per_call_differential": round(us_diff, 2),
                    "pct_of_hbm_peak_differential": round(100 * nbytes / (us_diff * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                    "plan_free_us_per_call": round(us_direct, 2),
                    "plan_free_pct_of_hbm_peak": round(100 * nbytes / (us_direct * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)})
    del d, plan, out
    torch.cuda.empty_cache()
    return row


def time_per_config(steps, warmup):
    """The default line's per-configuration block: every workload of the five
    configurations, cold median us per pa_decode call, KV GB/s, % of 8 TB/s and
    the tile / merge split."""
    import torch

    from paged_attention_decode_token_amd import inputs as I

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB > 256 MB last-level cache
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    rows = {}
    for cfg, attr in PER_CONFIG:
        spec = getattr(I, attr)
        case = I.make_case(spec)
        variants = [("", {})] + ([("_scaled_qk", {"mxfp4_scaled_qk": 1})] if attr in PER_CONFIG_SCALED_QK else [])
        for suffix, over in variants:
            row = {"config": cfg}
            row.update(time_case(case, steps, warmup, flush, flush_out, **over))
            rows[spec.name + suffix] = row
            print("%-6s %-42s %9.2f us  %7.1f GB/s  %5.1f%%  tile %8.2f us  merge %6.2f us" % (
                cfg, spec.name + suffix, row["us_per_call"], row["kv_GBps"], row["pct_of_hbm_peak"], row["tile_us"],
                row["merge_us"]), file=sys.stderr, flush=True)
        del case
    del flush
    torch.cuda.empty_cache()
    return rows


def time_all(steps, warmup, names=None, task_budgets=(0,)):
    """Per workload: cold-cache median us per pa_decode call, and the tile / merge
    kernel split from the library's events (inputs resident in HBM).

    Each event pair also brackets the event packets' own queue time (a few us,
    which is a tenth of a 60 us call). So a second, differential figure is taken
    too: `steps` cold calls (flush, call, flush, call, ...) between two events,
    minus `steps` flushes alone between two events, divided by `steps` (median
    of five alternating pairs of batches). With several task budgets (0: the
    planner's automatic choice) each workload is timed once per budget, and
    the rows of budgets other than 0 are keyed `name@budget`."""
    import torch

    from paged_attention_decode_token_amd import inputs as I

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB > 256 MB last-level cache
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    rows = {}
    specs = I.FULL if not names else [I.BY_NAME[n] for n in names]
    for spec in specs:
        case = I.make_case(spec)
        for budget in task_budgets:
            row = time_case(case, steps, warmup, flush, flush_out, extras=True, task_budget=budget)
            key = spec.name if budget == 0 else "%s@%d" % (spec.name, budget)
            rows[key] = row
            print("%-32s %9.2f us  %7.1f GB/s  %5.1f%%  differential %8.2f us %5.1f%%  tile %8.2f us  merge %6.2f us  "
                  "tasks %5d slots %4d  plan-free %8.2f us" % (
                      key, row["us_per_call"], row["kv_GBps"], row["pct_of_hbm_peak"],
                      row["us_per_call_differential"], row["pct_of_hbm_peak_differential"], row["tile_us"],
                      row["merge_us"], row["tasks"], row["slots"], row["plan_free_us_per_call"]),
                  file=sys.stderr, flush=True)
        del case
    return rows


def time_writes(steps, warmup):
    """Per MXFP4 cache-write workload: cold-cache median and warm mean us per
    pa_write_kv_mxfp4 call (one kernel on torch's current stream), and the
    algorithmic GB/s: valid tokens x KV heads x (4 D read + 2 (D/2 + D/32) written)."""
    import statistics

    import torch

    import paged_attention_decode_token_amd as pa
    from paged_attention_decode_token_amd import inputs as I

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    rows = {}
    for spec in I.WRITE_FULL:
        case = I.make_write_case(spec, device="cuda")
        args = (case.key, case.value, case.slot_mapping, case.key_cache, case.value_cache, case.key_scale,
                case.value_scale)

        def call():
            pa.pa_write_kv_mxfp4(*args)

        for _ in range(warmup):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            torch.amax(flush, dim=0, out=flush_out)
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        us = statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3
        a, b = ev[0]
        a.record()
        for _ in range(steps):
            call()
        b.record()
        torch.cuda.synchronize()
        us_warm = a.elapsed_time(b) * 1e3 / steps
        nbytes = case.bytes_moved()
        gbps = nbytes / (us * 1e-6) / 1e9
        rows[spec.name] = {"us_per_call": round(us, 2), "warm_us_per_call": round(us_warm, 2),
                           "tokens": case.num_tokens, "valid_tokens": case.valid_tokens(), "bytes": nbytes,
                           "GBps": round(gbps, 1), "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBS, 1),
                           "traffic": load_traffic(spec.name)}
        print("%-32s %9.2f us  %7.1f GB/s  %5.1f%%  warm %8.2f us  tokens %d" % (
            spec.name, us, gbps, 100 * gbps / HBM_PEAK_GBS, us_warm, case.num_tokens), file=sys.stderr, flush=True)
        del args, case
        torch.cuda.empty_cache()
    return rows


def time_mqa(steps, warmup):
    """Per MXFP4 MQA-logits workload: cold-cache median us per pa_mqa_logits_mxfp4
    call and the algorithmic GB/s: window positions x (one K row of 68 bytes
    read + one fp32 score written)."""
    import statistics

    import torch

    import paged_attention_decode_token_amd as pa
    from paged_attention_decode_token_amd import inputs as I

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    rows = {}
    for spec in I.MQA_FULL:
        case = I.make_mqa_case(spec, device="cuda")
        out = torch.full((case.num_rows, case.out_stride), float("-inf"), dtype=torch.float32, device="cuda")
        prob = pa.mqa_problem_of(case)
        args = (prob, case.q, case.q_scale, case.weights, case.k_cache, case.k_scale, case.block_tables,
                case.row_to_batch, case.local_starts, case.local_ends, out)

        def call():
            pa.pa_mqa_logits_mxfp4(*args)

        for _ in range(warmup):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            torch.amax(flush, dim=0, out=flush_out)
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        us = statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3
        nbytes = case.bytes_moved()
        gbps = nbytes / (us * 1e-6) / 1e9
        rows[spec.name] = {"us_per_call": round(us, 2), "rows": case.num_rows, "positions": case.window_tokens(),
                           "bytes": nbytes, "GBps": round(gbps, 1),
                           "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBS, 1),
                           "tflops": round(case.window_tokens() * case.num_heads * case.head_dim * 2 / (us * 1e-6)
                                           / 1e12, 1),
                           "traffic": load_traffic(spec.name)}
        print("%-40s %9.2f us  %7.1f GB/s  %5.1f%%  positions %d" % (
            spec.name, us, gbps, 100 * gbps / HBM_PEAK_GBS, case.window_tokens()), file=sys.stderr, flush=True)
        del args, case, out
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-configuration cold per-call block of the default line")
    ap.add_argument("--all", action="store_true",
                    help="also time every workload (one pa_decode call each) and print a table to stderr")
    ap.add_argument("--kv-write", action="store_true",
                    help="also time the MXFP4 cache-write workloads (implied by --all)")
    ap.add_argument("--mqa", action="store_true",
                    help="also time the MXFP4 paged MQA-logits workloads (implied by --all)")
    ap.add_argument("--workloads", default="",
                    help="with --all: comma-separated workload names to time (default: every workload)")
    ap.add_argument("--task-budgets", default="0",
                    help="with --all: comma-separated task budgets to plan each workload with "
                         "(0: the planner's automatic choice)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for counter calibration)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs of "
                         "`bench.py --calibrate-copy` into profiles/traffic.json")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], os.path.join(ROOT, "profiles", "traffic.json"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_attention_decode_token_amd as pa
    from paged_attention_decode_token_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    pa.lib()

    variants = []
    for spec in (I.BF16_P64, I.BF16_P128):
        case = I.make_case(spec)
        d = pa.device_tensors(case)
        plan = pa.pa_plan(pa.problem_of(case), case.context_lens)
        out = torch.empty((case.num_seqs, case.qlen, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                          device="cuda")
        variants.append(dict(spec=spec, case=case, d=d, plan=plan, out=out, bytes=case.kv_bytes()))
    torch.cuda.synchronize()

    def step():
        for v in variants:
            d = v["d"]
            pa.pa_decode(v["plan"], d["query"], d["key_cache"], d["value_cache"], d["k_scale"], d["v_scale"],
                         d["block_tables"], d["context_lens"], v["out"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calibrate_copy:
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        y = torch.empty_like(x)
        torch.neg(x, out=y)
        torch.cuda.synchronize()
        del x, y
    # timed steps: nothing but the decodes on the stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # the same steps again with the library's events around each kernel launch
    for v in variants:
        v["plan"].set_timing(True, args.steps)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_instr = start.elapsed_time(stop) / args.steps
    per = {}
    tile_bytes = tile_ms = 0.0
    for v in variants:
        t_ms, m_ms, n = v["plan"].read_timing()
        v["plan"].set_timing(False)
        tile_avg = t_ms / n
        inf = v["plan"].info()
        per[v["spec"].name] = {"tile_us": round(tile_avg * 1e3, 2),
                               "merge_us": round(m_ms / n * 1e3, 2) if inf.merge_needed else 0.0,
                               "kv_bytes": v["bytes"], "tile_kv_GBps": round(v["bytes"] / (tile_avg * 1e-3) / 1e9, 1),
                               "tasks": inf.num_tasks, "partitions_max": inf.max_parts}
        tile_bytes += v["bytes"]
        tile_ms += tile_avg
    step_bytes = sum(v["bytes"] for v in variants)
    value = step_bytes / (ms * 1e-3) / 1e9
    achieved = tile_bytes / (tile_ms * 1e-3) / 1e9
    traffic = None
    tr = [load_traffic(v["spec"].name) for v in variants]
    if all(t is not None for t in tr):
        traffic = sum(tr)
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 paged decode, page 64 and page 128 variants (one call each per step), "
                               "batch 64, context U[1000, 8192], 8 KV heads x GQA 8, head_dim 128, qlen 1",
                   "global_batch": 64, "seq_len": "U[1000,8192]", "parallelism": "none (1 GPU)"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "per_call": per,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "pa_tile_kernel (bf16, D 128, page 64 and 128)",
                     "algorithmic_bytes_per_step": tile_bytes,
                     "timing": "library HIP events around each tile launch, second pass of the timed steps "
                               "(%.4f ms per step with the events)" % ms_instr},
    }
    del variants
    torch.cuda.empty_cache()
    if not args.no_per_config:
        res["per_config"] = time_per_config(args.steps, args.warmup)
    if args.all:
        res["all_workloads"] = time_all(args.steps, args.warmup,
                                        [w for w in args.workloads.split(",") if w] or None,
                                        [int(b) for b in args.task_budgets.split(",") if b] or [0])
    if args.all or args.kv_write:
        res["kv_write"] = time_writes(args.steps, args.warmup)
    if args.all or args.mqa:
        res["mqa_logits"] = time_mqa(args.steps, args.warmup)
    if not args.no_cpu:
        res["cpu_baseline"] = time_cpu_oracle(I.make_case(I.BF16_P64))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
