"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, validates descriptors, and the host planner covers every
owned tile exactly once. No GPU is touched."""
import os
import re

import numpy as np
import pytest
import torch

from paged_attention_decode_token_amd import binding as B
from paged_attention_decode_token_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:pa_status|void|size_t|const char\*)\s+(pa_\w+)\s*\(", src, re.M)))


def test_header_symbols_are_exported():
    lib = B.lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def test_version():
    assert "gfx950" in B.pa_version()


def _prob(**kw):
    base = dict(num_seqs=4, qlen=1, num_kv_heads=2, q_per_kv=8, head_dim=128, page_size=16, num_blocks=100,
                max_blocks_per_seq=40, max_context_len=600)
    base.update(kw)
    return B.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=32), B.PA_ERR_UNSUPPORTED),
    (dict(head_dim=64), B.PA_ERR_UNSUPPORTED),
    (dict(qlen=9, q_per_kv=8), B.PA_ERR_UNSUPPORTED),  # 72 query rows per KV head
    (dict(qlen=5, q_per_kv=8, head_dim=256), B.PA_ERR_UNSUPPORTED),  # 40 rows at head_dim 256
    (dict(num_blocks=0), B.PA_ERR_INVALID_ARG),
    (dict(qlen=0), B.PA_ERR_INVALID_ARG),
    (dict(kv_dtype="fp8"), B.PA_ERR_INVALID_ARG),  # fp8 without scales
    (dict(kv_dtype="bf16", scale_mode="tensor"), B.PA_ERR_INVALID_ARG),
    (dict(kv_dtype="mxfp4", page_size=64), B.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype="mxfp4", page_size=128, head_dim=256), B.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype="mxfp4", page_size=128, qlen=2), B.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype="mxfp4", page_size=128, q_per_kv=32), B.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype="mxfp4", page_size=128, v_layout="trans"), B.PA_ERR_UNSUPPORTED),
    (dict(q_dtype="fp8"), B.PA_ERR_UNSUPPORTED),  # e4m3 query only with MXFP4
    (dict(softmax_scale=float("nan")), B.PA_ERR_INVALID_ARG),
    (dict(causal=2), B.PA_ERR_INVALID_ARG),
    (dict(window=-1), B.PA_ERR_INVALID_ARG),
    (dict(kv_dtype="mxfp4", page_size=128, window=64), B.PA_ERR_UNSUPPORTED),
])
def test_refusals(kw, status):
    with pytest.raises(B.PaError) as ei:
        B.pa_plan_host(_prob(**kw), [10, 20, 30, 40])
    assert ei.value.status == status
    assert B.pa_last_error()


@pytest.mark.parametrize("kw", [dict(qlen=4, q_per_kv=16), dict(qlen=5, q_per_kv=8), dict(qlen=2, q_per_kv=16),
                                dict(qlen=4, q_per_kv=8, head_dim=256), dict(qlen=8, q_per_kv=8, page_size=128)])
def test_row_counts_up_to_64_are_planned(kw):
    """Up to 64 query rows per KV head at head_dim 128 (ROCm/aiter PR #7092,
    "Tests": the (qlen 4, one KV head, GQA 16, head_dim 128) case), up to 32
    at head_dim 256."""
    tasks, parts, info = B.pa_plan_host(_prob(**kw), [10, 20, 300, 600])
    assert info.num_tasks > 0


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=32), B.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype="mxfp4", page_size=128, qlen=2), B.PA_ERR_UNSUPPORTED),
    (dict(qlen=0), B.PA_ERR_INVALID_ARG),
    (dict(), B.PA_ERR_INVALID_ARG),  # a valid problem with NULL pointers
])
def test_plan_free_refusals_come_before_the_device(kw, status):
    """pa_decode_direct validates the descriptor, then the pointers, and only
    then probes the device: every refusal here returns on a host without one."""
    st = B.lib().pa_decode_direct(B.ctypes.byref(_prob(**kw)), *([None] * 9))
    assert st == status
    assert B.pa_last_error()


def _wprob(**kw):
    base = dict(num_tokens=8, num_kv_heads=4, head_dim=128, page_size=128, num_blocks=10)
    base.update(kw)
    return B.pa_kv_write_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(head_dim=512), B.PA_ERR_UNSUPPORTED),
    (dict(num_tokens=-1), B.PA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), B.PA_ERR_INVALID_ARG),
    (dict(page_size=0), B.PA_ERR_INVALID_ARG),
    (dict(num_blocks=0), B.PA_ERR_INVALID_ARG),
    (dict(num_blocks=2 ** 24, page_size=256), B.PA_ERR_UNSUPPORTED),  # 2^32 slots
    (dict(num_tokens=2 ** 27, num_kv_heads=2, head_dim=64), B.PA_ERR_UNSUPPORTED),  # 2^34 elements
    (dict(), B.PA_ERR_INVALID_ARG),  # a valid problem with NULL pointers
])
def test_kv_write_refusals_come_before_the_device(kw, status):
    """pa_write_kv_mxfp4 checks the descriptor and the pointers before it
    probes the device: every refusal here returns on a host without one."""
    st = B.lib().pa_write_kv_mxfp4(B.ctypes.byref(_wprob(**kw)), *([None] * 8))
    assert st == status
    assert B.pa_last_error()


def test_kv_write_of_no_tokens_is_a_no_op():
    assert B.lib().pa_write_kv_mxfp4(B.ctypes.byref(_wprob(num_tokens=0)), *([None] * 8)) == B.PA_OK


def _mprob(**kw):
    base = dict(num_rows=4, num_heads=64, head_dim=128, page_size=64, num_blocks=10, num_seqs=2,
                max_blocks_per_seq=5, out_stride=400)
    base.update(kw)
    return B.pa_mqa_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), B.PA_ERR_UNSUPPORTED),
    (dict(num_heads=48), B.PA_ERR_UNSUPPORTED),
    (dict(page_size=8), B.PA_ERR_UNSUPPORTED),
    (dict(num_rows=-1), B.PA_ERR_INVALID_ARG),
    (dict(num_blocks=0), B.PA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=0), B.PA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=2 ** 26, page_size=64), B.PA_ERR_UNSUPPORTED),  # reach beyond 2^31
    (dict(), B.PA_ERR_INVALID_ARG),  # a valid problem with NULL pointers
])
def test_mqa_refusals_come_before_the_device(kw, status):
    st = B.lib().pa_mqa_logits_mxfp4(B.ctypes.byref(_mprob(**kw)), *([None] * 11))
    assert st == status
    assert B.pa_last_error()


def test_mqa_with_no_rows_is_a_no_op():
    assert B.lib().pa_mqa_logits_mxfp4(B.ctypes.byref(_mprob(num_rows=0)), *([None] * 11)) == B.PA_OK


def test_mqa_binding_checks_shapes_before_the_device():
    from paged_attention_decode_token_amd import inputs as MI
    case = MI.make_mqa_case(MI.small_mqa(MI.MQA_DECODE_LONG))
    prob = B.mqa_problem_of(case)
    out = torch.zeros((case.num_rows, case.out_stride), dtype=torch.float32)
    args = [case.q, case.q_scale, case.weights, case.k_cache, case.k_scale, case.block_tables, case.row_to_batch,
            case.local_starts, case.local_ends, out]
    for i, bad in ((0, case.q[:, :, :32]), (2, case.weights[:-1]), (5, case.block_tables[:, :-1]),
                   (9, out[:, :-16])):
        a = list(args)
        a[i] = bad.contiguous()
        with pytest.raises(ValueError, match="shape"):
            B.pa_mqa_logits_mxfp4(prob, *a)
    with pytest.raises(ValueError, match="device"):  # right shapes, host tensors
        B.pa_mqa_logits_mxfp4(prob, *args)


@pytest.mark.parametrize("spec", [I.TINY_BF16, I.small(I.FP8TOK_Q1), I.small(I.FP8_TRANS), I.small(I.MXFP4_SHORT_Q8)],
                         ids=lambda s: s.name)
def test_decode_binding_checks_sizes_before_the_device(spec):
    case = I.make_case(spec)
    prob = B.problem_of(case)
    t = case.tensors()
    out = torch.zeros((case.num_seqs, case.qlen, case.num_q_heads, case.head_dim), dtype=torch.bfloat16)
    args = dict(query=t["query"], key_cache=t["key_cache"], value_cache=t["value_cache"], k_scale=t["k_scale"],
                v_scale=t["v_scale"], block_tables=t["block_tables"], context_lens=t["context_lens"], out=out)
    for name, bad in (("key_cache", t["key_cache"][:-1]), ("block_tables", t["block_tables"][:, :-1]),
                      ("out", out[:-1]), ("query", t["query"][:, :, :-1])):
        a = dict(args)
        a[name] = bad.contiguous()
        with pytest.raises(ValueError, match="bytes|shape"):
            B.pa_decode_direct(prob, **a)
    with pytest.raises(ValueError, match="device"):  # right sizes, host tensors
        B.pa_decode_direct(prob, **args)


def test_host_length_checks():
    with pytest.raises(B.PaError):
        B.pa_plan_host(_prob(), [10, -1, 30, 40])
    with pytest.raises(B.PaError):  # longer than the table can address
        B.pa_plan_host(_prob(max_context_len=10 ** 6), [10, 20, 30, 40 * 16 + 1])
    with pytest.raises(B.PaError):  # longer than max_context_len
        B.pa_plan_host(_prob(), [10, 20, 30, 601])


@pytest.mark.parametrize("lens,budget,maxp", [
    ([0, 1, 255, 256, 257, 600], 0, 0),
    ([600] * 6, 0, 0),
    ([1, 600, 33, 0, 599, 512], 1000, 0),
    ([600, 600, 600, 600, 600, 600], 1000, 2),
    ([5000] * 3 + [1], 0, 0),
])
def test_planner_covers_every_owned_tile_once(lens, budget, maxp):
    n = len(lens)
    p = _prob(num_seqs=n, max_blocks_per_seq=400, max_context_len=max(lens), task_budget=budget,
              max_partitions=maxp)
    tasks, parts, info = B.pa_plan_host(p, lens, num_cus=16)
    H = p.num_kv_heads
    seen = {}
    for b, kp, t0, t1 in tasks.tolist():
        kvh, part = kp & 0xFFFF, kp >> 16
        assert 0 <= b < n and 0 <= kvh < H and 0 <= t0 <= t1
        assert part < parts[b * H + kvh, 0]
        for t in range(t0, t1):
            key = (b, kvh, t)
            assert key not in seen, key
            seen[key] = part
    for b, L in enumerate(lens):
        nt = (L + 255) // 256
        for kvh in range(H):
            for t in range(nt):
                assert (b, kvh, t) in seen
        assert all(t < nt for (bb, _, t) in seen if bb == b)
        # every (b, kvh) has exactly its partition count of tasks, partials only when split
        for kvh in range(H):
            cnt = sum(1 for r in tasks.tolist() if r[0] == b and (r[1] & 0xFFFF) == kvh)
            assert cnt == parts[b * H + kvh, 0]
            assert (parts[b * H + kvh, 1] >= 0) == (parts[b * H + kvh, 0] > 1)
    # longest first
    sizes = (tasks[:, 3] - tasks[:, 2]).tolist()
    assert sizes == sorted(sizes, reverse=True)
    if maxp:
        assert int(parts[:, 0].max()) <= maxp
    assert info.num_tasks == len(tasks)


@pytest.mark.parametrize("heads,pages", [(2, 16), (4, 16), (2, 64), (3, 16)])
def test_planner_pairs_heads_that_share_scale_lines(heads, pages):
    # fp8 with per-token scales: at 16-token pages the scale rows of heads 2k and 2k + 1 of a
    # page share a 128-byte line, and their tasks go 8 launch slots apart (one XCD)
    rng = np.random.default_rng(7)
    lens = rng.integers(2048, 32769, size=16).tolist()
    p = _prob(num_seqs=16, num_kv_heads=heads, head_dim=256, page_size=pages, kv_dtype=B.PA_KV_FP8_E4M3,
              scale_mode=B.PA_SCALE_PER_TOKEN, max_blocks_per_seq=32768 // pages, num_blocks=20000,
              max_context_len=32768)
    tasks, parts, info = B.pa_plan_host(p, lens, num_cus=256, blocks_per_cu=1)
    rows = tasks.tolist()
    # every owned tile exactly once
    seen = set()
    for b, kp, t0, t1 in rows:
        for t in range(t0, t1):
            assert (b, kp & 0xFFFF, t) not in seen
            seen.add((b, kp & 0xFFFF, t))
    assert seen == {(b, h, t) for b, L in enumerate(lens) for h in range(heads) for t in range((L + 255) // 256)}
    sizes = [t1 - t0 for _, _, t0, t1 in rows]
    n = len(rows)
    if pages == 16 and heads % 2 == 0:
        full = n // 16 * 16
        for m in range(0, full, 16):
            for x in range(8):
                a, c = rows[m + x], rows[m + 8 + x]
                assert a[0] == c[0] and a[2:] == c[2:] and (a[1] >> 16) == (c[1] >> 16)
                assert (a[1] & 0xFFFF) % 2 == 0 and (c[1] & 0xFFFF) == (a[1] & 0xFFFF) + 1
        runs = [sizes[m:m + 16] for m in range(0, full, 16)] + [[s] for s in sizes[full:]]
        for r0, r1 in zip(runs, runs[1:]):
            assert min(r0) >= max(r1)
        assert sizes[full:] == sorted(sizes[full:], reverse=True)
    else:
        assert sizes == sorted(sizes, reverse=True)


def test_planner_without_host_lengths_uses_max_context():
    p = _prob(num_seqs=3, max_context_len=1000, max_blocks_per_seq=100, task_budget=12)
    tasks, parts, info = B.pa_plan_host(p, None, num_cus=16)
    assert int(parts[:, 0].min()) == int(parts[:, 0].max())
    assert int(tasks[:, 3].max()) == 4  # ceil(1000/256)


def test_full_workload_plans():
    for spec in I.FULL:
        case_lens = I._lens(spec, torch.Generator().manual_seed(spec.seed))
        PG = spec.page_size
        width = max((L + PG - 1) // PG for L in case_lens) + 2
        p = B.make_problem(spec.num_seqs, spec.qlen, spec.num_kv_heads, spec.q_per_kv, spec.head_dim, PG, 10,
                           width, max(case_lens), spec.kv_dtype, spec.scale_mode, spec.v_layout, spec.q_dtype)
        tasks, parts, info = B.pa_plan_host(p, case_lens, num_cus=256)
        assert info.num_tasks >= 1 and info.max_parts <= 64


@pytest.mark.parametrize("window,causal", [(300, 0), (1000, 1), (1, 1)])
def test_planner_skips_tiles_before_the_window(window, causal):
    """With host lengths, tasks start at the first tile of the first query
    token's window and still cover every tile from there to ceil(L / 256)."""
    lens = [0, 5, 255, 256, 700, 5000]
    prob = _prob(num_seqs=len(lens), qlen=4, q_per_kv=4, max_blocks_per_seq=400, max_context_len=6000,
                 causal=causal, window=window)
    for budget in (0, 50, 100000):
        prob.task_budget = budget
        tasks, parts, info = B.pa_plan_host(prob, lens)
        for b, L in enumerate(lens):
            e0 = L - 4 + 1 if causal else L
            first = max(0, e0 - window) // 256
            ntiles = (L + 255) // 256
            for kvh in range(prob.num_kv_heads):
                mine = sorted((t[2], t[3]) for t in tasks.tolist() if t[0] == b and (t[1] & 0xFFFF) == kvh)
                covered = [x for t0, t1 in mine for x in range(t0, t1)]
                assert covered == list(range(min(first, ntiles), ntiles)), (b, L, mine)


def test_static_decode_refuses_partials_beyond_its_buffer_before_the_device():
    """pa_decode_static with an explicit partition count whose partials do not
    fit its static buffer is refused with PA_ERR_UNSUPPORTED before any device
    call (so on a host without one too); the pointers are never touched."""
    p = _prob(num_seqs=64, num_kv_heads=8, q_per_kv=8, max_context_len=64 * 256, max_blocks_per_seq=1100,
              max_partitions=64)
    fake = [B.ctypes.c_void_p(0x100000 + 0x1000 * i) for i in range(9)]
    st = B.lib().pa_decode_static(B.ctypes.byref(p), *fake)
    assert st == B.PA_ERR_UNSUPPORTED
    msg = B.pa_last_error()
    assert "static scratch" in msg and "partitions" in msg, msg

