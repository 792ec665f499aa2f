"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar: rel-L2 = ||gpu - o|| / ||o|| <= 3e-3
over the compared rows, and |gpu_i - o_i| <= 2e-2 * max(1, |o_i|) per element,
where o is the oracle's unrounded fp64 result and gpu is the bf16 output. Plus
the NaN contract: output finite and bit-identical between runs whose unowned
rows are zero-filled and runs where they hold NaN / Inf / random bytes
(ROCm/aiter PR #7092, section "Tests"), and bit-identical across repeated runs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_token_amd import binding as B
from paged_attention_decode_token_amd import inputs as I

pytestmark = pytest.mark.gpu

from parity_bar import REL_L2, check_parity, parity_stats  # the bar, shared with its CPU controls


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()  # raises when libpa.so is missing


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def run(case, **over):
    out, plan = B.decode_case(case, **over)
    torch.cuda.synchronize()
    return out, plan


SMALL = [I.small(s) for s in I.FULL if not s.name.endswith("l131072_qfp8") and not s.name.endswith("l131072_qbf16")]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_parity_small(spec):
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    out, plan = run(case)
    check_parity(out, ref, what=spec.name)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_poison_fills_are_bit_identical_to_zero_fill(spec):
    case = I.make_case(spec, fill="zero")
    ref_bits = _bits(run(case)[0])
    assert np.isfinite(run(case)[0].float().cpu().numpy()).all()
    for fill in ("nan", "inf", "random"):
        out = run(I.refill(case, fill))[0]
        assert np.array_equal(_bits(out), ref_bits), "%s fill changes the output" % fill


@pytest.mark.parametrize("spec", SMALL[:3] + SMALL[5:6], ids=lambda s: s.name)
def test_repeat_runs_are_bit_identical(spec):
    case = I.make_case(spec)
    d = B.device_tensors(case)
    plan = B.pa_plan(B.problem_of(case), case.context_lens)
    outs = []
    for _ in range(3):
        o = torch.full((case.num_seqs, case.qlen, case.num_q_heads, case.head_dim), float("nan"),
                       dtype=torch.bfloat16, device="cuda")
        B.pa_decode(plan, d["query"], d["key_cache"], d["value_cache"], d["k_scale"], d["v_scale"],
                    d["block_tables"], d["context_lens"], o)
        outs.append(_bits(o))
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])


@pytest.mark.parametrize("spec", [SMALL[1], SMALL[3], SMALL[5], SMALL[6]], ids=lambda s: s.name)
@pytest.mark.parametrize("variant", ["one_partition", "many_partitions", "no_host_lens"])
def test_plan_variants_agree_with_oracle(spec, variant):
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    if variant == "one_partition":
        out, plan = run(case, max_partitions=1)
        assert plan.info().merge_needed == 0
    elif variant == "many_partitions":
        out, plan = run(case, task_budget=100000)
        assert plan.info().max_parts > 1 or int(case.context_lens.max()) <= 256
    else:
        d = B.device_tensors(case)
        plan = B.pa_plan(B.problem_of(case), None)
        out = torch.full((case.num_seqs, case.qlen, case.num_q_heads, case.head_dim), float("nan"),
                         dtype=torch.bfloat16, device="cuda")
        B.pa_decode(plan, d["query"], d["key_cache"], d["value_cache"], d["k_scale"], d["v_scale"],
                    d["block_tables"], d["context_lens"], out)
        torch.cuda.synchronize()
    check_parity(out, ref, what="%s/%s" % (spec.name, variant))


EDGE_LENS = (0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 767, 1000)


@pytest.mark.parametrize("base", [I.TINY_BF16, I.BF16_P64, I.FP8TOK_Q1, I.FP8TOK_Q4, I.FP8_TRANS, I.MXFP4_SHORT_QBF],
                         ids=lambda s: s.name)
def test_edge_lengths(base):
    spec = base.replace(name=base.name + "_edges", num_seqs=len(EDGE_LENS), lens=("fixed", EDGE_LENS),
                        num_kv_heads=min(base.num_kv_heads, 2))
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    for over in ({}, {"task_budget": 100000}):
        out, _ = run(case, **over)
        check_parity(out, ref, what="%s %s" % (spec.name, over))
        z = out[0].float().cpu()  # L = 0 row is exactly zero
        assert torch.all(z == 0)


def test_rows_of_context_len_one_are_v_row_zero():
    spec = I.TINY_BF16.replace(name="len1", lens=("fixed", (1, 1, 1, 1)))
    case = I.make_case(spec)
    out, _ = run(case)
    for b in range(4):
        p = int(case.block_tables[b, 0])
        v0 = case.value_cache[p, 0, 0].view(torch.int16)
        for h in range(case.num_q_heads):
            assert torch.equal(out[b, 0, h].cpu().view(torch.int16), v0)


# ------------------------------------------------------------- full sizes

FULL_SAMPLE = {  # sequences the oracle recomputes at full size
    "tiny_bf16_p16": None,
}


@pytest.mark.slow
@pytest.mark.parametrize("spec", I.FULL, ids=lambda s: s.name)
def test_full_size_sampled_parity_and_poison(spec):
    case = I.make_case(spec)
    out, plan = run(case)
    seqs = list(range(case.num_seqs)) if case.num_seqs <= 4 else [0, 1, case.num_seqs // 2, case.num_seqs - 1]
    ref = oracle.pa_decode(case, seqs=seqs)
    check_parity(out, ref, seqs=seqs, what=spec.name + " (sampled)")
    assert torch.isfinite(out.float()).all()
    zero = run(I.refill(case, "zero"))[0]
    assert torch.equal(zero.view(torch.int16), out.view(torch.int16)), "poisoned != zero-filled at full size"


@pytest.mark.parametrize("spec", [s for s in SMALL if s.kv_dtype == "mxfp4"] +
                         [s for s in I.FULL if s.kv_dtype == "mxfp4"], ids=lambda s: s.name)
def test_mxfp4_scaled_qk_mode(spec):
    """The opt-in block-scaled fp4 x fp8 MFMA QK on every MXFP4 workload (full
    sizes on sampled sequences): the full bar, finite, poison invariant."""
    case = I.make_case(spec)
    seqs = None if case.num_seqs <= 4 else [0, 1, case.num_seqs // 2, case.num_seqs - 1]
    out, _ = run(case, mxfp4_scaled_qk=1)
    check_parity(out, oracle.pa_decode(case, seqs=seqs), seqs=seqs, what=spec.name + " scaled QK")
    zero = run(I.refill(case, "zero"), mxfp4_scaled_qk=1)[0]
    assert torch.equal(zero.view(torch.int16), out.view(torch.int16))


def test_mxfp4_scaled_qk_near_tie_exceeds_the_element_bound():
    """Why the scaled QK is opt-in: on the edge-length batch (bf16 query) one
    row's top logits nearly tie, and the instruction's block-sum error (see
    test_gpu_scaled_mfma_numerics) moves an element past 2e-2 * max(1, |o|),
    while rel-L2 stays within its bar; the default exact QK meets both."""
    spec = I.MXFP4_SHORT_QBF.replace(name="mxfp4_edges", num_seqs=len(EDGE_LENS), lens=("fixed", EDGE_LENS),
                                     num_kv_heads=2)
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    check_parity(run(case)[0], ref, what="exact QK")
    rel, worst, finite = parity_stats(run(case, mxfp4_scaled_qk=1)[0], ref)
    print("scaled QK: rel-L2 %.3e, worst |err|/bound %.3f" % (rel, worst))
    assert finite and rel <= REL_L2 and worst > 1.0


@pytest.mark.parametrize("scaled", [0, 1], ids=["exact_qk", "scaled_qk"])
@pytest.mark.parametrize("spec", [I.MXFP4_SPREAD_Q8, I.MXFP4_SPREAD_QBF], ids=lambda s: s.name)
def test_mxfp4_spread_softmax(spec, scaled):
    """MXFP4 with K scale bytes in [122, 127]: logits of order 1, so the
    softmax spreads over many tokens instead of being one-hot, and every step
    (the weights, their bf16 hi + lo parts, the weighted V sum, the partition
    merge) shows in the output. Full size (16 sequences x 2048 tokens x 4 KV
    heads), every sequence against the oracle, planned, split and plan-free,
    with both QK forms; poison invariant."""
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    out, _ = run(case, mxfp4_scaled_qk=scaled)
    check_parity(out, ref, what=spec.name + (" scaled QK" if scaled else ""))
    many, _ = run(case, mxfp4_scaled_qk=scaled, task_budget=100000)
    check_parity(many, ref, what=spec.name + " many partitions")
    if not scaled:
        check_parity(run_direct(case), ref, what=spec.name + " plan-free")
    zero = run(I.refill(case, "zero"), mxfp4_scaled_qk=scaled)[0]
    assert torch.equal(zero.view(torch.int16), out.view(torch.int16))


# ------------------------------------------------------------- plan-free path

def run_direct(case, fill_out=float("nan")):
    """pa_decode_direct on a Case (no plan); returns the bf16 output."""
    d = B.device_tensors(case)
    out = torch.full((case.num_seqs, case.qlen, case.num_q_heads, case.head_dim), fill_out, dtype=torch.bfloat16,
                     device="cuda")
    B.pa_decode_direct(B.problem_of(case), d["query"], d["key_cache"], d["value_cache"], d["k_scale"], d["v_scale"],
                       d["block_tables"], d["context_lens"], out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_plan_free_equals_one_partition_plan_and_oracle(spec):
    """The plan-free decode is bitwise equal to a plan with one partition per
    sequence (ROCm/aiter PR #7056, "Bandwidth") and meets the parity bar."""
    case = I.make_case(spec)
    direct = run_direct(case)
    planned, plan = run(case, max_partitions=1)
    assert plan.info().merge_needed == 0
    assert torch.equal(direct.view(torch.int16), planned.view(torch.int16))
    check_parity(direct, oracle.pa_decode(case), what=spec.name + " plan-free")


@pytest.mark.parametrize("base", [I.TINY_BF16, I.BF16_P64, I.FP8TOK_Q1, I.FP8TOK_Q4, I.FP8_TRANS, I.MXFP4_SHORT_QBF],
                         ids=lambda s: s.name)
def test_plan_free_edge_lengths_and_poison(base):
    spec = base.replace(name=base.name + "_edges", num_seqs=len(EDGE_LENS), lens=("fixed", EDGE_LENS),
                        num_kv_heads=min(base.num_kv_heads, 2))
    case = I.make_case(spec, fill="zero")
    out = run_direct(case)
    check_parity(out, oracle.pa_decode(case), what=spec.name + " plan-free")
    assert torch.all(out[0].float().cpu() == 0)  # L = 0 rows are written as zeros
    for fill in ("nan", "inf", "random"):
        assert torch.equal(run_direct(I.refill(case, fill)).view(torch.int16), out.view(torch.int16)), fill


@pytest.mark.slow
@pytest.mark.parametrize("spec", I.FULL, ids=lambda s: s.name)
def test_plan_free_full_size(spec):
    case = I.make_case(spec)
    out = run_direct(case)
    seqs = list(range(case.num_seqs)) if case.num_seqs <= 4 else [0, 1, case.num_seqs // 2, case.num_seqs - 1]
    check_parity(out, oracle.pa_decode(case, seqs=seqs), seqs=seqs, what=spec.name + " plan-free (sampled)")
    planned, _ = run(case, max_partitions=1)
    assert torch.equal(out.view(torch.int16), planned.view(torch.int16))


# ------------------------------------------------ causal and sliding window

GPU_MASK_SPECS = [
    I.Spec("g_bf16_q4_causal", 4, ("fixed", (1, 6, 300, 1030)), 4, 2, 2, 128, 16, "bf16", seed=41, causal=1),
    I.Spec("g_bf16_q2_win", 4, ("fixed", (2, 70, 700, 1500)), 2, 1, 4, 128, 64, "bf16", seed=42, window=300),
    I.Spec("g_fp8tok_q4_causal_win", 3, ("fixed", (257, 600, 1400)), 4, 1, 4, 256, 16, "fp8", "token", seed=43,
           causal=1, window=500),
    I.Spec("g_fp8trans_win", 3, ("fixed", (129, 513, 2000)), 1, 1, 8, 128, 128, "fp8", "tensor", "trans", seed=44,
           window=700),
    I.Spec("g_bf16_q2_causal_w1", 2, ("fixed", (1, 40)), 2, 1, 2, 128, 16, "bf16", seed=45, causal=1, window=1),
    I.Spec("g_bf16_p128_w256", 3, ("fixed", (255, 256, 2049)), 1, 2, 8, 128, 128, "bf16", seed=46, window=256),
    I.Spec("g_bf16_q4_g8_causal_win", 3, ("fixed", (3, 511, 1300)), 4, 1, 8, 128, 64, "bf16", seed=47, causal=1,
           window=257),
    # fp8 per-token caches with 16 query rows, head_dim 128 and 256, pages of
    # 64 and 128 tokens: the whole-stage-prefetch instances
    I.Spec("g_fp8tok_d128_p64_win", 3, ("fixed", (65, 700, 2100)), 1, 2, 8, 128, 64, "fp8", "token", seed=48,
           window=600),
    I.Spec("g_fp8tok_d256_p128_q2_causal", 3, ("fixed", (1, 383, 1800)), 2, 1, 8, 256, 128, "fp8", "token",
           seed=49, causal=1),
    # causal rows without a window on fp8 per-token caches (the causal-only
    # instances): lengths whose earliest row ends in the tile before the last
    # (L mod 256 in 1 .. qlen - 1), with 32 rows (two N tiles) at head_dim 256,
    # 16 rows (one N tile, whole-stage prefetch), and transposed V
    I.Spec("g_fp8tok_d256_p16_q4_causal_edges", 10, ("fixed", (1, 2, 3, 4, 257, 258, 259, 513, 1027, 767)), 4, 2,
           8, 256, 16, "fp8", "token", seed=54, causal=1),
    I.Spec("g_fp8tok_d256_p16_q2_causal_edges", 5, ("fixed", (1, 2, 257, 1025, 600)), 2, 1, 8, 256, 16, "fp8",
           "token", seed=55, causal=1),
    I.Spec("g_fp8tok_trans_d128_p64_q4_causal", 3, ("fixed", (3, 258, 700)), 4, 1, 4, 128, 64, "fp8", "token",
           "trans", seed=56, causal=1),
    # fp8 per-token caches with 32 query rows at head_dim 256 on the V-by-DMA
    # path (query fragments in LDS): page 64 plain, page 128 causal + window
    I.Spec("g_fp8tok_d256_p64_q4", 3, ("fixed", (2, 900, 2100)), 4, 1, 8, 256, 64, "fp8", "token", seed=50),
    # whole-stage prefetch, no mask rows: page 64 qlen 1, page 128 qlen 2 (16 rows)
    I.Spec("g_fp8tok_d256_p64_q1", 3, ("fixed", (63, 1025, 2300)), 1, 2, 8, 256, 64, "fp8", "token", seed=52),
    I.Spec("g_fp8tok_d256_p128_q2", 3, ("fixed", (128, 257, 1900)), 2, 1, 8, 256, 128, "fp8", "token", seed=53),
    I.Spec("g_fp8tok_d256_p128_q4_causal_win", 3, ("fixed", (3, 700, 2000)), 4, 1, 8, 256, 128, "fp8", "token",
           seed=51, causal=1, window=600),
]


@pytest.mark.parametrize("spec", GPU_MASK_SPECS, ids=lambda s: s.name)
def test_masked_rows_agree_with_oracle(spec):
    """Causal and windowed rows, planned (automatic and split into many
    partitions) and plan-free, against the oracle; poison bit-identity."""
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    out, _ = run(case)
    check_parity(out, ref, what=spec.name)
    many, _ = run(case, task_budget=100000)
    check_parity(many, ref, what=spec.name + " many partitions")
    direct = run_direct(case)
    check_parity(direct, ref, what=spec.name + " plan-free")
    one, _ = run(case, max_partitions=1)
    assert torch.equal(direct.view(torch.int16), one.view(torch.int16))
    zero = run(I.refill(case, "zero"))[0]
    assert torch.equal(zero.view(torch.int16), out.view(torch.int16))
    # rows whose range is empty (causal with L < qlen) are written as zeros
    ref_zero = np.all(ref == 0, axis=-1)
    assert torch.all(out.float().cpu()[torch.from_numpy(ref_zero)] == 0)


def test_mxfp4_refuses_a_window():
    case = I.make_case(I.small(I.MXFP4_SHORT_QBF))
    with pytest.raises(B.PaError) as ei:
        B.pa_plan(B.problem_of(case, window=128), case.context_lens)
    assert ei.value.status == B.PA_ERR_UNSUPPORTED


WINDOW_SPECS = [s for s in GPU_MASK_SPECS if s.window > 0]


def _decode_modes(case):
    """The planned decode (automatic and split into many partitions) and the
    plan-free decode of a case."""
    return {"auto": run(case)[0], "many": run(case, task_budget=100000)[0], "direct": run_direct(case)}


@pytest.mark.parametrize("spec", WINDOW_SPECS, ids=lambda s: s.name)
def test_prewindow_rows_and_columns_are_inert(spec):
    """A caller that frees the pages a sliding window has left behind points
    their table columns at block 0 and leaves garbage in the earlier rows of
    the window's first page. Those rows and their per-token scales hold NaN,
    Inf or random bytes here; the output must stay finite and bit-identical to
    the zero-filled run with the original table (ROCm/aiter PR #7092, "Tests":
    the wider probe's sliding-window shapes under NaN / Inf / random fills)."""
    case = I.make_case(spec, fill="zero")
    base = _decode_modes(case)
    ref = oracle.pa_decode(case)
    for fill in ("nan", "inf", "random"):
        pc = I.poison_prewindow(case, fill)
        got = _decode_modes(pc)
        for mode, out in got.items():
            assert torch.isfinite(out.float()).all(), "%s %s: non-finite output" % (fill, mode)
            assert torch.equal(out.view(torch.int16), base[mode].view(torch.int16)), \
                "%s %s: pre-window fill changes the output" % (fill, mode)
    check_parity(base["auto"], ref, what=spec.name)


@pytest.mark.slow
def test_prewindow_rows_are_inert_at_full_size():
    """The same contract on the full-size 1024-token window workload."""
    case = I.make_case(I.BF16_P64_W1024, fill="zero")
    base = run(case)[0]
    for fill in ("nan", "random"):
        out = run(I.poison_prewindow(case, fill))[0]
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out.view(torch.int16), base.view(torch.int16)), fill


@pytest.mark.parametrize("spec", [s for s in WINDOW_SPECS if s.name in (
    "g_bf16_q2_win", "g_fp8tok_q4_causal_win", "g_fp8trans_win", "g_fp8tok_d256_p128_q4_causal_win")],
    ids=lambda s: s.name)
def test_window_plan_with_shorter_device_lengths(spec):
    """A plan made from host lengths, decoded with shorter device lengths: the
    device window starts earlier than the planned one, and its tiles must
    still be read (pa_plan: device lengths may be equal or shorter)."""
    case = I.make_case(spec)
    host = case.context_lens.clone()
    for cut in (1, 37, 300, 1000):
        short = dataclasses.replace(case, context_lens=(host - cut).clamp(min=0).to(torch.int32))
        ref = oracle.pa_decode(short)
        for over in ({}, {"task_budget": 100000}):
            plan = B.pa_plan(B.problem_of(case, **over), host)
            out, _ = B.decode_case(short, plan=plan)
            torch.cuda.synchronize()
            check_parity(out, ref, what="%s cut %d %s" % (spec.name, cut, over))


# Transposed V ([D][page] per page and head) with one N tile at head_dim 128, at every page size, for
# bf16 and fp8 per-tensor caches: the instances whose K goes by whole-line loads and a lane exchange
# (and, at page 128 fp8, the transposed-V workload's). Ragged lengths with partial first and last
# pages, planned (automatic and one tile per task), plan-free, and with poisoned unowned rows.
VT_SPECS = [
    I.Spec("g_%s_trans_p%d" % (kv, pg), 6, ("fixed", (1, 17, 63, 300, 777, 1300)), 1, 2, 8, 128, pg, kv,
           "tensor" if kv == "fp8" else "none", "trans", seed=70 + 3 * i + j)
    for i, kv in enumerate(("bf16", "fp8")) for j, pg in enumerate((16, 64, 128))
] + [
    I.Spec("g_%s_trans_p%d_q2_causal" % (kv, pg), 4, ("fixed", (2, 65, 700, 1025)), 2, 1, 8, 128, pg, kv,
           "tensor" if kv == "fp8" else "none", "trans", seed=80 + j, causal=1)
    for j, (kv, pg) in enumerate((("bf16", 16), ("fp8", 64)))
]


@pytest.mark.parametrize("spec", VT_SPECS, ids=lambda s: s.name)
def test_transposed_v_page_sizes(spec):
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    for over in ({}, {"task_budget": 100000}):
        out, _ = run(case, **over)
        check_parity(out, ref, what="%s %s" % (spec.name, over))
    check_parity(run_direct(case), ref, what="%s plan-free" % spec.name)
    zero = I.make_case(spec, fill="zero")
    ref_bits = _bits(run(zero)[0])
    for fill in ("nan", "random"):
        assert np.array_equal(_bits(run(I.refill(zero, fill))[0]), ref_bits), "%s: %s fill" % (spec.name, fill)
