"""GPU parity of the MXFP4 paged MQA logits: the HIP kernel through the C ABI
against the fp64 oracle.

Bar, from the arithmetic: every score is a sum of num_heads weighted products,
each product an exact MFMA block sum, accumulated in fp32; the rounding error is
at most about num_heads * 2^-24 times mag = sum_h |w_h| * sum_d |qhat * khat|,
which the oracle reports per position. The test allows 1e-5 * mag (2.5 times
that bound at 64 heads). NaN must appear exactly where the oracle has it, and
every position outside a window must keep the caller's bytes.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_token_amd import binding as B
from paged_attention_decode_token_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()  # raises when libpa.so is missing


def run(case, fill=float("-inf")):
    d = {k: getattr(case, k).cuda() for k in ("q", "q_scale", "weights", "k_cache", "k_scale", "block_tables",
                                               "row_to_batch", "local_starts", "local_ends")}
    out = torch.full((case.num_rows, case.out_stride), fill, dtype=torch.float32, device="cuda")
    B.pa_mqa_logits_mxfp4(B.mqa_problem_of(case), d["q"], d["q_scale"], d["weights"], d["k_cache"], d["k_scale"],
                          d["block_tables"], d["row_to_batch"], d["local_starts"], d["local_ends"], out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(got, case, what):
    ref, mag = oracle.mqa_logits_mxfp4(case, fill=float("-inf"))
    outside = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), outside), "%s: writes outside the windows" % what
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "%s: NaN positions differ" % what
    m = ~outside & ~np.isnan(ref)
    err = np.abs(got[m].astype(np.float64) - ref[m])
    worst = float((err / np.maximum(TOL * mag[m], 1e-300)).max()) if m.any() else 0.0
    print("%s: %d positions, worst |err| / (%.0e mag) = %.3f" % (what, int(m.sum()), TOL, worst))
    assert worst <= 1.0, "%s: error %.3f x bound" % (what, worst)


SMALL = [I.small_mqa(s) for s in I.MQA_FULL] + [
    I.small_mqa(I.MQA_DECODE_LONG).replace(name="h16_p16", num_heads=16, page_size=16, seed=5),
    I.small_mqa(I.MQA_DECODE_LONG).replace(name="h32_p128_rows3", num_heads=32, page_size=128, rows_per_seq=3,
                                           seed=6),
    I.small_mqa(I.MQA_DECODE_LONG).replace(name="h128_p48_rows2", num_heads=128, page_size=48, rows_per_seq=2,
                                           seed=7),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_matches_oracle(spec):
    case = I.make_mqa_case(spec)
    print("mqa parity", spec.name, "rows", case.num_rows, flush=True)
    check(run(case), case, spec.name)


def test_unowned_rows_do_not_leak():
    spec = I.small_mqa(I.MQA_MTP2).replace(name="leak", seed=31)
    a = run(I.make_mqa_case(spec))
    b = run(I.make_mqa_case(spec.replace(fill="random")))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_windows_with_offsets_and_pad_rows():
    case = I.make_mqa_case(I.small_mqa(I.MQA_MTP2).replace(name="offsets", seed=32))
    g = torch.Generator().manual_seed(4)
    ends = case.local_ends.clone()
    starts = torch.minimum(torch.randint(0, 200, ends.shape, generator=g, dtype=torch.int32), ends)
    starts[0] = -5  # clamped to 0
    rtb = case.row_to_batch.clone()
    rtb[1] = case.num_seqs  # out of range: a pad row
    case = dataclasses.replace(case, local_starts=starts, row_to_batch=rtb)
    check(run(case), case, "offsets")


def test_nan_scale_reaches_exactly_its_positions():
    case = I.make_mqa_case(I.small_mqa(I.MQA_DECODE_LONG).replace(name="nan", seed=33))
    ks = case.k_scale.clone()
    for b, t in ((3, 250), (2, 17), (3, 1029)):
        page = int(case.block_tables[b, t // case.page_size])
        ks[page, t % case.page_size, 2] = 0xFF
    case = dataclasses.replace(case, k_scale=ks)
    got = run(case)
    assert np.isnan(got).sum() >= 3
    check(got, case, "nan scales")


def test_bad_table_entries_past_the_windows_cannot_fault():
    case = I.make_mqa_case(I.small_mqa(I.MQA_DECODE_LONG).replace(name="badtable", seed=34))
    bt = case.block_tables.clone()
    for b in range(case.num_seqs):
        used = (int(case.context_lens[b]) + case.page_size - 1) // case.page_size
        bt[b, used:] = torch.tensor([2 ** 31 - 1, -7], dtype=torch.int32).repeat(bt.shape[1])[:bt.shape[1] - used]
    a = run(case)
    b = run(dataclasses.replace(case, block_tables=bt))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_deterministic():
    case = I.make_mqa_case(I.small_mqa(I.MQA_MTP2).replace(name="det", seed=35))
    assert np.array_equal(run(case).view(np.uint32), run(case).view(np.uint32))


@pytest.mark.slow
@pytest.mark.parametrize("spec", I.MQA_FULL, ids=lambda s: s.name)
def test_full_size_sampled(spec):
    case = I.make_mqa_case(spec, device="cuda")
    print("mqa full size", spec.name, "rows", case.num_rows, flush=True)
    out = torch.full((case.num_rows, case.out_stride), float("-inf"), dtype=torch.float32, device="cuda")
    B.pa_mqa_logits_mxfp4(B.mqa_problem_of(case), case.q, case.q_scale, case.weights, case.k_cache, case.k_scale,
                          case.block_tables, case.row_to_batch, case.local_starts, case.local_ends, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # at any size: every window position written and finite, nothing else written
    ends = case.local_ends.cpu().numpy()
    rtb = case.row_to_batch.cpu().numpy()
    pos = np.arange(case.out_stride)[None, :]
    inside = (pos < ends[:, None]) & (rtb[:, None] >= 0)
    assert np.isfinite(got[inside]).all()
    assert np.isneginf(got[~inside]).all()
    # sampled: the oracle on 512-position sub-windows of every live row
    host = dataclasses.replace(case, **{k: getattr(case, k).cpu() for k in (
        "q", "q_scale", "weights", "k_cache", "k_scale", "block_tables", "row_to_batch", "local_starts",
        "local_ends")})
    g = torch.Generator().manual_seed(6)
    starts = torch.zeros_like(host.local_starts)
    sub_ends = torch.zeros_like(host.local_ends)
    for r in range(case.num_rows):
        e = int(host.local_ends[r])
        if rtb[r] >= 0 and e > 0:
            s0 = int(torch.randint(0, max(e - 512, 0) + 1, (1,), generator=g))
            starts[r], sub_ends[r] = s0, min(s0 + 512, e)
    sub = dataclasses.replace(host, local_starts=starts, local_ends=sub_ends)
    ref, mag = oracle.mqa_logits_mxfp4(sub, fill=float("-inf"))
    m = ~np.isneginf(ref)
    assert m.sum() > 0
    err = np.abs(got[m].astype(np.float64) - ref[m])
    worst = float((err / (TOL * mag[m])).max())
    print("sampled %d positions, worst %.3f" % (int(m.sum()), worst))
    assert worst <= 1.0
