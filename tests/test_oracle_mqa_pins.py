"""Pins of the oracle's MXFP4 paged MQA logits against facts that are not the oracle.

What fixes each expected value:
  - a brute-force dense implementation written here with numpy (decode q and
    the window's K rows with the e2m1 table of the OCP MX specification,
    tests/golden/e2m1_ocp_mx.txt, then weights . relu(q K^T));
  - closed forms: q equal to a K row gives its squared norm, q equal to the
    negated row gives exactly zero;
  - invariants: scaling the weights scales the scores, page relabelling changes
    nothing, positions outside a window and pad rows are never written;
  - NaN in an e8m0 scale reaches exactly the positions that read it.
A negative control checks that dropping the relu is caught.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_token_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1():
    vals = {}
    for line in open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")):
        if line.strip() and not line.startswith("#"):
            c, v = line.split()
            vals[int(c)] = float(v)
    return np.array([vals[c & 7] * (-1 if c & 8 else 1) for c in range(16)])


E2M1 = _e2m1()


def _deq(data, scale):
    """u8 [..., D/2] data and u8 [..., D/32] scales -> fp64 [..., D]."""
    data = np.asarray(data, dtype=np.uint8)
    lo, hi = E2M1[data & 0xF], E2M1[data >> 4]
    x = np.stack([lo, hi], axis=-1).reshape(*data.shape[:-1], data.shape[-1] * 2)
    sc = np.asarray(scale, dtype=np.int64)
    f = np.where(sc == 255, np.nan, np.exp2(sc.astype(np.float64) - 127))
    return x * np.repeat(f, 32, axis=-1)


def dense(case, relu=True):
    """Scores at every window position, NaN elsewhere."""
    out = np.full((case.num_rows, case.out_stride), np.nan)
    q = _deq(case.q.numpy(), case.q_scale.numpy())  # [R, H, D]
    kc = _deq(case.k_cache.numpy(), case.k_scale.numpy())  # [NB, PG, D]
    w = case.weights.double().numpy()
    PG = case.page_size
    for r in range(case.num_rows):
        b = int(case.row_to_batch[r])
        if b < 0 or b >= case.num_seqs:
            continue
        t0 = max(int(case.local_starts[r]), 0)
        t1 = min(int(case.local_ends[r]), case.max_blocks_per_seq * PG, case.out_stride)
        if t1 <= t0:
            continue
        t = np.arange(t0, t1)
        pages = case.block_tables[b].numpy()[t // PG]
        K = kc[pages, t % PG]  # [T, D]
        s = q[r] @ K.T  # [H, T]
        if relu:
            s = np.where(s < 0, 0.0, s)
        out[r, t0:t1] = w[r] @ s
    return out


SPECS = [I.small_mqa(s) for s in I.MQA_FULL] + [
    I.small_mqa(I.MQA_DECODE_LONG).replace(name="h16_d64_p16", num_heads=16, head_dim=64, page_size=16, seed=5),
    I.small_mqa(I.MQA_DECODE_LONG).replace(name="h32_p128_rows3", num_heads=32, page_size=128, rows_per_seq=3,
                                           seed=6),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_oracle_matches_dense_brute_force(spec):
    case = I.make_mqa_case(spec)
    got, mag = oracle.mqa_logits_mxfp4(case)
    ref = dense(case)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.all(np.abs(got[m] - ref[m]) <= 1e-12 * mag[m])
    assert np.all(mag[m] >= np.abs(got[m]))


def _one_row_case(q_equals_k_sign):
    spec = I.MqaSpec("closed", 1, ("fixed", (40,)), 1, 1, 128, 16, seed=9)
    case = I.make_mqa_case(spec)
    t = 17
    page = int(case.block_tables[0, t // 16])
    kd = case.k_cache[page, t % 16].clone()
    ks = case.k_scale[page, t % 16].clone()
    qd = kd if q_equals_k_sign > 0 else kd ^ 0x88  # flip every sign bit
    case = dataclasses.replace(case, q=qd.view(1, 1, 64).clone(), q_scale=ks.view(1, 1, 4).clone(),
                               weights=torch.ones((1, 1)))
    return case, t, _deq(kd.numpy(), ks.numpy())


def test_query_equal_to_a_key_gives_its_squared_norm():
    case, t, k = _one_row_case(+1)
    got, _ = oracle.mqa_logits_mxfp4(case)
    assert got[0, t] == pytest.approx(float(np.dot(k, k)), rel=1e-15)


def test_query_opposite_to_a_key_gives_zero():
    case, t, _ = _one_row_case(-1)
    got, _ = oracle.mqa_logits_mxfp4(case)
    assert got[0, t] == 0.0


def test_scores_scale_with_the_weights():
    case = I.make_mqa_case(SPECS[0])
    a, _ = oracle.mqa_logits_mxfp4(case)
    b, _ = oracle.mqa_logits_mxfp4(dataclasses.replace(case, weights=case.weights * 2))
    m = ~np.isnan(a)
    assert np.array_equal(b[m], 2 * a[m])


def test_windows_and_pad_rows_bound_the_writes():
    case = I.make_mqa_case(SPECS[1])
    got, _ = oracle.mqa_logits_mxfp4(case, fill=-np.inf)
    for r in range(case.num_rows):
        b, s, e = int(case.row_to_batch[r]), int(case.local_starts[r]), int(case.local_ends[r])
        written = ~np.isneginf(got[r])
        if b < 0:
            assert not written.any()
        else:
            assert np.array_equal(np.nonzero(written)[0], np.arange(max(s, 0), e))


def test_page_relabelling_changes_nothing():
    case = I.make_mqa_case(SPECS[0])
    a, _ = oracle.mqa_logits_mxfp4(case)
    g = torch.Generator().manual_seed(3)
    perm = torch.randperm(case.num_blocks, generator=g)
    inv = torch.argsort(perm)
    relabeled = dataclasses.replace(case, k_cache=case.k_cache[inv], k_scale=case.k_scale[inv],
                                    block_tables=perm[case.block_tables.long()].to(torch.int32))
    b, _ = oracle.mqa_logits_mxfp4(relabeled)
    assert np.array_equal(a, b, equal_nan=True)


def test_nan_scale_reaches_exactly_its_position():
    case = I.make_mqa_case(SPECS[0])
    t = 250
    b = 3
    page = int(case.block_tables[b, t // case.page_size])
    ks = case.k_scale.clone()
    ks[page, t % case.page_size, 1] = 0xFF
    a, _ = oracle.mqa_logits_mxfp4(case)
    got, _ = oracle.mqa_logits_mxfp4(dataclasses.replace(case, k_scale=ks))
    rows = [r for r in range(case.num_rows) if int(case.row_to_batch[r]) == b and int(case.local_ends[r]) > t]
    assert rows
    for r in range(case.num_rows):
        if r in rows:
            assert np.isnan(got[r, t])
            got[r, t] = a[r, t]
    assert np.array_equal(a, got, equal_nan=True)


def test_negative_control_without_relu_is_caught():
    case = I.make_mqa_case(SPECS[0])
    got, mag = oracle.mqa_logits_mxfp4(case)
    wrong = dense(case, relu=False)
    m = ~np.isnan(got)
    assert np.any(np.abs(got[m] - wrong[m]) > 1e-6 * mag[m])


def test_block_table_entry_outside_the_pool_is_refused():
    case = I.make_mqa_case(SPECS[0])
    bt = case.block_tables.clone()
    bt[3, 0] = case.num_blocks
    with pytest.raises(ValueError):
        oracle.mqa_logits_mxfp4(dataclasses.replace(case, block_tables=bt))
