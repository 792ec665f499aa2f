"""Negative controls for the GPU parity checker, on the CPU.

The bar the GPU tests apply (parity_bar.check_parity) must pass an output that
differs from the fp64 oracle only by bf16 output rounding, and must fail each
deliberate break the pages show their own checker catching (ROCm/aiter
PR #7056, "Validation and unverified scope"): one element off by 0.05, one
NaN, V dequantized with a wrong value scale, and MXFP4 K block scales rolled
by one position. The broken outputs are the oracle's own results on broken
inputs, rounded to bf16 like a GPU output.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_token_amd import inputs as I
from parity_bar import check_parity, parity_stats

FP8_TENSOR = I.small(I.FP8_TRANS)
MXFP4 = I.small(I.MXFP4_SHORT_Q8)
CASES = [I.small(I.BF16_P64), FP8_TENSOR, I.small(I.FP8TOK_Q1), MXFP4]


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def _fails(got, ref):
    rel, worst, finite = parity_stats(got, ref)
    return (not finite) or rel > 3e-3 or worst > 1.0


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_bf16_rounded_oracle_passes(spec):
    ref = oracle.pa_decode(I.make_case(spec))
    check_parity(_bf16(ref), ref, what=spec.name + " bf16(oracle)")


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_one_element_off_by_005_fails(spec):
    ref = oracle.pa_decode(I.make_case(spec))
    got = _bf16(ref).double().numpy()
    idx = np.unravel_index(np.argmin(np.abs(ref) + (ref == 0) * 1e9), ref.shape)  # a nonzero element with |o| <= 1
    assert abs(ref[idx]) <= 1.0
    got[idx] += 0.05
    assert _fails(got, ref)


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_one_nan_fails(spec):
    ref = oracle.pa_decode(I.make_case(spec))
    got = _bf16(ref).double().numpy()
    got.flat[got.size // 2] = np.nan
    assert _fails(got, ref)


@pytest.mark.parametrize("spec", [FP8_TENSOR, I.small(I.FP8TOK_Q4)], ids=lambda s: s.name)
def test_wrong_value_scale_fails(spec):
    """V dequantized with v_scale x 1.05 (per-tensor or per-token)."""
    case = I.make_case(spec)
    ref = oracle.pa_decode(case)
    wrong = dataclasses.replace(case, v_scale=case.v_scale * 1.05)
    assert _fails(_bf16(oracle.pa_decode(wrong)), ref)


def test_rolled_mxfp4_k_block_scales_fail():
    """Each K row's four e8m0 block scales rolled by one position."""
    case = I.make_case(MXFP4)
    ref = oracle.pa_decode(case)
    wrong = dataclasses.replace(case, k_scale=torch.roll(case.k_scale, 1, dims=-1).contiguous())
    assert _fails(_bf16(oracle.pa_decode(wrong)), ref)
