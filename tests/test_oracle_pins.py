"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value:
  - library casts (torch's bfloat16 / float8_e4m3fn / float8_e8m0fnu conversions),
  - format tables printed in specifications (tests/golden/*.txt, cited there),
  - closed forms of attention (constant V, one key, identical keys, one token),
  - a brute-force dense implementation written here with numpy and torch
    (gather every owned row, then softmax(q K^T) V) on tiny inputs,
  - algebraic invariants (log-sum-exp split/merge, page relabelling, poison fills).
Negative controls check that a plausible mistake in the reference (wrong GQA
grouping, scale off by 5 %, transposed V read as plain) is caught.
"""
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_token_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    tab = np.zeros(16)
    for c in range(8):
        tab[c] = vals[c]
        tab[c | 8] = -vals[c]
    return tab


# ------------------------------------------------------------------ decoders

def test_bf16_decoder_matches_torch_all_codes():
    codes = np.arange(65536, dtype=np.int64)
    ref = torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(c) for c in codes[::7]])
    r = ref[::7]
    assert np.array_equal(np.isnan(got), np.isnan(r))
    m = ~np.isnan(r)
    assert np.array_equal(got[m], r[m])


def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_f64(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    # specials: largest finite, smallest normal, smallest subnormal
    assert oracle.e4m3_to_f64(0x7E) == 448.0
    assert oracle.e4m3_to_f64(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_f64(0x01) == 2.0 ** -9


def test_e8m0_decoder_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0_to_f64(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])


def test_e2m1_decoder_matches_spec_table():
    tab = _e2m1_table()
    got = np.array([oracle.e2m1_to_f64(c) for c in range(16)])
    assert np.array_equal(got, tab)


def test_format_facts_from_the_pages():
    with open(os.path.join(GOLDEN, "format_facts.txt")) as f:
        for line in f:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            if p[0] == "e4m3":
                v = oracle.e4m3_to_f64(int(p[1], 16))
            elif p[0] == "e8m0":
                v = oracle.e8m0_to_f64(int(p[1], 16))
            else:
                continue
            if p[2] == "nan":
                assert math.isnan(v), line
            else:
                assert v == float(p[2]), line


def test_bf16_rne_matches_torch_on_float32_values():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(4000, generator=g, dtype=torch.float32) * torch.exp2(torch.randint(-20, 20, (4000,), generator=g)
                                                                          .float())
    # include exact ties: bf16 midpoints
    ties = (torch.arange(1, 200, dtype=torch.int32) << 16 | 0x8000).view(torch.float32)
    x = torch.cat([x, ties, -ties])
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in x.numpy()], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_e4m3_rne_matches_torch_in_range():
    g = torch.Generator().manual_seed(6)
    x = (torch.rand(3000, generator=g) * 2 - 1) * 448
    x = torch.cat([x, torch.randn(1000, generator=g) * 0.01])
    # exact midpoints between neighbouring e4m3 values (ties to even)
    vals = torch.arange(0, 0x7E, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float()
    mids = (vals[:-1] + vals[1:]) / 2
    x = torch.cat([x, mids, -mids])
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f64_to_e4m3(float(v)) for v in x.numpy()], dtype=np.uint8)
    assert np.array_equal(got, ref)
    assert oracle.f64_to_e4m3(1000.0) == 0x7E and oracle.f64_to_e4m3(-500.0) == 0xFE  # saturation


def test_q_row_exponent_closed_form():
    # smallest e with amax <= 448 * 2^e
    assert oracle.q_row_exponent(448.0) == 0
    assert oracle.q_row_exponent(448.0 * (1 + 2 ** -20)) == 1
    assert oracle.q_row_exponent(224.0) == -1
    assert oracle.q_row_exponent(1.0) == -8  # 448/256 = 1.75 >= 1 > 448/512
    assert oracle.q_row_exponent(0.0) == 0
    for a in [1e-3, 0.37, 3.9, 17.0, 1e5]:
        e = oracle.q_row_exponent(a)
        assert a <= 448 * 2.0 ** e and a > 448 * 2.0 ** (e - 1)


# ------------------------------------------------------- brute-force dense

def _deq_rows(case, cache, scale, pages, kvh, transposed, mx_scale=None, nibble_swap=False):
    """[npages*page, D] fp64 rows of one head (torch casts, the spec table)."""
    D, PG = case.head_dim, case.page_size
    c = cache[pages.long(), kvh]
    if case.kv_dtype == "mxfp4":
        tab = _e2m1_table()
        data = c.numpy().astype(np.int64)  # [n, PG, D/2]
        lo, hi = (data >> 4, data & 15) if nibble_swap else (data & 15, data >> 4)
        nib = np.stack([lo, hi], axis=-1).reshape(len(pages), PG, D)
        vals = tab[nib]
        sc = mx_scale[pages.long(), kvh].numpy()  # [n, PG, D/32]
        sc = torch.from_numpy(sc).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        vals = vals * np.repeat(sc, 32, axis=-1)
        return vals.reshape(-1, D)
    if case.kv_dtype == "bf16":
        vals = c.view(torch.bfloat16).to(torch.float64).numpy()
    else:
        vals = c.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if transposed:
        vals = np.swapaxes(vals, 1, 2)
    vals = vals.reshape(-1, D)
    return vals


def dense_reference(case, gqa=lambda h, G, H: h // G, sigma_mult=1.0, v_transposed=None, nibble_swap=False,
                    causal_shift=0):
    B, QL, H, G, D, PG = case.num_seqs, case.qlen, case.num_kv_heads, case.q_per_kv, case.head_dim, case.page_size
    Hq = H * G
    sigma = sigma_mult / math.sqrt(D)
    vt = (case.v_layout == "trans") if v_transposed is None else v_transposed
    out = np.zeros((B, QL, Hq, D))
    for b in range(B):
        L = int(case.context_lens[b])
        if L == 0:
            continue
        n = (L + PG - 1) // PG
        pages = case.block_tables[b, :n]
        for i in range(QL):
            for h in range(Hq):
                kvh = gqa(h, G, H)
                K = _deq_rows(case, case.key_cache, case.k_scale, pages, kvh, False, case.k_scale, nibble_swap)[:L]
                V = _deq_rows(case, case.value_cache, case.v_scale, pages, kvh, vt, case.v_scale, nibble_swap)[:L]
                if case.kv_dtype == "fp8":
                    if case.scale_mode == "tensor":
                        K = K * float(case.k_scale[0])
                        V = V * float(case.v_scale[0])
                    else:
                        ks = case.k_scale[pages.long(), kvh].reshape(-1).double().numpy()[:L]
                        vs = case.v_scale[pages.long(), kvh].reshape(-1).double().numpy()[:L]
                        K = K * ks[:, None]
                        V = V * vs[:, None]
                if case.q_dtype == "fp8":
                    q = case.query[b, i, h].view(torch.float8_e4m3fn).to(torch.float64).numpy()
                else:
                    q = case.query[b, i, h].to(torch.float64).numpy()
                    if case.kv_dtype == "mxfp4":
                        amax = np.abs(q).max()
                        if amax > 0:
                            fr, ex = np.frexp(amax)
                            e = ex - 9 if fr <= 0.875 else ex - 8
                        else:
                            e = 0
                        q8 = torch.from_numpy(q / 2.0 ** e).to(torch.float8_e4m3fn).to(torch.float64).numpy()
                        q = q8 * 2.0 ** e
                s = (K @ q) * sigma
                # query token i sits at position L - qlen + i when causal; a
                # window keeps the last `window` positions up to and including it
                pos = np.arange(L)
                keep = np.ones(L, dtype=bool)
                last = (L - QL + i + causal_shift) if case.causal else L - 1
                if case.causal:
                    keep &= pos <= last
                if case.window > 0:
                    keep &= pos > last - case.window
                if not keep.any():
                    continue
                s = np.where(keep, s, -np.inf)
                w = np.exp(s - s[keep].max())
                out[b, i, h] = (w / w.sum()) @ V
    return out


TINY_SPECS = [
    I.Spec("t_bf16_p16", 3, ("fixed", (1, 37, 300)), 1, 2, 3, 128, 16, "bf16", seed=11),
    I.Spec("t_bf16_p64_trans", 2, ("fixed", (65, 200)), 2, 1, 4, 128, 64, "bf16", v_layout="trans", seed=12),
    I.Spec("t_bf16_d256", 2, ("fixed", (90, 17)), 1, 2, 2, 256, 16, "bf16", seed=13),
    I.Spec("t_fp8_tensor_trans", 2, ("fixed", (129, 256)), 1, 1, 4, 128, 128, "fp8", "tensor", "trans", seed=14),
    I.Spec("t_fp8_token", 3, ("fixed", (5, 48, 211)), 2, 2, 2, 256, 16, "fp8", "token", seed=15),
    I.Spec("t_fp8_token_p64", 2, ("fixed", (64, 150)), 1, 1, 8, 128, 64, "fp8", "token", seed=16),
    I.Spec("t_mxfp4_qfp8", 2, ("fixed", (130, 255)), 1, 2, 4, 128, 128, "mxfp4", q_dtype="fp8", seed=17),
    I.Spec("t_mxfp4_qbf16", 2, ("fixed", (1, 260)), 1, 1, 16, 128, 128, "mxfp4", q_dtype="bf16", seed=18),
    # K scale bytes in [122, 127]: logits of order 1, a softmax spread over many tokens
    I.Spec("t_mxfp4_qfp8_spread", 2, ("fixed", (200, 385)), 1, 2, 4, 128, 128, "mxfp4", q_dtype="fp8", seed=19,
           mx_k_scale=(122, 127)),
]


@pytest.mark.parametrize("spec", TINY_SPECS, ids=lambda s: s.name)
def test_oracle_equals_brute_force_dense(spec):
    case = I.make_case(spec)
    got = oracle.pa_decode(case)
    ref = dense_reference(case)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("spec", TINY_SPECS[:1] + TINY_SPECS[3:5] + TINY_SPECS[6:7] + TINY_SPECS[8:9],
                         ids=lambda s: s.name)
def test_negative_controls_are_caught(spec):
    """Plausible mistakes in a reference fail the brute-force comparison."""
    case = I.make_case(spec)
    got = oracle.pa_decode(case)
    if case.kv_dtype == "mxfp4":
        # a swapped nibble order is caught on any MXFP4 case; a 5 % scale error
        # only where the softmax is not one-hot (the workload recipe's scale
        # bytes put logits in the thousands)
        bad = dense_reference(case, nibble_swap=True)
        assert not np.allclose(got, bad, rtol=1e-6, atol=1e-9)
        if spec.mx_k_scale != (118, 136):
            bad_scale = dense_reference(case, sigma_mult=1.05)
            assert not np.allclose(got, bad_scale, rtol=1e-6, atol=1e-9)
    else:
        bad_scale = dense_reference(case, sigma_mult=1.05)
        assert not np.allclose(got, bad_scale, rtol=1e-6, atol=1e-9)
    if case.num_kv_heads > 1:
        bad_gqa = dense_reference(case, gqa=lambda h, G, H: h % H)
        assert not np.allclose(got, bad_gqa, rtol=1e-6, atol=1e-9)
    if case.v_layout == "trans":
        bad_v = dense_reference(case, v_transposed=False)
        assert not np.allclose(got, bad_v, rtol=1e-6, atol=1e-9)


# ------------------------------------------------------------ closed forms

def _with(case, **tensors):
    import copy
    c = copy.copy(case)
    for k, v in tensors.items():
        setattr(c, k, v)
    return c


def test_softmax_weights_sum_to_one_constant_v():
    """V = 1 everywhere (owned rows): every output element equals sum(pi) = 1."""
    case = I.make_case(TINY_SPECS[0], fill="zero")
    V = torch.full_like(case.value_cache.view(torch.int16), 0x3F80)  # bf16 1.0
    c = _with(case, value_cache=V.view(torch.bfloat16))
    out = oracle.pa_decode(c)
    L = case.context_lens.numpy()
    for b in range(case.num_seqs):
        if L[b] > 0:
            assert np.abs(out[b] - 1.0).max() < 1e-13


def test_context_len_one_gives_v_row_zero_exactly():
    for spec in [TINY_SPECS[0], TINY_SPECS[4], TINY_SPECS[6]]:
        case = I.make_case(spec.replace(lens=("fixed", tuple([1] * spec.num_seqs))))
        out = oracle.pa_decode(case)
        for b in range(case.num_seqs):
            p = case.block_tables[b, :1]
            for i in range(case.qlen):
                for h in range(case.num_q_heads):
                    kvh = h // case.q_per_kv
                    v0 = _deq_rows(case, case.value_cache, None, p, kvh, case.v_layout == "trans", case.v_scale)[0]
                    if case.kv_dtype == "fp8":
                        if case.scale_mode == "tensor":
                            v0 = v0 * float(case.v_scale[0])
                        else:
                            v0 = v0 * float(case.v_scale[int(p[0]), kvh, 0])
                    assert np.array_equal(out[b, i, h], v0)
        if spec.kv_dtype == "bf16":
            codes = oracle.bf16_round_array(out[0, 0, 0])
            ref = case.value_cache[int(case.block_tables[0, 0]), 0, 0].view(torch.int16).numpy().astype(np.uint16)
            assert np.array_equal(codes, ref)


def test_identical_keys_give_mean_of_v():
    case = I.make_case(TINY_SPECS[0], fill="zero")
    K = case.key_cache.clone()
    K[:] = K[1, :, 3:4, :]  # every row holds the same key
    c = _with(case, key_cache=K)
    out = oracle.pa_decode(c)
    for b in range(case.num_seqs):
        L = int(case.context_lens[b])
        n = (L + 15) // 16
        for h in range(case.num_q_heads):
            kvh = h // case.q_per_kv
            V = _deq_rows(case, case.value_cache, None, case.block_tables[b, :n], kvh, False)[:L]
            np.testing.assert_allclose(out[b, 0, h], V.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_one_dominant_key_selects_its_v_row():
    spec = TINY_SPECS[0].replace(lens=("fixed", (40, 40, 40)))
    case = I.make_case(spec, fill="zero")
    K = torch.zeros_like(case.key_cache)
    # token 7 of sequence 0 gets a key aligned with the query of head 0
    p = int(case.block_tables[0, 0])
    q = case.query[0, 0, 0].float()
    K[p, 0, 7] = (q * 64).to(torch.bfloat16)  # score ~ 64|q|^2/sqrt(128): far above every other (0)
    c = _with(case, key_cache=K)
    out = oracle.pa_decode(c)
    v7 = case.value_cache[p, 0, 7].to(torch.float64).numpy()
    np.testing.assert_allclose(out[0, 0, 0], v7, rtol=0, atol=1e-12)


# -------------------------------------------------------------- invariants

@pytest.mark.parametrize("spec", [TINY_SPECS[0], TINY_SPECS[4], TINY_SPECS[7]], ids=lambda s: s.name)
def test_lse_merge_of_any_split_equals_full(spec):
    case = I.make_case(spec)
    full, lse_full = oracle.pa_decode(case, with_lse=True)
    Lmax = int(case.context_lens.max())
    for cuts in ([0, 17, Lmax], [0, 1, 2, 256, Lmax], [0, Lmax // 3, 2 * Lmax // 3, Lmax]):
        parts = [oracle.pa_decode(case, t_begin=a, t_end=b, with_lse=True) for a, b in zip(cuts[:-1], cuts[1:])]
        for b in range(case.num_seqs):
            for i in range(case.qlen):
                for h in range(case.num_q_heads):
                    o = [p[0][b, i, h] for p in parts]
                    s = [p[1][b, i, h] for p in parts]
                    m, lse = oracle.lse_merge(o, s)
                    np.testing.assert_allclose(m, full[b, i, h], rtol=1e-12, atol=1e-13)
                    if case.context_lens[b] > 0:
                        assert abs(lse - lse_full[b, i, h]) < 1e-12 * max(1, abs(lse))


def test_page_relabelling_is_invisible():
    case = I.make_case(TINY_SPECS[4])
    out = oracle.pa_decode(case)
    g = torch.Generator().manual_seed(99)
    perm = torch.randperm(case.num_blocks - 1, generator=g) + 1  # new id of page p is perm[p-1]; keep block 0
    newid = torch.cat([torch.zeros(1, dtype=torch.long), perm])
    inv = torch.empty_like(newid)
    inv[newid] = torch.arange(case.num_blocks)
    c = _with(case, key_cache=case.key_cache[inv], value_cache=case.value_cache[inv], k_scale=case.k_scale[inv],
              v_scale=case.v_scale[inv], block_tables=newid[case.block_tables.long()].to(torch.int32))
    out2 = oracle.pa_decode(c)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("spec", TINY_SPECS, ids=lambda s: s.name)
def test_unowned_rows_never_matter(spec):
    outs = [oracle.pa_decode(I.make_case(spec, fill=f)) for f in ("zero", "nan", "inf", "random")]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert np.isfinite(outs[0]).all()


def test_gqa_grouping_heads_share_their_kv_head():
    spec = I.Spec("t_gqa", 1, ("fixed", (50,)), 1, 3, 4, 128, 16, "bf16", seed=21)
    case = I.make_case(spec, fill="zero")
    V = case.value_cache.clone()
    for kvh in range(3):
        V[:, kvh] = float(kvh + 1)
    out = oracle.pa_decode(_with(case, value_cache=V))
    for h in range(12):
        np.testing.assert_allclose(out[0, 0, h], h // 4 + 1, rtol=1e-14)


def test_zero_length_sequence_gives_zero_row():
    spec = I.Spec("t_zero", 3, ("fixed", (0, 5, 0)), 1, 1, 2, 128, 16, "bf16", seed=22)
    case = I.make_case(spec)
    out, lse = oracle.pa_decode(case, with_lse=True)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0]))
    assert np.all(out[1] != 0)


def test_qlen_rows_are_independent_non_causal():
    """Reading: every query token of a sequence attends to all of [0, L)."""
    spec = I.Spec("t_mtp", 2, ("fixed", (33, 70)), 4, 1, 2, 128, 16, "bf16", seed=23)
    case = I.make_case(spec)
    out = oracle.pa_decode(case)
    for i in range(4):
        single = _with(case, qlen=1, query=case.query[:, i:i + 1].contiguous())
        o1 = oracle.pa_decode(single)
        assert np.array_equal(out[:, i], o1[:, 0])


# ------------------------------------------------ causal and sliding window

MASK_SPECS = [
    I.Spec("m_bf16_q4_causal", 3, ("fixed", (1, 6, 300)), 4, 2, 2, 128, 16, "bf16", seed=31, causal=1),
    I.Spec("m_bf16_q3_win", 3, ("fixed", (2, 70, 300)), 3, 1, 3, 128, 64, "bf16", seed=32, window=37),
    I.Spec("m_fp8tok_q4_causal_win", 2, ("fixed", (257, 600)), 4, 1, 4, 256, 16, "fp8", "token", seed=33,
           causal=1, window=100),
    I.Spec("m_fp8_trans_q1_win", 2, ("fixed", (129, 513)), 1, 1, 8, 128, 128, "fp8", "tensor", "trans", seed=34,
           window=256),
    I.Spec("m_bf16_q2_causal_w1", 2, ("fixed", (1, 40)), 2, 1, 2, 128, 16, "bf16", seed=35, causal=1, window=1),
]


@pytest.mark.parametrize("spec", MASK_SPECS, ids=lambda s: s.name)
def test_masked_oracle_equals_brute_force_dense(spec):
    """Causal and windowed rows against dense attention with an explicit position mask."""
    case = I.make_case(spec)
    got = oracle.pa_decode(case)
    want = dense_reference(case)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("spec", [MASK_SPECS[0], MASK_SPECS[2]], ids=lambda s: s.name)
def test_causal_off_by_one_is_caught(spec):
    case = I.make_case(spec)
    got = oracle.pa_decode(case)
    for shift in (-1, 1):
        wrong = dense_reference(case, causal_shift=shift)
        assert np.abs(got - wrong).max() > 1e-3


def test_causal_row_equals_shorter_non_causal_decode():
    """Row i of a causal decode over L tokens is the plain decode over the
    first L - qlen + i + 1 tokens (same pages, same query row)."""
    case = I.make_case(MASK_SPECS[0].replace(lens=("fixed", (9, 40, 300))), fill="zero")
    got = oracle.pa_decode(case)
    QL = case.qlen
    for i in range(QL):
        lens = (case.context_lens - QL + i + 1).clamp(min=0)
        short = dataclasses.replace(case, context_lens=lens.to(torch.int32), causal=0)
        want = oracle.pa_decode(short)
        np.testing.assert_array_equal(got[:, i], want[:, i])


def test_window_of_one_gives_the_last_v_row_exactly():
    """A one-token window puts all weight on position e_i - 1: the output is that V row."""
    spec = I.Spec("w1", 2, ("fixed", (5, 100)), 2, 1, 2, 128, 16, "bf16", seed=36, window=1, causal=1)
    case = I.make_case(spec, fill="zero")
    got = oracle.pa_decode(case)
    for b in range(case.num_seqs):
        L = int(case.context_lens[b])
        for i in range(case.qlen):
            t = L - case.qlen + i
            page = int(case.block_tables[b, t // case.page_size])
            for h in range(case.num_q_heads):
                v = case.value_cache[page, h // case.q_per_kv, t % case.page_size].double().numpy()
                np.testing.assert_array_equal(got[b, i, h], v)


def test_window_at_least_the_context_is_no_window():
    spec = MASK_SPECS[1].replace(window=300)
    case = I.make_case(spec)
    got = oracle.pa_decode(case)
    plain = oracle.pa_decode(dataclasses.replace(case, window=0))
    np.testing.assert_array_equal(got, plain)
    tighter = oracle.pa_decode(dataclasses.replace(case, window=299))
    assert np.abs(tighter[2] - got[2]).max() > 0  # L = 300: a 299-token window drops position 0


def test_empty_causal_rows_are_zero():
    """With L < qlen the first query tokens see no position: their rows are 0."""
    case = I.make_case(MASK_SPECS[0])  # L = 1 with qlen 4
    got = oracle.pa_decode(case)
    assert np.all(got[0, :3] == 0) and np.any(got[0, 3] != 0)


@pytest.mark.parametrize("spec", MASK_SPECS[1:4], ids=lambda s: s.name)
def test_prewindow_poison_is_invisible_to_the_oracle(spec):
    """Freeing what every row's window has left behind (table columns wholly
    before it pointed at block 0, earlier rows of its first page filled with
    NaN / Inf / random bytes and scales) leaves the decode unchanged: the
    definition reads only positions inside some row's range."""
    case = I.make_case(spec.replace(lens=("fixed", tuple(L + 300 for L in spec.lens[1]))), fill="zero")
    want = oracle.pa_decode(case)
    moved = 0
    for fill in ("nan", "inf", "random"):
        pc = I.poison_prewindow(case, fill)
        moved += int((pc.block_tables != case.block_tables).sum())
        np.testing.assert_array_equal(oracle.pa_decode(pc), want)
    assert moved > 0  # some table column lies wholly before a window
