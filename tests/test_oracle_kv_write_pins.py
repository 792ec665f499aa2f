"""Pins of the oracle's MXFP4 cache write against facts that are not the oracle.

What fixes each expected value:
  - a table of blocks encoded by hand from the OCP Microscaling conversion and
    the E2M1 magnitudes (tests/golden/mxfp4_encode_ocp_mx.txt, cited there):
    ties to even, saturation, signed zero, scale clamping, NaN/Inf blocks,
    nibble order;
  - exact round trips: a block of E2M1 values times a power of two is
    representable, so decoding its encoding with the pinned decoders must
    give it back exactly;
  - the properties the conversion guarantees: max|v| / 2^E lies in [4, 8),
    every element is within half a grid step of v / 2^E (or clipped to 6),
    scaling by 2^k moves only the scale byte, negation flips only sign bits;
  - composition with the decode: pages written from representable K/V, read
    by the oracle decode, give the brute-force dense attention over the
    original values.
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
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _golden_cases():
    cases = []
    with open(os.path.join(GOLDEN, "mxfp4_encode_ocp_mx.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, sc, data, start, vals = [x.strip() for x in line.split(";")]
            v = np.zeros(32)
            for i, t in enumerate(vals.split()):
                v[int(start) + i] = float.fromhex(t) if "x" in t else float(t)
            cases.append((name, v, int(sc), bytes.fromhex(data)))
    return cases


def _decode_block(data, scale):
    s = oracle.e8m0_to_f64(scale)
    out = np.zeros(32)
    for i in range(32):
        nib = (int(data[i // 2]) >> (4 * (i & 1))) & 0xF
        out[i] = oracle.e2m1_to_f64(nib) * s
    return out


def _representable_block(rng, k):
    codes = rng.integers(0, 16, size=32)
    mags = E2M1[codes & 7]
    return np.where(codes >= 8, -mags, mags) * 2.0 ** k


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_encoder_matches_hand_derived_table(case):
    _, v, sc, data = case
    got_d, got_s = oracle.mxfp4_encode_block(v)
    assert got_s == sc
    assert got_d.tobytes() == data


def test_e2m1_scalar_encoder_rounds_ties_to_even():
    # the midpoints between neighbouring magnitudes, and the code each must take
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in mids.items():
        assert oracle.f64_to_e2m1(x) == c
        assert oracle.f64_to_e2m1(-x) == c | 8
    for c in range(8):  # every magnitude maps to its own code
        assert oracle.f64_to_e2m1(E2M1[c]) == c


def test_e2m1_scalar_encoder_saturates_every_large_magnitude():
    # saturation: anything at or beyond the largest magnitude, 6, takes code 7,
    # however far beyond (distances to the grid lose precision there)
    for x in (6.0, 6.5, 7.99, 8.0, 1e6, 2.0 ** 60, 7.26e16, 1e300, float("inf")):
        assert oracle.f64_to_e2m1(x) == 7
        assert oracle.f64_to_e2m1(-x) == 15


def test_round_trip_of_representable_blocks_is_exact():
    rng = np.random.default_rng(7)
    for _ in range(400):
        k = int(rng.integers(-120, 121))
        v = _representable_block(rng, k)
        d, s = oracle.mxfp4_encode_block(v)
        assert 1 <= s <= 254
        assert np.array_equal(_decode_block(d, s), v)


def test_scale_puts_block_max_in_four_to_eight():
    rng = np.random.default_rng(8)
    for _ in range(400):
        v = rng.standard_normal(32) * 2.0 ** rng.uniform(-100, 100)
        d, s = oracle.mxfp4_encode_block(v)
        ratio = np.abs(v).max() / 2.0 ** (s - 127)
        assert 4.0 <= ratio < 8.0


def test_elements_within_half_a_grid_step():
    rng = np.random.default_rng(9)
    for _ in range(300):
        v = rng.standard_normal(32) * 2.0 ** rng.uniform(-20, 20)
        v[rng.integers(0, 32)] *= 3.0  # push some blocks into the clipped range
        d, s = oracle.mxfp4_encode_block(v)
        x = v / 2.0 ** (s - 127)
        got = _decode_block(d, s) / 2.0 ** (s - 127)
        ax = np.abs(x)
        step = np.where(ax < 2, 0.5, np.where(ax < 4, 1.0, 2.0))
        inside = ax <= 6
        assert np.all(np.abs(got[inside] - x[inside]) <= step[inside] / 2)
        assert np.all(got[~inside] == np.sign(x[~inside]) * 6.0)


def test_scaling_by_a_power_of_two_moves_only_the_scale():
    rng = np.random.default_rng(10)
    for _ in range(100):
        v = rng.standard_normal(32)
        d0, s0 = oracle.mxfp4_encode_block(v)
        for k in (-40, -3, 1, 17, 60):
            d, s = oracle.mxfp4_encode_block(v * 2.0 ** k)
            assert s == s0 + k
            assert np.array_equal(d, d0)


def test_negation_flips_only_sign_bits():
    rng = np.random.default_rng(11)
    for _ in range(100):
        v = rng.standard_normal(32)
        d0, s0 = oracle.mxfp4_encode_block(v)
        d1, s1 = oracle.mxfp4_encode_block(-v)
        assert s1 == s0
        assert np.array_equal(d1, d0 ^ 0x88)


def test_negative_controls_are_caught():
    # an encoding off by one in the scale, or with its nibbles swapped, fails
    # the exact round trip that the correct one passes
    rng = np.random.default_rng(12)
    v = _representable_block(rng, 3)
    v[0] = 6 * 8.0  # make the block's maximum code 7 so a nibble swap shows
    v[1] = 0.5 * 8.0
    d, s = oracle.mxfp4_encode_block(v)
    assert np.array_equal(_decode_block(d, s), v)
    assert not np.array_equal(_decode_block(d, s + 1), v)
    swapped = ((d & 0x0F) << 4) | (d >> 4)
    assert not np.array_equal(_decode_block(swapped, s), v)


# ------------------------------------------------------------- the cache write

def _write_inputs(N, H, D, PG, NB, seed):
    g = torch.Generator().manual_seed(seed)
    key = (torch.randn((N, H, D), generator=g) * 4).to(torch.bfloat16)
    value = (torch.randn((N, H, D), generator=g) * 0.05).to(torch.bfloat16)
    kc = torch.randint(0, 256, (NB, H, PG, D // 2), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (NB, H, PG, D // 2), generator=g, dtype=torch.uint8)
    ks = torch.randint(0, 256, (NB, H, PG, D // 32), generator=g, dtype=torch.uint8)
    vs = torch.randint(0, 256, (NB, H, PG, D // 32), generator=g, dtype=torch.uint8)
    return key, value, kc, vc, ks, vs


@pytest.mark.parametrize("D", [64, 128, 256])
def test_write_places_each_token_row_and_skips_the_rest(D):
    N, H, PG, NB = 23, 3, 16, 5
    key, value, kc, vc, ks, vs = _write_inputs(N, H, D, PG, NB, seed=100 + D)
    rng = np.random.default_rng(D)
    slots = rng.permutation(NB * PG)[:N].astype(np.int32)
    slots[4] = -1            # padding token
    slots[9] = NB * PG       # one past the last slot
    slots[15] = 2 ** 31 - 1  # far out of range
    okc, ovc, oks, ovs = oracle.write_kv_mxfp4(key, value, slots, kc, vc, ks, vs)
    ekc, evc, eks, evs = (a.numpy().copy() for a in (kc, vc, ks, vs))
    kbits = key.view(torch.int16).numpy().view(np.uint16)
    vbits = value.view(torch.int16).numpy().view(np.uint16)
    for n in range(N):
        s = int(slots[n])
        if not 0 <= s < NB * PG:
            continue
        page, row = divmod(s, PG)
        for h in range(H):
            for src, dc, dsc in ((kbits, ekc, eks), (vbits, evc, evs)):
                vals = np.array([oracle.bf16_to_f64(c) for c in src[n, h]])
                for j in range(D // 32):
                    d, sc = oracle.mxfp4_encode_block(vals[32 * j:32 * j + 32])
                    dc[page, h, row, 16 * j:16 * j + 16] = d
                    dsc[page, h, row, j] = sc
    for got, exp in ((okc, ekc), (ovc, evc), (oks, eks), (ovs, evs)):
        assert np.array_equal(got, exp)
    # rows no token maps to keep their bytes
    untouched = np.ones((NB * PG,), dtype=bool)
    untouched[[int(s) for s in slots if 0 <= s < NB * PG]] = False
    pages, rows = np.divmod(np.nonzero(untouched)[0], PG)
    assert np.array_equal(okc[pages, :, rows], kc.numpy()[pages, :, rows])
    assert np.array_equal(ovs[pages, :, rows], vs.numpy()[pages, :, rows])


def test_written_pages_decode_to_dense_attention_of_the_originals():
    # K/V made of e2m1 values times a power of two per block are stored exactly,
    # so the oracle decode over the written pages must equal dense attention over
    # the original rows (brute force written here).
    spec = I.Spec("w_compose", 3, ("fixed", (1, 130, 255)), 1, 2, 4, 128, 128, "mxfp4", q_dtype="fp8", seed=31)
    case = I.make_case(spec, fill="nan")
    B, H, D, PG = case.num_seqs, case.num_kv_heads, case.head_dim, case.page_size
    lens = [int(x) for x in case.context_lens]
    N = sum(lens)
    rng = np.random.default_rng(5)
    kv = np.zeros((2, N, H, D))
    for t in range(2):
        for n in range(N):
            for h in range(H):
                for j in range(D // 32):
                    kv[t, n, h, 32 * j:32 * j + 32] = _representable_block(rng, int(rng.integers(-3, 4)))
    key = torch.from_numpy(kv[0]).to(torch.bfloat16)
    value = torch.from_numpy(kv[1]).to(torch.bfloat16)
    assert np.array_equal(key.double().numpy(), kv[0])
    slots = []
    for b in range(B):
        for t in range(lens[b]):
            slots.append(int(case.block_tables[b, t // PG]) * PG + t % PG)
    kc, vc, ks, vs = oracle.write_kv_mxfp4(key, value, np.array(slots, np.int32), case.key_cache, case.value_cache,
                                           case.k_scale, case.v_scale)
    written = dataclasses.replace(case, key_cache=torch.from_numpy(kc), value_cache=torch.from_numpy(vc),
                                  k_scale=torch.from_numpy(ks), v_scale=torch.from_numpy(vs))
    got = oracle.pa_decode(written)
    G = case.q_per_kv
    off = 0
    for b in range(B):
        L = lens[b]
        K, V = kv[0, off:off + L], kv[1, off:off + L]
        off += L
        for h in range(H * G):
            q = case.query[b, 0, h].view(torch.float8_e4m3fn).to(torch.float64).numpy()
            if L == 0:
                assert np.all(got[b, 0, h] == 0)
                continue
            s = K[:, h // G] @ q / math.sqrt(D)
            p = np.exp(s - s.max())
            p /= p.sum()
            exp = p @ V[:, h // G]
            assert np.allclose(got[b, 0, h], exp, rtol=1e-12, atol=1e-12)


def test_write_rejects_a_bad_description():
    key, value, kc, vc, ks, vs = _write_inputs(2, 1, 64, 16, 2, seed=3)
    with pytest.raises(ValueError):
        oracle.write_kv_mxfp4(key, value, np.zeros(2, np.int32), kc[:, :, :, :16], vc, ks, vs)
