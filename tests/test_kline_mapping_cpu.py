"""The whole-line K load mapping and its lane exchange (pa_kernels.hip, load_k
and fix_k), emulated on the CPU: each load instruction covers whole 128-byte
lines, and after the exchange every lane holds the bytes the MFMA operand
layout of the ordinary mapping puts there. The GPU parity tests check the
kernels; this pins the index arithmetic the comments state."""
import pytest


def ordinary(lane, c, u):
    ln, lg = lane % 16, lane // 16
    return (16 * (ln >> 2) + (ln & 3) + 4 * c, 64 * u + 16 * lg)  # (token, first byte of 16)


def whole_line_load(lane, c, u):
    ln, lg = lane % 16, lane // 16
    tok = 16 * (ln >> 2) + (ln & 2) + 4 * c + (u & 1)  # call 2L: token t(2p), call 2L + 1: t(2p) + 1
    return (tok, 128 * (u >> 1) + 64 * (ln & 1) + 16 * lg)


def exchange(regs, c, L):
    """DPP quad_perm [1, 0, 3, 2] (lane ^ 1) and the select of fix_k."""
    lo = {l: regs[(l, c, 2 * L)] for l in range(64)}
    hi = {l: regs[(l, c, 2 * L + 1)] for l in range(64)}
    for l in range(64):
        odd = (l % 16) & 1
        regs[(l, c, 2 * L)] = hi[l ^ 1] if odd else lo[l]
        regs[(l, c, 2 * L + 1)] = hi[l] if odd else lo[l ^ 1]


@pytest.mark.parametrize("row_bytes", [128, 256])  # fp8 and bf16 K rows at head_dim 128
def test_each_load_covers_whole_lines_and_the_exchange_restores_the_layout(row_bytes):
    kloads = row_bytes // 64
    for c in range(4):
        for u in range(kloads):
            chunks = {whole_line_load(l, c, u) for l in range(64)}
            lines = {}
            for tok, b in chunks:
                lines.setdefault((tok, b // 128), set()).add(b % 128)
            assert len(chunks) == 64 and len(lines) == 8
            assert all(v == set(range(0, 128, 16)) for v in lines.values())
    regs = {(l, c, u): whole_line_load(l, c, u) for l in range(64) for c in range(4) for u in range(kloads)}
    for c in range(4):
        for L in range(kloads // 2):
            exchange(regs, c, L)
    for key, val in regs.items():
        assert val == ordinary(*key), key


def test_a_lane_pair_stays_inside_one_16_token_group():
    # tokens t(2p) and t(2p) + 1 lie in the same group of 16, so in the same page at page 16
    for lane in range(64):
        for c in range(4):
            a, b = whole_line_load(lane, c, 0)[0], whole_line_load(lane, c, 1)[0]
            assert b == a + 1 and a // 16 == b // 16
