"""Numerics of the block-scaled fp4 x fp8 MFMA the MXFP4 decode's QK uses.

v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 K rows (e8m0 scale per 32 values)
and e4m3 query rows (ROCm/aiter PR #7056, "Behavior and intent"), on operands
drawn like the MXFP4 workload's: uniform fp4 bytes, K scale bytes in
[118, 136], the query N(0, 1) cast to e4m3 (as stored, unit scale) or scaled
per row so its largest value reaches 448 (the bf16-query path). Every product
of an e2m1 and an e4m3 value is exact, so fp64 gives the exact dot products.

What it shows (finite data only):
- the instruction's error stays within 2^-12 of the largest product of its dot;
- computing the 128-deep reduction as one instruction, as four one-block
  instructions accumulating in C, as four with their results added in fp32,
  or as two half-depth instructions gives the same error: the precision is
  lost inside a 32-element block's sum, so no split of the reduction across
  instructions recovers fp32 accuracy;
- that error is far above an fp32 accumulation's (2^-24 per add) on some dots.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "mfma_probe", "libmxprobe.so")
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
NTILES = 1024
VARIANTS = ("one instruction", "per block, C accumulates", "per block, summed in fp32", "two halves, C accumulates")


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    if not os.path.exists(LIB):
        raise RuntimeError("%s is not built (run the build entry point first)" % LIB)
    lib = ctypes.CDLL(LIB)
    lib.mx_probe_run.restype = ctypes.c_int
    lib.mx_probe_run.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_void_p]
    return lib


def _operands(qmode, seed):
    g = torch.Generator().manual_seed(seed)
    A = torch.randint(0, 256, (NTILES, 16, 64), generator=g, dtype=torch.int32).to(torch.uint8)
    As = torch.randint(118, 137, (NTILES, 16, 4), generator=g, dtype=torch.int32).to(torch.uint8)
    q = torch.randn(NTILES, 16, 128, generator=g)
    if qmode == 0:
        e = torch.zeros(NTILES, 16)
    else:  # the smallest e with max|q| <= 448 * 2^e
        e = torch.ceil(torch.log2(q.abs().amax(-1) / 448.0))
    Bf = (q / torch.exp2(e)[..., None]).to(torch.float8_e4m3fn)
    Bq = Bf.view(torch.uint8)
    Bs = (127 + e).to(torch.uint8)[..., None].expand(NTILES, 16, 4).contiguous()
    # exact dot products S[tile][token][row] and the largest |product| of each
    a_lo, a_hi = (A & 15).long(), (A >> 4).long()
    av = torch.from_numpy(E2M1)[torch.stack((a_lo, a_hi), -1).reshape(NTILES, 16, 128)]
    av = av * torch.exp2(As.double() - 127).repeat_interleave(32, -1)
    bv = Bf.double() * torch.exp2(Bs.double() - 127).repeat_interleave(32, -1)
    exact = torch.einsum("tmk,tnk->tmn", av, bv)
    maxprod = (av.abs()[:, :, None, :] * bv.abs()[:, None, :, :]).amax(-1)
    sumabs = torch.einsum("tmk,tnk->tmn", av.abs(), bv.abs())
    return (A, As, Bq, Bs), exact.numpy(), maxprod.numpy(), sumabs.numpy()


@pytest.mark.parametrize("qmode", [0, 1], ids=["q_e4m3_as_stored", "q_row_scaled_to_448"])
def test_scaled_mfma_block_sum_precision(probe, qmode):
    ops, exact, maxprod, sumabs = _operands(qmode, 2024 + qmode)
    dev = [t.cuda() for t in ops]
    out = torch.empty(NTILES * 4 * 256, dtype=torch.float32, device="cuda")
    st = probe.mx_probe_run(*[ctypes.c_void_p(t.data_ptr()) for t in dev], ctypes.c_void_p(out.data_ptr()), NTILES,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(NTILES, 4, 16, 16)
    rel = []
    for v, name in enumerate(VARIANTS):
        err = np.abs(got[:, v] - exact)
        worst = float((err / np.maximum(maxprod, 1e-300)).max())
        beyond = int((err > 128 * 2.0 ** -24 * sumabs).sum())
        print("%s, %s: max|err| %.4g, max|err|/max|product| 2^%.2f, rms %.3g, %d of %d dots beyond an fp32 "
              "sum's bound" % (["q e4m3", "q scaled to 448"][qmode], name, err.max(), np.log2(worst),
                               np.sqrt((err ** 2).mean()), beyond, err.size))
        assert worst <= 2.0 ** -12
        rel.append(worst)
        if v == 0:
            assert beyond > 0  # coarser than fp32 accumulation somewhere
    assert max(rel) <= 1.02 * min(rel)  # no split of the reduction changes the error
