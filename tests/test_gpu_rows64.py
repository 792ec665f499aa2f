"""GPU parity for 33-64 query rows per KV head (four 16-row N tiles).

The pages' unowned-row test matrix includes qlen 4 with one KV head and 16
query heads per KV head at head_dim 128, i.e. 64 query rows sharing one KV
head (ROCm/aiter PR #7092, "Tests"; its follow-up commit raises the row tile
to four MFMA tiles). Every format with a head_dim-128 instance runs that case
over lengths {1, 17, 255, 257, 1000}, block 0 unowned and 2 padded columns:
parity with the fp64 oracle (planned, split into many partitions, plan-free),
NaN / Inf / random poison bit-identical to zero fill, and repeat runs
bit-identical. Causal and windowed rows and a 40-row (padded) case as well.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_token_amd import binding as B
from paged_attention_decode_token_amd import inputs as I

from parity_bar import check_parity
from test_gpu_parity import run, run_direct

pytestmark = pytest.mark.gpu

LENS = (1, 17, 255, 257, 1000)

FORMATS = [("bf16", "none", "plain"), ("bf16", "none", "trans"), ("fp8", "tensor", "plain"),
           ("fp8", "tensor", "trans"), ("fp8", "token", "plain")]

ROWS64 = [I.Spec("r64_%s_%s_%s_p%d" % (kv, sc, vl, pg), len(LENS), ("fixed", LENS), 4, 1, 16, 128, pg, kv, sc, vl,
                 seed=60 + 5 * i + j)
          for i, (kv, sc, vl) in enumerate(FORMATS) for j, pg in enumerate((16, 64, 128))]

MASKED = [
    I.Spec("r64_bf16_p64_causal", 5, ("fixed", LENS), 4, 1, 16, 128, 64, "bf16", seed=90, causal=1),
    I.Spec("r64_fp8tok_p16_causal_w300", 5, ("fixed", LENS), 4, 1, 16, 128, 16, "fp8", "token", seed=91, causal=1,
           window=300),
    I.Spec("r64_fp8trans_p128_w200", 5, ("fixed", LENS), 4, 1, 16, 128, 128, "fp8", "tensor", "trans", seed=92,
           window=200),
    I.Spec("r40_bf16_p64_q5_g8", 4, ("fixed", (3, 300, 700, 1500)), 5, 2, 8, 128, 64, "bf16", seed=93),
    I.Spec("r48_fp8tok_p16_q3_g16_causal", 3, ("fixed", (2, 600, 1300)), 3, 1, 16, 128, 16, "fp8", "token", seed=94,
           causal=1),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("spec", ROWS64 + MASKED, ids=lambda s: s.name)
def test_rows_up_to_64_parity_poison_determinism(spec):
    case = I.make_case(spec, fill="zero")
    ref = oracle.pa_decode(case)
    out, plan = run(case)
    check_parity(out, ref, what=spec.name)
    many, _ = run(case, task_budget=100000)
    check_parity(many, ref, what=spec.name + " many partitions")
    direct = run_direct(case)
    check_parity(direct, ref, what=spec.name + " plan-free")
    one, _ = run(case, max_partitions=1)
    assert torch.equal(direct.view(torch.int16), one.view(torch.int16))
    base = _bits(out)
    for fill in ("nan", "inf", "random"):
        poisoned = run(I.refill(case, fill))[0]
        assert np.array_equal(_bits(poisoned), base), "%s fill changes the output" % fill
    for _ in range(2):
        assert np.array_equal(_bits(run(case)[0]), base), "repeat run differs"
    # context length 1 (sequence 0 of the bf16 cases): every row is exactly V row 0
    if spec.kv_dtype == "bf16" and spec.v_layout == "plain" and not spec.causal and int(case.context_lens[0]) == 1:
        p = int(case.block_tables[0, 0])
        for h in range(case.num_q_heads):
            v0 = case.value_cache[p, h // case.q_per_kv, 0].view(torch.int16)
            for i in range(case.qlen):
                assert torch.equal(out[0, i, h].cpu().view(torch.int16), v0)
