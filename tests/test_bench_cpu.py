"""bench.py's host-side contract, on the CPU: the one-GPU refusal, the
algorithmic byte counts behind the reported GB/s, and the kernel tags that
key the HBM counter summaries to kernel instances."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_attention_decode_token_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_window_bytes_count_the_tokens_some_row_sees():
    # qlen 3, causal, window 100: row i of a sequence of length L sees
    # [L - 3 + i + 1 - 100, L - 3 + i + 1); the union over rows is
    # [max(0, L - 2 - 100), L)
    spec = I.Spec("win_bytes", 4, ("fixed", (1, 50, 101, 700)), 3, 2, 4, 128, 16, "bf16", seed=7, causal=1,
                  window=100)
    case = I.make_case(spec)
    per_token_head = 4 * 128
    expect = sum(L - max(0, L - 2 - 100) for L in (1, 50, 101, 700)) * 2 * per_token_head
    assert bench.read_bytes(case) == expect
    # without a window every owned token counts
    plain = I.make_case(spec.replace(name="plain_bytes", window=0, causal=0))
    assert bench.read_bytes(plain) == (1 + 50 + 101 + 700) * 2 * per_token_head == plain.kv_bytes()


def test_kernel_tags_name_the_instances_rocprofv3_prints():
    assert bench.kernel_tag_of(I.BF16_P64) == "Cfg<0, 0, 0, 128, 64, 1, 0, 0, 0>"
    assert bench.kernel_tag_of(I.BF16_P128) == "Cfg<0, 0, 0, 128, 128, 1, 0, 0, 0>"
    assert bench.kernel_tag_of(I.FP8TOK_Q1) == "Cfg<1, 2, 0, 256, 16, 1, 0, 0, 0>"
    assert bench.kernel_tag_of(I.FP8TOK_Q4) == "Cfg<1, 2, 0, 256, 16, 2, 0, 0, 0>"
    assert bench.kernel_tag_of(I.FP8TOK_Q4_CAUSAL) == "Cfg<1, 2, 0, 256, 16, 2, 0, 0, 2>"
    assert bench.kernel_tag_of(I.BF16_P64_W1024) == "Cfg<0, 0, 0, 128, 64, 1, 0, 0, 1>"
    assert bench.kernel_tag_of(I.FP8_TRANS) == "Cfg<1, 1, 1, 128, 128, 1, 0, 0, 0>"


def test_traffic_is_keyed_to_the_kernel_source():
    # the committed counter summary is used only for the kernel source it was taken on
    tr = bench.load_traffic("bf16_p64_b64")
    import json
    doc = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    if doc["kernel_source"] == bench.kernel_source_hash():
        assert tr == doc["kernels"]["bf16_p64_b64"]["hbm_bytes_per_launch"]
    else:
        assert tr is None


def test_page_shapes_are_bench_only_and_follow_the_pages_recipe():
    # timed by `bench.py --all --workloads`, not part of the parity batches
    full = {s.name for s in I.FULL}
    for s in I.PAGE_SHAPES:
        assert s.name not in full and I.BY_NAME[s.name] is s
        assert (s.num_kv_heads, s.q_per_kv, s.head_dim) == (2, 8, 256)
        kind, lo, hi = s.lens
        # ctx - U[0, 255] tokens per sequence
        assert kind == "uniform" and hi - lo == 255 and hi & (hi - 1) == 0
    tags = {bench.kernel_tag_of(s) for s in I.PAGE_SHAPES}
    assert "Cfg<1, 2, 0, 256, 16, 1, 0, 0, 0>" in tags and "Cfg<1, 1, 0, 256, 128, 1, 0, 0, 0>" in tags


def test_task_budgets_option_is_parsed_for_the_all_table():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "--task-budgets" in r.stdout
