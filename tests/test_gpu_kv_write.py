"""GPU parity of the MXFP4 KV-cache write: the HIP kernel through the C ABI
against the fp64 oracle.

The write is byte work, so the bar is bit-exact: every byte of both caches and
both scale tables, the written rows and the stale rows no token maps to, must
equal the oracle's. At full size, sampled tokens are encoded by the oracle and
compared at their slots; properties that hold at any size are checked on the
whole cache.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_token_amd import binding as B
from paged_attention_decode_token_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()  # raises when libpa.so is missing


def _gpu_write(case, key=None, value=None, slots=None):
    key = case.key if key is None else key
    value = case.value if value is None else value
    slots = case.slot_mapping if slots is None else slots
    d = [t.cuda().contiguous() for t in (key, value, slots)]
    bufs = [t.cuda().clone() for t in (case.key_cache, case.value_cache, case.key_scale, case.value_scale)]
    B.pa_write_kv_mxfp4(d[0], d[1], d[2], *bufs)
    torch.cuda.synchronize()
    return [b.cpu().numpy() for b in bufs]


def _oracle_write(case, key=None, value=None, slots=None):
    key = case.key if key is None else key
    value = case.value if value is None else value
    slots = case.slot_mapping if slots is None else slots
    return oracle.write_kv_mxfp4(key.cpu(), value.cpu(), slots.cpu().numpy(), case.key_cache.cpu(),
                                 case.value_cache.cpu(), case.key_scale.cpu(), case.value_scale.cpu())


def _assert_same(got, exp, what):
    names = ("key_cache", "value_cache", "key_scale", "value_scale")
    for g, e, n in zip(got, exp, names):
        if not np.array_equal(g, e):
            bad = np.argwhere(g != e)
            raise AssertionError("%s: %s differs at %d bytes, first %s (gpu %d, oracle %d)" % (
                what, n, len(bad), tuple(bad[0]), g[tuple(bad[0])], e[tuple(bad[0])]))


SMALL_WRITE = [I.small_write(s) for s in I.WRITE_FULL] + [
    I.small_write(I.MXFP4_WRITE_FILL).replace(name="d64_p16_h1", head_dim=64, page_size=16, num_kv_heads=1, seed=7),
    I.small_write(I.MXFP4_WRITE_FILL).replace(name="d256_p64_h3", head_dim=256, page_size=64, num_kv_heads=3,
                                              seed=8),
    I.small_write(I.MXFP4_WRITE_FILL).replace(name="d128_p128_h8_ragged", num_kv_heads=8, num_seqs=4,
                                              lens=("fixed", (129, 1, 255, 640)), pad_tokens=3, seed=9),
    # a page size that is not a power of two takes the division path for the slot
    I.small_write(I.MXFP4_WRITE_FILL).replace(name="d128_p48_h4", num_kv_heads=4, page_size=48, seed=10),
]


@pytest.mark.parametrize("spec", SMALL_WRITE, ids=lambda s: s.name)
def test_write_matches_oracle_bit_exact(spec):
    case = I.make_write_case(spec)
    print("write parity", spec.name, "tokens", case.num_tokens, flush=True)
    _assert_same(_gpu_write(case), _oracle_write(case), spec.name)


def _bits_case(seed, bits_fn, H=2, D=128):
    spec = I.small_write(I.MXFP4_WRITE_FILL).replace(name="bits%d" % seed, num_kv_heads=H, head_dim=D, seed=seed)
    case = I.make_write_case(spec)
    g = torch.Generator().manual_seed(seed)
    n = case.num_tokens
    key = bits_fn(g, (n, H, D)).view(torch.bfloat16)
    value = bits_fn(g, (n, H, D)).view(torch.bfloat16)
    return case, key, value


def _random_bits(g, shape):
    return torch.randint(-32768, 32768, shape, generator=g, dtype=torch.int32).to(torch.int16)


def _finite_bits(g, shape):
    # every sign and mantissa, exponent fields 0..254 (zero, subnormal, normal)
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 15
    exp = torch.randint(0, 255, shape, generator=g, dtype=torch.int32) << 7
    man = torch.randint(0, 128, shape, generator=g, dtype=torch.int32)
    v = sign | exp | man
    return (v - (v >= 32768).to(torch.int32) * 65536).to(torch.int16)


def _narrow_bits(g, shape):
    # exponents close together, so most elements land inside the e2m1 grid,
    # including exact midpoints (mantissas with few bits set)
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 15
    exp = torch.randint(124, 131, shape, generator=g, dtype=torch.int32) << 7
    man = torch.randint(0, 8, shape, generator=g, dtype=torch.int32) << 4
    v = sign | exp | man
    return (v - (v >= 32768).to(torch.int32) * 65536).to(torch.int16)


@pytest.mark.parametrize("kind,fn", [("all_bit_patterns", _random_bits), ("finite_any_exponent", _finite_bits),
                                     ("near_the_grid", _narrow_bits)], ids=lambda x: x if isinstance(x, str) else "")
def test_write_random_bit_patterns(kind, fn):
    case, key, value = _bits_case(40 + len(kind), fn)
    print("write bits", kind, flush=True)
    _assert_same(_gpu_write(case, key, value), _oracle_write(case, key, value), kind)


def test_write_special_blocks():
    # blocks taken from hand-derived encoding cases: ties, clipping, signed
    # zero, all-zero, NaN, infinities, the smallest and largest scales
    rows = []
    for line in open(__file__.replace("test_gpu_kv_write.py", "golden/mxfp4_encode_ocp_mx.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        _, _, _, start, vals = [x.strip() for x in line.split(";")]
        v = np.zeros(32)
        for i, t in enumerate(vals.split()):
            v[int(start) + i] = float.fromhex(t) if "x" in t else float(t)
        rows.append(v)
    blocks = np.stack(rows)  # [nb, 32]
    spec = I.small_write(I.MXFP4_WRITE_FILL).replace(name="special", num_kv_heads=1, seed=77)
    case = I.make_write_case(spec)
    n = case.num_tokens
    rng = np.random.default_rng(3)
    pick = rng.integers(0, len(blocks), size=(n, 1, 4))
    k = torch.from_numpy(blocks[pick].reshape(n, 1, 128)).to(torch.bfloat16)
    v = torch.from_numpy(-blocks[pick[:, :, ::-1]].reshape(n, 1, 128)).to(torch.bfloat16)
    _assert_same(_gpu_write(case, k, v), _oracle_write(case, k, v), "special blocks")


def test_write_skips_slots_outside_the_cache():
    spec = I.small_write(I.MXFP4_WRITE_FILL).replace(name="bad_slots", seed=12)
    case = I.make_write_case(spec)
    s = case.slot_mapping.clone()
    nslots = case.num_blocks * case.page_size
    s[0], s[7], s[100], s[200] = -1, nslots, 2 ** 31 - 1, -(2 ** 31)
    _assert_same(_gpu_write(case, slots=s), _oracle_write(case, slots=s), "bad slots")


def test_write_of_no_tokens_leaves_the_cache():
    spec = I.small_write(I.MXFP4_WRITE_FILL).replace(name="empty", seed=13)
    case = I.make_write_case(spec)
    e = torch.zeros((0, case.num_kv_heads, case.head_dim), dtype=torch.bfloat16)
    got = _gpu_write(case, e, e, torch.zeros(0, dtype=torch.int32))
    _assert_same(got, [t.numpy() for t in (case.key_cache, case.value_cache, case.key_scale, case.value_scale)],
                 "empty")


def test_written_pages_decode_like_the_oracle():
    # write a decode case's pages from bf16 rows with the GPU kernel, decode them
    # on the GPU, and compare with the oracle decode of the oracle-written pages
    import dataclasses

    from test_gpu_parity import check_parity

    dspec = I.small(I.MXFP4_SHORT_Q8).replace(name="write_then_decode", seed=21)
    dcase = I.make_case(dspec)
    wspec = I.WriteSpec("w", dcase.num_seqs, ("fixed", tuple(int(x) for x in dcase.context_lens)),
                        dcase.num_kv_heads, 128, 128, "fill", seed=22)
    wcase = I.make_write_case(wspec)
    wcase = dataclasses.replace(wcase, block_tables=dcase.block_tables, key_cache=dcase.key_cache,
                                value_cache=dcase.value_cache, key_scale=dcase.k_scale, value_scale=dcase.v_scale,
                                num_blocks=dcase.num_blocks)
    PG = 128
    slots = torch.cat([dcase.block_tables[b, torch.arange(L) // PG].long() * PG + torch.arange(L) % PG
                       for b, L in enumerate(dcase.context_lens.tolist())]).to(torch.int32)
    slots = torch.cat([slots, torch.full((wcase.num_tokens - slots.numel(),), -1, dtype=torch.int32)])
    got = _gpu_write(wcase, slots=slots)
    exp = _oracle_write(wcase, slots=slots)
    _assert_same(got, exp, "decode pages")
    written = dataclasses.replace(dcase, key_cache=torch.from_numpy(got[0]), value_cache=torch.from_numpy(got[1]),
                                  k_scale=torch.from_numpy(got[2]), v_scale=torch.from_numpy(got[3]))
    out, _ = B.decode_case(written)
    torch.cuda.synchronize()
    check_parity(out, oracle.pa_decode(written), what="decode of written pages")


def test_write_is_deterministic():
    case = I.make_write_case(I.small_write(I.MXFP4_WRITE_FILL).replace(seed=14))
    a, b = _gpu_write(case), _gpu_write(case)
    _assert_same(a, b, "repeat")


@pytest.mark.slow
@pytest.mark.parametrize("spec", I.WRITE_FULL, ids=lambda s: s.name)
def test_write_full_size_sampled(spec):
    case = I.make_write_case(spec, device="cuda")
    print("write full size", spec.name, "tokens", case.num_tokens, flush=True)
    bufs = [t.clone() for t in (case.key_cache, case.value_cache, case.key_scale, case.value_scale)]
    block0 = [b[0].clone() for b in bufs]
    B.pa_write_kv_mxfp4(case.key, case.value, case.slot_mapping, *bufs)
    torch.cuda.synchronize()
    # sampled tokens: the oracle encodes them into a small cache of its own
    slots = case.slot_mapping.cpu()
    valid = torch.nonzero(slots >= 0).view(-1)
    g = torch.Generator().manual_seed(5)
    idx = valid[torch.randperm(valid.numel(), generator=g)[:1500]]
    PG, H = case.page_size, case.num_kv_heads
    S = idx.numel()
    nb = (S + PG - 1) // PG
    z = lambda w: torch.zeros((nb, H, PG, w), dtype=torch.uint8)  # noqa: E731
    ekc, evc, eks, evs = oracle.write_kv_mxfp4(case.key[idx.cuda()].cpu(), case.value[idx.cuda()].cpu(),
                                               np.arange(S, dtype=np.int32), z(64), z(64), z(4), z(4))
    s = slots[idx].long()
    pages, rows = (s // PG).cuda(), (s % PG).cuda()
    i = torch.arange(S)
    for got, exp, name in ((bufs[0], ekc, "key_cache"), (bufs[1], evc, "value_cache"), (bufs[2], eks, "key_scale"),
                           (bufs[3], evs, "value_scale")):
        g_rows = got[pages, :, rows].cpu().numpy()  # [S, H, w]
        e_rows = exp[(i // PG).numpy(), :, (i % PG).numpy()]
        assert np.array_equal(g_rows, e_rows), name
    # properties over the whole cache: finite inputs give scale bytes 1..254 in
    # every written row, and block 0 (never mapped) keeps its stale bytes
    w = slots[valid].long()
    wp, wr = (w // PG).cuda(), (w % PG).cuda()
    for sc in (bufs[2], bufs[3]):
        rows_sc = sc[wp, :, wr]
        assert int(rows_sc.min()) >= 1 and int(rows_sc.max()) <= 254
    for b, b0 in zip(bufs, block0):
        assert torch.equal(b[0], b0)
