"""Seeded synthetic inputs for paged-attention decode.

This module only draws random numbers and lays them out in the cache formats;
it holds none of the attention arithmetic. The GPU path (through the C ABI)
and the fp64 oracle both read what it builds.

Layouts (the same ones the C ABI documents):
  query          [num_seqs, qlen, Hq, D]        bf16, or e4m3fn bytes (MXFP4 only)
  key/value      [num_blocks, Hkv, page, D]     bf16 or e4m3fn bytes
  value, trans   [num_blocks, Hkv, D, page]     (transposed V)
  MXFP4 data     [num_blocks, Hkv, page, D/2]   uint8, element 2i in the low nibble
  MXFP4 scales   [num_blocks, Hkv, page, D/32]  uint8 e8m0 (passed as k_scale / v_scale)
  per-tensor     fp32 [1] each for K and V
  per-token      fp32 [num_blocks, Hkv, page] each for K and V
  block_tables   [num_seqs, max_blocks_per_seq] int32
  context_lens   [num_seqs] int32

MXFP4 cache-write inputs (WriteSpec / make_write_case):
  key, value     [num_tokens, Hkv, D]           bf16 rows to store
  slot_mapping   [num_tokens] int32             page * page_size + row, -1 for padding
  caches/scales  as the MXFP4 layouts above, holding random stale bytes

Structure (ROCm/aiter PR #7092, section "Tests"): each sequence's pages are the
next ceil(L/page) entries of a seeded permutation of pages 1..N, so block 0 is
never owned; every table row ends with at least 2 padded columns that point to
block 0. Rows no sequence owns -- all of block 0 and the tail of each last page
past the context length -- receive the requested fill ("zero", "nan", "inf" or
"random"), together with their per-token or block scales.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

PAGE_TILE = 256  # tokens per planning tile (PR #7092, "Root cause")


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    num_seqs: int
    lens: tuple  # ("fixed", (l0, l1, ...)) | ("uniform", lo, hi) | ("const", L)
    qlen: int
    num_kv_heads: int
    q_per_kv: int
    head_dim: int
    page_size: int
    kv_dtype: str  # bf16 | fp8 | mxfp4
    scale_mode: str = "none"  # none | tensor | token
    v_layout: str = "plain"  # plain | trans
    q_dtype: str = "bf16"  # bf16 | fp8
    fill: str = "nan"  # nan | inf | zero | random
    seed: int = 0
    pad_cols: int = 2
    causal: int = 0  # 1: query token i attends to t < L - qlen + i + 1
    window: int = 0  # > 0: sliding window of that many tokens ending there
    mx_k_scale: tuple = (118, 136)  # MXFP4: K scale bytes drawn uniformly from [lo, hi]

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass
class Case:
    spec: Spec
    num_seqs: int
    qlen: int
    num_kv_heads: int
    q_per_kv: int
    head_dim: int
    page_size: int
    num_blocks: int
    max_blocks_per_seq: int
    max_context_len: int
    kv_dtype: str
    scale_mode: str
    v_layout: str
    q_dtype: str
    softmax_scale: float
    query: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    causal: int = 0
    window: int = 0

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.q_per_kv

    def kv_bytes_per_token_head(self) -> int:
        D = self.head_dim
        if self.kv_dtype == "bf16":
            return 4 * D
        if self.kv_dtype == "fp8":
            return 2 * D + (8 if self.scale_mode == "token" else 0)
        return 2 * (D // 2 + D // 32)

    def kv_bytes(self, seqs: Optional[Sequence[int]] = None) -> int:
        """Bytes of K, V and their scales for the owned tokens (nominal KV payload)."""
        lens = self.context_lens.tolist()
        if seqs is not None:
            lens = [lens[i] for i in seqs]
        return sum(lens) * self.num_kv_heads * self.kv_bytes_per_token_head()

    def tensors(self):
        return dict(query=self.query, key_cache=self.key_cache, value_cache=self.value_cache,
                    k_scale=self.k_scale, v_scale=self.v_scale, block_tables=self.block_tables,
                    context_lens=self.context_lens)


# ---------------------------------------------------------------- workloads

def _spec(name, **kw):
    return Spec(name=name, **kw)


# Workloads at their stated sizes.
TINY_BF16 = _spec("tiny_bf16_p16", num_seqs=4, lens=("fixed", (1, 17, 255, 257)), qlen=1, num_kv_heads=1,
                  q_per_kv=8, head_dim=128, page_size=16, kv_dtype="bf16", fill="nan", seed=1000)
BF16_P64 = _spec("bf16_p64_b64", num_seqs=64, lens=("uniform", 1000, 8192), qlen=1, num_kv_heads=8, q_per_kv=8,
                 head_dim=128, page_size=64, kv_dtype="bf16", fill="inf", seed=1001)
BF16_P128 = BF16_P64.replace(name="bf16_p128_b64", page_size=128, seed=1002)
FP8TOK_Q1 = _spec("fp8tok_p16_b16_q1", num_seqs=16, lens=("uniform", 2048, 32768), qlen=1, num_kv_heads=2,
                  q_per_kv=8, head_dim=256, page_size=16, kv_dtype="fp8", scale_mode="token", fill="nan", seed=1003)
FP8TOK_Q4 = FP8TOK_Q1.replace(name="fp8tok_p16_b16_q4", qlen=4, seed=1004)
FP8_TRANS = _spec("fp8_transv_p128_b256", num_seqs=256, lens=("const", 16384), qlen=1, num_kv_heads=1, q_per_kv=16,
                  head_dim=128, page_size=128, kv_dtype="fp8", scale_mode="tensor", v_layout="trans", fill="nan",
                  seed=1005)
MXFP4_SHORT_Q8 = _spec("mxfp4_p128_b16_l2048_qfp8", num_seqs=16, lens=("const", 2048), qlen=1, num_kv_heads=4,
                       q_per_kv=16, head_dim=128, page_size=128, kv_dtype="mxfp4", q_dtype="fp8", fill="nan",
                       seed=1006)
MXFP4_SHORT_QBF = MXFP4_SHORT_Q8.replace(name="mxfp4_p128_b16_l2048_qbf16", q_dtype="bf16", seed=1007)
MXFP4_LONG_Q8 = MXFP4_SHORT_Q8.replace(name="mxfp4_p128_b16_l131072_qfp8", lens=("const", 131072), seed=1008)
MXFP4_LONG_QBF = MXFP4_LONG_Q8.replace(name="mxfp4_p128_b16_l131072_qbf16", q_dtype="bf16", seed=1009)

# The MXFP4 workloads' scale bytes put logits in the thousands, so their softmax
# is one-hot. These two draw K scale bytes from [122, 127] instead: logits of
# standard deviation about 1.4 and about 50 tokens of effective weight per row,
# so every step of the softmax and the weighted V sum shows in the output.
MXFP4_SPREAD_Q8 = MXFP4_SHORT_Q8.replace(name="mxfp4_p128_b16_l2048_qfp8_kscale122-127", mx_k_scale=(122, 127),
                                         seed=1020)
MXFP4_SPREAD_QBF = MXFP4_SPREAD_Q8.replace(name="mxfp4_p128_b16_l2048_qbf16_kscale122-127", q_dtype="bf16",
                                           seed=1021)

# Masked variants: a 1024-token sliding window on the bf16 batch, and causal
# multi-token verification (qlen 4) on the fp8 per-token batch.
BF16_P64_W1024 = BF16_P64.replace(name="bf16_p64_b64_w1024", window=1024, seed=1010)
FP8TOK_Q4_CAUSAL = FP8TOK_Q4.replace(name="fp8tok_p16_b16_q4_causal", causal=1, seed=1011)

FULL = [TINY_BF16, BF16_P64, BF16_P128, FP8TOK_Q1, FP8TOK_Q4, FP8_TRANS, MXFP4_SHORT_Q8, MXFP4_SHORT_QBF,
        MXFP4_LONG_Q8, MXFP4_LONG_QBF, BF16_P64_W1024, FP8TOK_Q4_CAUSAL]
# The kernel-performance shapes of the NaN-safe V mask page (ROCm/aiter PR #7092, "All 513 shapes")
# for fp8 per-token page-16 caches, 2 KV heads x GQA 8, head_dim 256, batch 16: every sequence holds
# ctx - U[0, 255] tokens. Timed by `bench.py --all --workloads ...` only; not parity batches.
FP8TOK_Q1_C16K = FP8TOK_Q1.replace(name="fp8tok_p16_b16_q1_c16384", lens=("uniform", 16129, 16384), seed=1030)
FP8TOK_Q4_C16K = FP8TOK_Q4.replace(name="fp8tok_p16_b16_q4_c16384", lens=("uniform", 16129, 16384), seed=1031)
FP8TOK_Q1_C64K = FP8TOK_Q1.replace(name="fp8tok_p16_b16_q1_c65536", lens=("uniform", 65281, 65536), seed=1032)
FP8TOK_Q4_C64K = FP8TOK_Q4.replace(name="fp8tok_p16_b16_q4_c65536", lens=("uniform", 65281, 65536), seed=1033)
# the same page's bf16 and fp8 per-tensor shapes (2 KV heads x GQA 8, head_dim 256, qlen 1)
BF16_D256_P64_C4K = _spec("bf16_d256_p64_b64_c4096", num_seqs=64, lens=("uniform", 3841, 4096), qlen=1,
                          num_kv_heads=2, q_per_kv=8, head_dim=256, page_size=64, kv_dtype="bf16", fill="inf",
                          seed=1034)
BF16_D256_P128_C4K = BF16_D256_P64_C4K.replace(name="bf16_d256_p128_b64_c4096", page_size=128, seed=1035)
BF16_D256_P64_C16K = BF16_D256_P64_C4K.replace(name="bf16_d256_p64_b64_c16384", lens=("uniform", 16129, 16384),
                                               seed=1036)
BF16_D256_P128_C16K = BF16_D256_P64_C16K.replace(name="bf16_d256_p128_b64_c16384", page_size=128, seed=1037)
FP8_D256_P128_B64_C16K = BF16_D256_P128_C16K.replace(name="fp8_d256_p128_b64_c16384", kv_dtype="fp8",
                                                     scale_mode="tensor", fill="nan", seed=1038)
FP8_D256_P128_B256_C16K = FP8_D256_P128_B64_C16K.replace(name="fp8_d256_p128_b256_c16384", num_seqs=256,
                                                         seed=1039)
BF16_D256_P16_B1_C1K = BF16_D256_P64_C4K.replace(name="bf16_d256_p16_b1_c1024", num_seqs=1, lens=("uniform", 769, 1024),
                                                 page_size=16, seed=1040)
PAGE_SHAPES = [FP8TOK_Q1_C16K, FP8TOK_Q4_C16K, FP8TOK_Q1_C64K, FP8TOK_Q4_C64K, BF16_D256_P64_C4K, BF16_D256_P128_C4K,
               BF16_D256_P64_C16K, BF16_D256_P128_C16K, FP8_D256_P128_B64_C16K, FP8_D256_P128_B256_C16K,
               BF16_D256_P16_B1_C1K]
BY_NAME = {s.name: s for s in FULL + PAGE_SHAPES}


def small(spec: Spec) -> Spec:
    """Same structure at sizes the oracle finishes in about a second: several
    256-token tiles, ragged tails, all head/page/dtype parameters unchanged."""
    kind = spec.lens[0]
    if kind == "fixed":
        return spec
    if spec.name.startswith("bf16"):
        return spec.replace(name=spec.name + "_small", num_seqs=5, num_kv_heads=2, lens=("uniform", 1, 1500))
    if spec.name.startswith("fp8tok"):
        return spec.replace(name=spec.name + "_small", num_seqs=4, lens=("uniform", 200, 1400))
    if spec.name.startswith("fp8_trans"):
        return spec.replace(name=spec.name + "_small", num_seqs=4, lens=("fixed", (1024, 1024, 768, 1280)))
    if spec.name.startswith("mxfp4"):
        return spec.replace(name=spec.name + "_small", num_seqs=3, num_kv_heads=2, lens=("fixed", (1, 300, 1100)))
    return spec


# ---------------------------------------------------------------- generation

def _lens(spec: Spec, g: torch.Generator):
    kind = spec.lens[0]
    if kind == "fixed":
        vals = list(spec.lens[1])
        assert len(vals) == spec.num_seqs
        return vals
    if kind == "const":
        return [int(spec.lens[1])] * spec.num_seqs
    lo, hi = spec.lens[1], spec.lens[2]
    return torch.randint(lo, hi + 1, (spec.num_seqs,), generator=g).tolist()


def _randn(shape, g, chunk=1 << 26):
    """float32 N(0,1) drawn in chunks (keeps peak memory bounded)."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=torch.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = torch.randn(e - s, generator=g)
    return out.view(*shape)


def _randn_to(shape, g, dtype, scale=None, chunk=1 << 26):
    """N(0,1) cast to `dtype` chunk by chunk (values divided by `scale` first and
    clamped to the e4m3 range when dtype is float8)."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=dtype)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=g)
        if scale is not None:
            x = x / scale
        if dtype == torch.float8_e4m3fn:
            x = x.clamp_(-448.0, 448.0)
        out[s:e] = x.to(dtype)
    return out.view(*shape)


def _poison_value(kind, fill, g, n):
    """Fill pattern for n unowned elements of a given storage kind."""
    if fill == "zero":
        base = {"bf16": torch.zeros(n, dtype=torch.int16), "u8": torch.zeros(n, dtype=torch.uint8),
                "f32": torch.zeros(n, dtype=torch.float32), "e8m0": torch.zeros(n, dtype=torch.uint8)}
        return base[kind]
    if fill == "random":
        if kind == "bf16":
            return torch.randint(-32768, 32768, (n,), generator=g, dtype=torch.int32).to(torch.int16)
        if kind in ("u8", "e8m0"):
            return torch.randint(0, 256, (n,), generator=g, dtype=torch.int32).to(torch.uint8)
        return torch.randint(-2 ** 31, 2 ** 31, (n,), generator=g, dtype=torch.int64).to(torch.int32).view(
            torch.float32)
    if fill == "nan":
        return {"bf16": torch.full((n,), 0x7FC0, dtype=torch.int16),
                "u8": torch.full((n,), 0xFF, dtype=torch.uint8),
                "f32": torch.full((n,), float("nan")),
                "e8m0": torch.full((n,), 0xFF, dtype=torch.uint8)}[kind]
    if fill == "inf":
        alt = torch.arange(n) % 2 == 0
        if kind == "bf16":
            return torch.where(alt, torch.tensor(0x7F80, dtype=torch.int16),
                               torch.tensor(-128, dtype=torch.int16))  # 0x7F80 / 0xFF80
        if kind == "u8":  # e4m3 has no infinity: +-448 (0x7E / 0xFE)
            return torch.where(alt, torch.tensor(0x7E, dtype=torch.uint8), torch.tensor(0xFE, dtype=torch.uint8))
        if kind == "e8m0":  # largest finite scale, 2^127
            return torch.full((n,), 0xFE, dtype=torch.uint8)
        return torch.where(alt, torch.tensor(float("inf")), torch.tensor(float("-inf")))
    raise ValueError(fill)


def make_case(spec: Spec, fill: Optional[str] = None, seed: Optional[int] = None) -> Case:
    """Build one seeded case on the host. The owned content depends only on
    (spec, seed); `fill` changes only the rows no sequence owns."""
    fill = spec.fill if fill is None else fill
    seed = spec.seed if seed is None else seed
    g = torch.Generator().manual_seed(seed)
    B, QL, H, G, D, PG = spec.num_seqs, spec.qlen, spec.num_kv_heads, spec.q_per_kv, spec.head_dim, spec.page_size
    Hq = H * G
    lens = _lens(spec, g)
    npages = [(L + PG - 1) // PG for L in lens]
    N = sum(npages)
    num_blocks = N + 1
    width = max(npages + [0]) + spec.pad_cols
    perm = (torch.randperm(N, generator=g) + 1).to(torch.int32) if N > 0 else torch.zeros(0, dtype=torch.int32)
    bt = torch.zeros(B, width, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]

    # query
    if spec.q_dtype == "fp8":
        query = _randn_to((B, QL, Hq, D), g, torch.float8_e4m3fn)
    else:
        query = _randn_to((B, QL, Hq, D), g, torch.bfloat16)

    k_scale = v_scale = None
    if spec.kv_dtype == "bf16":
        K = _randn_to((num_blocks, H, PG, D), g, torch.bfloat16)
        V = _randn_to((num_blocks, H, PG, D), g, torch.bfloat16)
    elif spec.kv_dtype == "fp8":
        if spec.scale_mode == "tensor":
            Kf = _randn((num_blocks, H, PG, D), g)
            Vf = _randn((num_blocks, H, PG, D), g)
            ks = float(Kf.abs().max()) / 448.0
            vs = float(Vf.abs().max()) / 448.0
            ks32 = torch.tensor([ks], dtype=torch.float32)
            vs32 = torch.tensor([vs], dtype=torch.float32)
            K = (Kf / ks32).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
            V = (Vf / vs32).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
            del Kf, Vf
            k_scale, v_scale = ks32, vs32
        else:
            K = _randn_to((num_blocks, H, PG, D), g, torch.float8_e4m3fn)
            V = _randn_to((num_blocks, H, PG, D), g, torch.float8_e4m3fn)
            if spec.scale_mode == "token":
                k_scale = torch.rand(num_blocks, H, PG, generator=g) * 0.09 + 0.01
                v_scale = torch.rand(num_blocks, H, PG, generator=g) * 0.09 + 0.01
        K = K.view(torch.uint8)
        V = V.view(torch.uint8)
    elif spec.kv_dtype == "mxfp4":
        K = torch.randint(0, 256, (num_blocks, H, PG, D // 2), generator=g, dtype=torch.int32).to(torch.uint8)
        V = torch.randint(0, 256, (num_blocks, H, PG, D // 2), generator=g, dtype=torch.int32).to(torch.uint8)
        k_scale = torch.randint(spec.mx_k_scale[0], spec.mx_k_scale[1] + 1, (num_blocks, H, PG, D // 32),
                                generator=g, dtype=torch.int32).to(torch.uint8)
        v_scale = torch.randint(118, 137, (num_blocks, H, PG, D // 32), generator=g, dtype=torch.int32).to(
            torch.uint8)
    else:
        raise ValueError(spec.kv_dtype)

    K, V, k_scale, v_scale = _apply_fill(spec.kv_dtype, spec.scale_mode, K, V, k_scale, v_scale, bt, lens, PG,
                                         fill, seed)
    if spec.v_layout == "trans":
        V = V.transpose(2, 3).contiguous()  # [num_blocks, H, D, PG]

    return Case(spec=spec, num_seqs=B, qlen=QL, num_kv_heads=H, q_per_kv=G, head_dim=D, page_size=PG,
                num_blocks=num_blocks, max_blocks_per_seq=width, max_context_len=max(lens + [0]),
                kv_dtype=spec.kv_dtype, scale_mode=spec.scale_mode, v_layout=spec.v_layout, q_dtype=spec.q_dtype,
                softmax_scale=0.0, query=query, key_cache=K, value_cache=V, k_scale=k_scale, v_scale=v_scale,
                block_tables=bt, context_lens=torch.tensor(lens, dtype=torch.int32), causal=spec.causal,
                window=spec.window)


# ---------------------------------------------------------- MXFP4 cache write

@dataclasses.dataclass(frozen=True)
class WriteSpec:
    name: str
    num_seqs: int
    lens: tuple  # as Spec.lens
    num_kv_heads: int
    head_dim: int
    page_size: int
    mode: str  # "fill": positions [0, L) of every sequence (a prefill); "step": position L - 1 only (a decode step)
    pad_tokens: int = 0  # trailing tokens with slot -1
    seed: int = 0

    def replace(self, **kw) -> "WriteSpec":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass
class WriteCase:
    spec: WriteSpec
    num_tokens: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_blocks: int
    key: torch.Tensor
    value: torch.Tensor
    slot_mapping: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    key_scale: torch.Tensor
    value_scale: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor

    def valid_tokens(self) -> int:
        s = self.slot_mapping
        return int(((s >= 0) & (s < self.num_blocks * self.page_size)).sum())

    def bytes_per_token_head(self) -> int:
        """HBM bytes per (token, KV head): K and V read as bf16, written as MXFP4."""
        D = self.head_dim
        return 2 * 2 * D + 2 * (D // 2 + D // 32)

    def bytes_moved(self) -> int:
        return self.valid_tokens() * self.num_kv_heads * self.bytes_per_token_head()


# The pages of the long MXFP4 decode workload (16 sequences x 131072 tokens,
# 4 KV heads, head_dim 128, page 128), written in one prefill-sized call, and
# the one-token-per-sequence write of a decode step on the same cache shape.
MXFP4_WRITE_FILL = WriteSpec("mxfp4_write_fill_b16_l131072", 16, ("const", 131072), 4, 128, 128, "fill", seed=1012)
MXFP4_WRITE_STEP = WriteSpec("mxfp4_write_step_b16_l131072", 16, ("const", 131072), 4, 128, 128, "step", seed=1013)
WRITE_FULL = [MXFP4_WRITE_FILL, MXFP4_WRITE_STEP]


def write_bytes(spec: WriteSpec, part: str = "all") -> int:
    """Algorithmic HBM bytes of one write call of `spec` without building it:
    valid tokens x KV heads x (4 D read; 2 (D/2 + D/32) written)."""
    gh = torch.Generator().manual_seed(spec.seed)  # the same first draw as make_write_case
    lens = _lens(Spec("w", spec.num_seqs, spec.lens, 1, 1, 1, spec.head_dim, spec.page_size, "mxfp4"), gh)
    tokens = sum(lens) if spec.mode == "fill" else sum(1 for L in lens if L > 0)
    D = spec.head_dim
    per = {"read": 4 * D, "write": 2 * (D // 2 + D // 32), "all": 4 * D + 2 * (D // 2 + D // 32)}[part]
    return tokens * spec.num_kv_heads * per


def small_write(spec: WriteSpec) -> WriteSpec:
    """The same structure at oracle-friendly sizes (ragged lengths, padding)."""
    return spec.replace(name=spec.name + "_small", num_seqs=3, num_kv_heads=2, lens=("fixed", (1, 300, 1100)),
                        pad_tokens=5)


def make_write_case(spec: WriteSpec, device="cpu") -> WriteCase:
    """Seeded cache-write inputs, drawn on `device`. K rows are N(0,1) times a
    power of two 2^k, k uniform in [-4, 4], per (KV head, channel), so blocks of
    one row sit at different scales; V rows are N(0,1). The caches hold random
    stale bytes, which rows no token maps to must keep."""
    g = torch.Generator(device=device).manual_seed(spec.seed)
    B, H, D, PG = spec.num_seqs, spec.num_kv_heads, spec.head_dim, spec.page_size
    gh = torch.Generator().manual_seed(spec.seed)  # host draws: lengths and the page permutation
    lens = _lens(Spec("w", B, spec.lens, 1, 1, 1, D, PG, "mxfp4"), gh)
    npages = [(L + PG - 1) // PG for L in lens]
    NP = sum(npages)
    num_blocks = NP + 1
    width = max(npages + [0]) + 2
    perm = (torch.randperm(NP, generator=gh) + 1).to(torch.int32) if NP > 0 else torch.zeros(0, dtype=torch.int32)
    bt = torch.zeros(B, width, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]
    slots = []
    for b in range(B):
        pos = torch.arange(lens[b], dtype=torch.int64) if spec.mode == "fill" else \
            torch.arange(max(lens[b] - 1, 0), lens[b], dtype=torch.int64)
        slots.append(bt[b].to(torch.int64)[pos // PG] * PG + pos % PG)
    slots.append(torch.full((spec.pad_tokens,), -1, dtype=torch.int64))
    slot_mapping = torch.cat(slots).to(torch.int32).to(device)
    N = int(slot_mapping.numel())

    def draw_bf16(shape, scale=None):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = out.view(-1)
        n, step = flat.numel(), 1 << 26
        row = math.prod(shape[1:]) if len(shape) > 1 else 1
        for s0 in range(0, n, step):
            e0 = min(n, s0 + step)
            x = torch.randn(e0 - s0, generator=g, device=device)
            if scale is not None:  # per (head, channel) factor, repeated along tokens
                idx = torch.arange(s0, e0, device=device) % row
                x = x * scale.view(-1)[idx]
            flat[s0:e0] = x.to(torch.bfloat16)
        return out

    kscale = torch.exp2(torch.randint(-4, 5, (H, D), generator=g, device=device).to(torch.float32))
    key = draw_bf16((N, H, D), kscale)
    value = draw_bf16((N, H, D))

    def stale(shape):
        return torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.int32).to(torch.uint8)

    return WriteCase(spec=spec, num_tokens=N, num_kv_heads=H, head_dim=D, page_size=PG, num_blocks=num_blocks,
                     key=key, value=value, slot_mapping=slot_mapping,
                     key_cache=stale((num_blocks, H, PG, D // 2)), value_cache=stale((num_blocks, H, PG, D // 2)),
                     key_scale=stale((num_blocks, H, PG, D // 32)), value_scale=stale((num_blocks, H, PG, D // 32)),
                     block_tables=bt, context_lens=torch.tensor(lens, dtype=torch.int32))


# ------------------------------------------------- MXFP4 paged MQA logits

@dataclasses.dataclass(frozen=True)
class MqaSpec:
    name: str
    num_seqs: int
    lens: tuple  # as Spec.lens
    rows_per_seq: int  # query rows per sequence (1: decode; >1: causal multi-token rows)
    num_heads: int
    head_dim: int
    page_size: int
    pad_rows: int = 0  # trailing rows of no sequence (row_to_batch -1, empty window)
    fill: str = "nan"  # bytes of K rows no window covers: "nan" (0xFF data and scale) or "random"
    seed: int = 0

    def replace(self, **kw) -> "MqaSpec":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass
class MqaCase:
    spec: MqaSpec
    num_rows: int
    num_heads: int
    head_dim: int
    page_size: int
    num_blocks: int
    num_seqs: int
    max_blocks_per_seq: int
    out_stride: int
    q: torch.Tensor            # u8 [R, H, D/2]
    q_scale: torch.Tensor      # u8 [R, H, D/32]
    weights: torch.Tensor      # fp32 [R, H]
    k_cache: torch.Tensor      # u8 [NB, PG, D/2]
    k_scale: torch.Tensor      # u8 [NB, PG, D/32]
    block_tables: torch.Tensor  # int32 [B, W]
    row_to_batch: torch.Tensor  # int32 [R]
    local_starts: torch.Tensor  # int32 [R]
    local_ends: torch.Tensor    # int32 [R]
    context_lens: torch.Tensor  # int32 [B]

    def window_tokens(self) -> int:
        live = self.row_to_batch >= 0
        return int((self.local_ends - self.local_starts).clamp(min=0)[live].sum())

    def bytes_per_row_token(self) -> int:
        """HBM bytes per (row, window position): one K row (data + scales) read, one fp32 score written."""
        D = self.head_dim
        return D // 2 + D // 32 + 4

    def bytes_moved(self) -> int:
        return self.window_tokens() * self.bytes_per_row_token()


# The long MXFP4 decode shape as an indexer: 16 sequences of 131072 tokens,
# one query row each, 64 index heads of 128 (a 4 KB MXFP4 query row), an index
# cache with 64-token pages; and two causal rows per sequence (a multi-token
# step) over 32768 tokens.
MQA_DECODE_LONG = MqaSpec("mqa_mxfp4_h64_p64_b16_l131072", 16, ("const", 131072), 1, 64, 128, 64, seed=1014)
MQA_MTP2 = MqaSpec("mqa_mxfp4_h64_p64_b16_l32768_rows2", 16, ("const", 32768), 2, 64, 128, 64, pad_rows=3,
                   seed=1015)
MQA_FULL = [MQA_DECODE_LONG, MQA_MTP2]


def small_mqa(spec: MqaSpec) -> MqaSpec:
    """Oracle-friendly sizes with ragged lengths, short windows and pad rows."""
    return spec.replace(name=spec.name + "_small", num_seqs=4, lens=("fixed", (1, 77, 300, 1030)), pad_rows=2)


def make_mqa_case(spec: MqaSpec, device="cpu") -> MqaCase:
    """Seeded MQA-logits inputs. Row i of a sequence of length L with n rows
    has the causal window [0, L - n + i + 1); pad rows have row_to_batch -1 and
    an empty window. q and K data bytes are uniform (all 16 e2m1 codes per
    nibble), q scales uniform in [120, 134], K scales in [118, 136], weights
    N(0, 1) / 8. K rows that no window covers hold the fill."""
    g = torch.Generator().manual_seed(spec.seed)
    B, H, D, PG, n = spec.num_seqs, spec.num_heads, spec.head_dim, spec.page_size, spec.rows_per_seq
    lens = _lens(Spec("m", B, spec.lens, 1, 1, 1, D, PG, "mxfp4"), g)
    npages = [(L + PG - 1) // PG for L in lens]
    NP = sum(npages)
    num_blocks = NP + 1
    W = max(npages + [0]) + 2
    perm = (torch.randperm(NP, generator=g) + 1).to(torch.int32) if NP > 0 else torch.zeros(0, dtype=torch.int32)
    bt = torch.zeros(B, W, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]
    rtb, starts, ends = [], [], []
    for b in range(B):
        for i in range(n):
            rtb.append(b)
            starts.append(0)
            ends.append(max(lens[b] - n + i + 1, 0))
    for _ in range(spec.pad_rows):
        rtb.append(-1)
        starts.append(0)
        ends.append(0)
    R = len(rtb)
    out_stride = max([e for e in ends] + [0])
    out_stride = (out_stride + 15) // 16 * 16 + 16
    gd = torch.Generator(device=device).manual_seed(spec.seed + 7)

    def u8(shape, lo, hi):
        return torch.randint(lo, hi, shape, generator=gd, device=device, dtype=torch.int32).to(torch.uint8)

    q = u8((R, H, D // 2), 0, 256)
    q_scale = u8((R, H, D // 32), 120, 135)
    weights = torch.randn((R, H), generator=gd, device=device) / 8
    k_cache = u8((num_blocks, PG, D // 2), 0, 256)
    k_scale = u8((num_blocks, PG, D // 32), 118, 137)
    if spec.fill == "nan":
        # every K row outside the sequences' owned tokens: block 0 and last-page tails
        k_cache[0] = 0xFF
        k_scale[0] = 0xFF
        for b in range(B):
            if lens[b] % PG:
                last = int(bt[b, npages[b] - 1])
                k_cache[last, lens[b] % PG:] = 0xFF
                k_scale[last, lens[b] % PG:] = 0xFF
    return MqaCase(spec=spec, num_rows=R, num_heads=H, head_dim=D, page_size=PG, num_blocks=num_blocks, num_seqs=B,
                   max_blocks_per_seq=W, out_stride=out_stride, q=q, q_scale=q_scale, weights=weights,
                   k_cache=k_cache, k_scale=k_scale, block_tables=bt.to(device),
                   row_to_batch=torch.tensor(rtb, dtype=torch.int32).to(device),
                   local_starts=torch.tensor(starts, dtype=torch.int32).to(device),
                   local_ends=torch.tensor(ends, dtype=torch.int32).to(device),
                   context_lens=torch.tensor(lens, dtype=torch.int32))


def _unowned_pairs(bt, lens, PG):
    """(pages, slots) of every row no sequence owns: all of block 0, then the
    tail of each sequence's last page."""
    pages = [torch.zeros(PG, dtype=torch.int64)]
    slots = [torch.arange(PG, dtype=torch.int64)]
    for b, L in enumerate(lens):
        if L > 0 and L % PG != 0:
            last = int(bt[b, (L + PG - 1) // PG - 1])
            s = torch.arange(L % PG, PG, dtype=torch.int64)
            pages.append(torch.full_like(s, last))
            slots.append(s)
    return torch.cat(pages), torch.cat(slots)


def _apply_fill(kv_dtype, scale_mode, K, V, k_scale, v_scale, bt, lens, PG, fill, seed):
    """Write `fill` into every unowned row of K, V (token-major) and their scales, in place."""
    up, us = _unowned_pairs(bt, lens, PG)
    n_un = int(up.numel())
    H = K.shape[1]
    gp = torch.Generator().manual_seed(seed + 7919)  # poison stream, independent of the owned content

    def poison_rows(t: torch.Tensor, kind: str):
        # t: [num_blocks, H, PG] or [num_blocks, H, PG, X]
        store = t.view(torch.int16) if kind == "bf16" else t
        if t.dim() == 3:
            store[up, :, us] = _poison_value(kind, fill, gp, n_un * H).view(n_un, H)
        else:
            X = t.shape[3]
            store[up, :, us, :] = _poison_value(kind, fill, gp, n_un * H * X).view(n_un, H, X)

    if kv_dtype == "bf16":
        poison_rows(K, "bf16")
        poison_rows(V, "bf16")
    elif kv_dtype == "fp8":
        poison_rows(K, "u8")
        poison_rows(V, "u8")
        if scale_mode == "token":
            poison_rows(k_scale, "f32")
            poison_rows(v_scale, "f32")
    else:
        poison_rows(K, "u8")
        poison_rows(V, "u8")
        poison_rows(k_scale, "e8m0")
        poison_rows(v_scale, "e8m0")
    return K, V, k_scale, v_scale


def refill(case: Case, fill: str, seed: Optional[int] = None) -> Case:
    """A copy of `case` whose unowned rows hold `fill`; owned rows are identical."""
    seed = case.spec.seed if seed is None else seed
    K = case.key_cache.clone()
    V = case.value_cache.clone()
    trans = case.v_layout == "trans"
    if trans:
        V = V.transpose(2, 3).contiguous()
    ks = None if case.k_scale is None else case.k_scale.clone()
    vs = None if case.v_scale is None else case.v_scale.clone()
    if case.kv_dtype == "fp8" and case.scale_mode == "tensor":
        ks, vs = case.k_scale, case.v_scale
    K, V, ks, vs = _apply_fill(case.kv_dtype, case.scale_mode, K, V, ks, vs, case.block_tables,
                               case.context_lens.tolist(), case.page_size, fill, seed)
    if trans:
        V = V.transpose(2, 3).contiguous()
    return dataclasses.replace(case, key_cache=K, value_cache=V, k_scale=ks, v_scale=vs)


def owned_mask(case: Case) -> torch.Tensor:
    """Boolean [num_blocks, page] map of the (page, slot) rows some sequence owns."""
    m = torch.zeros(case.num_blocks, case.page_size, dtype=torch.bool)
    PG = case.page_size
    for b in range(case.num_seqs):
        L = int(case.context_lens[b])
        for j in range((L + PG - 1) // PG):
            p = int(case.block_tables[b, j])
            m[p, :min(PG, L - j * PG)] = True
    return m


def window_start(case: Case, b: int) -> int:
    """s_lo of sequence b: the first token any query row's window covers (0
    without a window). Row i's window ends at e_i = L - qlen + i + 1 when
    causal, else L, and starts W tokens earlier; row 0 starts first."""
    if not getattr(case, "window", 0):
        return 0
    L = int(case.context_lens[b])
    e0 = L - case.qlen + 1 if case.causal else L
    return max(0, e0 - case.window)


def poison_prewindow(case: Case, fill: str, seed: Optional[int] = None) -> Case:
    """A copy of `case` (unowned rows refilled with `fill`) in which everything
    before each sequence's window start s_lo is treated as freed: table
    columns wholly before s_lo point at block 0, and the rows of the page
    holding s_lo that lie before it -- K, V and per-token scales -- hold
    `fill` too. A caller that releases the pages a sliding window has left
    behind leaves exactly this state."""
    seed = case.spec.seed if seed is None else seed
    base = refill(case, fill, seed)
    gp = torch.Generator().manual_seed(seed + 104729)
    K, V = base.key_cache.clone(), base.value_cache.clone()
    token_scales = case.kv_dtype == "fp8" and case.scale_mode == "token"
    ks = base.k_scale.clone() if token_scales else base.k_scale
    vs = base.v_scale.clone() if token_scales else base.v_scale
    bt = base.block_tables.clone()
    PG, H, D = case.page_size, case.num_kv_heads, case.head_dim
    kind = "bf16" if case.kv_dtype == "bf16" else "u8"
    trans = case.v_layout == "trans"
    for b in range(case.num_seqs):
        s = window_start(case, b)
        c, n = s // PG, s % PG
        bt[b, :c] = 0
        if n == 0:
            continue
        p = int(case.block_tables[b, c])
        Ks = K.view(torch.int16) if kind == "bf16" else K
        Vs = V.view(torch.int16) if kind == "bf16" else V
        Ks[p, :, :n, :] = _poison_value(kind, fill, gp, H * n * D).view(H, n, D)
        if trans:
            Vs[p, :, :, :n] = _poison_value(kind, fill, gp, H * D * n).view(H, D, n)
        else:
            Vs[p, :, :n, :] = _poison_value(kind, fill, gp, H * n * D).view(H, n, D)
        if token_scales:
            ks[p, :, :n] = _poison_value("f32", fill, gp, H * n).view(H, n)
            vs[p, :, :n] = _poison_value("f32", fill, gp, H * n).view(H, n)
    return dataclasses.replace(base, key_cache=K, value_cache=V, k_scale=ks, v_scale=vs, block_tables=bt)
