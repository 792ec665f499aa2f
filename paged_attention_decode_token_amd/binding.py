"""ctypes binding of libpa.so (include/pa.h): argument marshalling only.

Every step of the decode runs in the HIP kernels behind the C ABI. This module
turns torch tensors into device pointers and checks that they are device
tensors with the layouts the ABI documents; it computes nothing itself. If
libpa.so is missing it raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_OOM = 0, 1, 2, 3, 4
PA_KV_BF16, PA_KV_FP8_E4M3, PA_KV_MXFP4 = 0, 1, 2
PA_SCALE_NONE, PA_SCALE_PER_TENSOR, PA_SCALE_PER_TOKEN = 0, 1, 2
PA_V_PLAIN, PA_V_TRANSPOSED = 0, 1
PA_Q_BF16, PA_Q_FP8_E4M3 = 0, 1

KV_DTYPES = {"bf16": PA_KV_BF16, "fp8": PA_KV_FP8_E4M3, "mxfp4": PA_KV_MXFP4}
SCALE_MODES = {"none": PA_SCALE_NONE, "tensor": PA_SCALE_PER_TENSOR, "token": PA_SCALE_PER_TOKEN}
V_LAYOUTS = {"plain": PA_V_PLAIN, "trans": PA_V_TRANSPOSED}
Q_DTYPES = {"bf16": PA_Q_BF16, "fp8": PA_Q_FP8_E4M3}


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("pa status %d: %s" % (status, msg))
        self.status = status


class pa_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "qlen", "num_kv_heads", "q_per_kv", "head_dim", "page_size", "num_blocks",
        "max_blocks_per_seq", "max_context_len", "kv_dtype", "scale_mode", "v_layout", "q_dtype")] + [
        ("softmax_scale", ctypes.c_float), ("max_partitions", ctypes.c_int32), ("task_budget", ctypes.c_int32),
        ("mxfp4_scaled_qk", ctypes.c_int32), ("causal", ctypes.c_int32), ("window", ctypes.c_int32)]


class pa_plan_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tasks", "max_parts", "total_parts", "tiles_per_task", "merge_needed", "num_cus", "slots")]


class pa_kv_write_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_tokens", "num_kv_heads", "head_dim", "page_size", "num_blocks")]


class pa_mqa_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_rows", "num_heads", "head_dim", "page_size", "num_blocks",
                                              "num_seqs", "max_blocks_per_seq", "out_stride")]


EXPORTS = ["pa_plan", "pa_decode", "pa_decode_direct", "pa_decode_static", "pa_write_kv_mxfp4", "pa_mqa_logits_mxfp4", "pa_plan_destroy", "pa_plan_workspace_bytes", "pa_plan_get_info",
           "pa_plan_host", "pa_plan_set_timing", "pa_plan_read_timing", "pa_last_error", "pa_version"]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libpa.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libpa.so is not built (%s); run `python __graft_entry__.py` or "
                           "`python -m paged_attention_decode_token_amd.build` first" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
    L.pa_plan.restype = ctypes.c_int
    L.pa_plan.argtypes = [P(pa_problem), vp, vp, P(vp)]
    L.pa_decode.restype = ctypes.c_int
    L.pa_decode.argtypes = [vp] * 10
    L.pa_decode_direct.restype = ctypes.c_int
    L.pa_decode_direct.argtypes = [P(pa_problem)] + [vp] * 9
    L.pa_decode_static.restype = ctypes.c_int
    L.pa_decode_static.argtypes = [P(pa_problem)] + [vp] * 9
    L.pa_write_kv_mxfp4.restype = ctypes.c_int
    L.pa_write_kv_mxfp4.argtypes = [P(pa_kv_write_problem)] + [vp] * 8
    L.pa_mqa_logits_mxfp4.restype = ctypes.c_int
    L.pa_mqa_logits_mxfp4.argtypes = [P(pa_mqa_problem)] + [vp] * 11
    L.pa_plan_destroy.restype = None
    L.pa_plan_destroy.argtypes = [vp]
    L.pa_plan_workspace_bytes.restype = ctypes.c_size_t
    L.pa_plan_workspace_bytes.argtypes = [vp]
    L.pa_plan_get_info.restype = ctypes.c_int
    L.pa_plan_get_info.argtypes = [vp, P(pa_plan_info)]
    L.pa_plan_host.restype = ctypes.c_int
    L.pa_plan_host.argtypes = [P(pa_problem), vp, i32, i32, vp, i32, P(i32), vp, P(pa_plan_info)]
    L.pa_plan_set_timing.restype = ctypes.c_int
    L.pa_plan_set_timing.argtypes = [vp, i32, i32]
    L.pa_plan_read_timing.restype = ctypes.c_int
    L.pa_plan_read_timing.argtypes = [vp, P(ctypes.c_double), P(ctypes.c_double), P(i32)]
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_version.restype = ctypes.c_char_p
    L.pa_version.argtypes = []
    _lib = L
    return L


def pa_last_error() -> str:
    return lib().pa_last_error().decode()


def pa_version() -> str:
    return lib().pa_version().decode()


def _check(st: int):
    if st != PA_OK:
        raise PaError(st, pa_last_error())


def make_problem(num_seqs, qlen, num_kv_heads, q_per_kv, head_dim, page_size, num_blocks, max_blocks_per_seq,
                 max_context_len, kv_dtype="bf16", scale_mode="none", v_layout="plain", q_dtype="bf16",
                 softmax_scale=0.0, max_partitions=0, task_budget=0, mxfp4_scaled_qk=0, causal=0,
                 window=0) -> pa_problem:
    return pa_problem(num_seqs, qlen, num_kv_heads, q_per_kv, head_dim, page_size, num_blocks, max_blocks_per_seq,
                      max_context_len, KV_DTYPES.get(kv_dtype, kv_dtype), SCALE_MODES.get(scale_mode, scale_mode),
                      V_LAYOUTS.get(v_layout, v_layout), Q_DTYPES.get(q_dtype, q_dtype), float(softmax_scale),
                      max_partitions, task_budget, int(mxfp4_scaled_qk), int(causal), int(window))


def problem_of(case, **over) -> pa_problem:
    """pa_problem of a paged_attention_decode_token_amd.inputs.Case."""
    kw = dict(num_seqs=case.num_seqs, qlen=case.qlen, num_kv_heads=case.num_kv_heads, q_per_kv=case.q_per_kv,
              head_dim=case.head_dim, page_size=case.page_size, num_blocks=case.num_blocks,
              max_blocks_per_seq=case.max_blocks_per_seq, max_context_len=case.max_context_len,
              kv_dtype=case.kv_dtype, scale_mode=case.scale_mode, v_layout=case.v_layout, q_dtype=case.q_dtype,
              softmax_scale=case.softmax_scale or 0.0, causal=getattr(case, "causal", 0),
              window=getattr(case, "window", 0))
    kw.update(over)
    return make_problem(**kw)


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns a pa_plan_t*; destroyed with the object (or by .close())."""

    def __init__(self, ptr: int, problem: pa_problem):
        self.ptr = ptr
        self.problem = problem

    def info(self) -> pa_plan_info:
        inf = pa_plan_info()
        _check(lib().pa_plan_get_info(self.ptr, ctypes.byref(inf)))
        return inf

    def workspace_bytes(self) -> int:
        return int(lib().pa_plan_workspace_bytes(self.ptr))

    def set_timing(self, enable: bool, max_calls: int = 1024):
        _check(lib().pa_plan_set_timing(self.ptr, int(bool(enable)), int(max_calls)))

    def read_timing(self):
        t, m, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
        _check(lib().pa_plan_read_timing(self.ptr, ctypes.byref(t), ctypes.byref(m), ctypes.byref(n)))
        return t.value, m.value, n.value

    def close(self):
        if self.ptr:
            lib().pa_plan_destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pa_plan(problem: pa_problem, host_context_lens=None, stream=None) -> Plan:
    lens_buf = None
    if host_context_lens is not None:
        t = torch.as_tensor(host_context_lens, dtype=torch.int32).cpu().contiguous()
        lens_buf = t
    out = ctypes.c_void_p()
    st = lib().pa_plan(ctypes.byref(problem), None if lens_buf is None else ctypes.c_void_p(lens_buf.data_ptr()),
                       ctypes.c_void_p(_stream_ptr(stream)), ctypes.byref(out))
    _check(st)
    return Plan(out.value, problem)


def _dev(t, name, nullable=False):
    if t is None:
        if nullable:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a device (cuda) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _check_decode_sizes(p: pa_problem, query, key_cache, value_cache, k_scale, v_scale, block_tables,
                        context_lens, out):
    """The C ABI sees only pointers: check here that every tensor holds exactly
    the bytes the problem implies for its format and layout."""
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    B, QL, H, D, PG, NB = p.num_seqs, p.qlen, p.num_kv_heads, p.head_dim, p.page_size, p.num_blocks
    Hq = H * p.q_per_kv
    row = {PA_KV_BF16: 2 * D, PA_KV_FP8_E4M3: D, PA_KV_MXFP4: D // 2}[p.kv_dtype]
    need = [(query, "query", B * QL * Hq * D * (1 if p.q_dtype == PA_Q_FP8_E4M3 else 2)),
            (key_cache, "key_cache", NB * H * PG * row), (value_cache, "value_cache", NB * H * PG * row),
            (out, "out", B * QL * Hq * D * 2), (context_lens, "context_lens", B * 4)]
    if p.kv_dtype == PA_KV_MXFP4:
        need += [(k_scale, "k_scale", NB * H * PG * (D // 32)), (v_scale, "v_scale", NB * H * PG * (D // 32))]
    elif p.scale_mode == PA_SCALE_PER_TOKEN:
        need += [(k_scale, "k_scale", NB * H * PG * 4), (v_scale, "v_scale", NB * H * PG * 4)]
    elif p.scale_mode == PA_SCALE_PER_TENSOR:
        need += [(k_scale, "k_scale", 4), (v_scale, "v_scale", 4)]
    for t, name, nbytes in need:
        if t is None:
            raise ValueError("%s is required" % name)
        if t.numel() * t.element_size() != nbytes:
            raise ValueError("%s holds %d bytes, the problem needs %d" % (name, t.numel() * t.element_size(), nbytes))
    if tuple(block_tables.shape) != (B, p.max_blocks_per_seq):
        raise ValueError("block_tables has shape %s, the problem needs %s" % (
            tuple(block_tables.shape), (B, p.max_blocks_per_seq)))


def pa_decode(plan: Plan, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, out,
              stream=None):
    """Enqueue one decode on `stream` (torch's current stream by default)."""
    _check_decode_sizes(plan.problem, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens,
                        out)
    st = lib().pa_decode(ctypes.c_void_p(plan.ptr), _dev(query, "query"), _dev(key_cache, "key_cache"),
                         _dev(value_cache, "value_cache"), _dev(k_scale, "k_scale", True),
                         _dev(v_scale, "v_scale", True), _dev(block_tables, "block_tables"),
                         _dev(context_lens, "context_lens"), _dev(out, "out"),
                         ctypes.c_void_p(_stream_ptr(stream)))
    _check(st)
    return out


def pa_decode_direct(problem: pa_problem, query, key_cache, value_cache, k_scale, v_scale, block_tables,
                     context_lens, out, stream=None):
    """Plan-free decode (one task per sequence and KV head); enqueued on `stream`."""
    _check_decode_sizes(problem, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, out)
    st = lib().pa_decode_direct(ctypes.byref(problem), _dev(query, "query"), _dev(key_cache, "key_cache"),
                                _dev(value_cache, "value_cache"), _dev(k_scale, "k_scale", True),
                                _dev(v_scale, "v_scale", True), _dev(block_tables, "block_tables"),
                                _dev(context_lens, "context_lens"), _dev(out, "out"),
                                ctypes.c_void_p(_stream_ptr(stream)))
    _check(st)
    return out


def pa_decode_static(problem: pa_problem, query, key_cache, value_cache, k_scale, v_scale, block_tables,
                     context_lens, out, stream=None):
    """Allocation-free decode (uniform partitions, partials in the library's
    static device buffer); enqueued on `stream`."""
    _check_decode_sizes(problem, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, out)
    st = lib().pa_decode_static(ctypes.byref(problem), _dev(query, "query"), _dev(key_cache, "key_cache"),
                                _dev(value_cache, "value_cache"), _dev(k_scale, "k_scale", True),
                                _dev(v_scale, "v_scale", True), _dev(block_tables, "block_tables"),
                                _dev(context_lens, "context_lens"), _dev(out, "out"),
                                ctypes.c_void_p(_stream_ptr(stream)))
    _check(st)
    return out


def pa_plan_host(problem: pa_problem, host_context_lens=None, num_cus: int = 256, blocks_per_cu: int = 2):
    """Host-only planner: (tasks int32 [n, 4], pair_parts int32 [B * Hkv, 2], info)."""
    lens_buf = None if host_context_lens is None else torch.as_tensor(host_context_lens, dtype=torch.int32).contiguous()
    n = ctypes.c_int32()
    info = pa_plan_info()
    lp = None if lens_buf is None else ctypes.c_void_p(lens_buf.data_ptr())
    _check(lib().pa_plan_host(ctypes.byref(problem), lp, num_cus, blocks_per_cu, None, 0, ctypes.byref(n), None,
                              ctypes.byref(info)))
    npairs = max(1, problem.num_seqs * problem.num_kv_heads)
    tasks = torch.zeros((max(1, n.value), 4), dtype=torch.int32)
    parts = torch.zeros((npairs, 2), dtype=torch.int32)
    _check(lib().pa_plan_host(ctypes.byref(problem), lp, num_cus, blocks_per_cu, ctypes.c_void_p(tasks.data_ptr()),
                              n.value, ctypes.byref(n), ctypes.c_void_p(parts.data_ptr()), ctypes.byref(info)))
    return tasks[:n.value], parts[:problem.num_seqs * problem.num_kv_heads], info


def device_tensors(case, device="cuda"):
    """Copy a Case's host tensors to the device (dict of torch tensors)."""
    return {k: (None if v is None else v.to(device)) for k, v in case.tensors().items()}


def decode_case(case, plan=None, out=None, stream=None, **problem_over):
    """Plan (with host lengths) and decode a Case; returns (out bf16 device tensor, plan)."""
    d = device_tensors(case)
    if plan is None:
        plan = pa_plan(problem_of(case, **problem_over), case.context_lens, stream)
    if out is None:
        out = torch.full((case.num_seqs, case.qlen, case.num_q_heads, case.head_dim), float("nan"),
                         dtype=torch.bfloat16, device="cuda")
    pa_decode(plan, d["query"], d["key_cache"], d["value_cache"], d["k_scale"], d["v_scale"], d["block_tables"],
              d["context_lens"], out, stream)
    return out, plan


def pa_write_kv_mxfp4(key, value, slot_mapping, key_cache, value_cache, key_scale, value_scale, stream=None,
                      problem: Optional[pa_kv_write_problem] = None):
    """Enqueue the MXFP4 KV-cache write on `stream`.

    key, value: bf16 [num_tokens, Hkv, D]; slot_mapping: int32 [num_tokens];
    key_cache, value_cache: uint8 [blocks, Hkv, page, D/2]; key_scale,
    value_scale: uint8 [blocks, Hkv, page, D/32]. The sizes come from the
    tensors unless `problem` is given (then it is passed through as is)."""
    if problem is None:
        if key.dim() != 3 or key_cache.dim() != 4:
            raise ValueError("key must be [tokens, heads, head_dim] and key_cache [blocks, heads, page, head_dim/2]")
        if key.dtype != torch.bfloat16 or value.dtype != torch.bfloat16:
            raise ValueError("key and value must be bfloat16")
        if slot_mapping.dtype != torch.int32:
            raise ValueError("slot_mapping must be int32")
        for t, name in ((key_cache, "key_cache"), (value_cache, "value_cache"), (key_scale, "key_scale"),
                        (value_scale, "value_scale")):
            if t.dtype != torch.uint8:
                raise ValueError("%s must be uint8" % name)
        N, H, D = key.shape
        NB, HC, PG, DB = key_cache.shape
        if (value.shape != key.shape or tuple(slot_mapping.shape) != (N,) or HC != H or DB * 2 != D
                or value_cache.shape != key_cache.shape or tuple(key_scale.shape) != (NB, H, PG, D // 32)
                or value_scale.shape != key_scale.shape):
            raise ValueError("inconsistent shapes for the MXFP4 KV write")
        problem = pa_kv_write_problem(N, H, D, PG, NB)
    st = lib().pa_write_kv_mxfp4(ctypes.byref(problem), _dev(key, "key"), _dev(value, "value"),
                                 _dev(slot_mapping, "slot_mapping"), _dev(key_cache, "key_cache"),
                                 _dev(value_cache, "value_cache"), _dev(key_scale, "key_scale"),
                                 _dev(value_scale, "value_scale"), ctypes.c_void_p(_stream_ptr(stream)))
    _check(st)


def mqa_problem_of(case) -> pa_mqa_problem:
    """pa_mqa_problem of a paged_attention_decode_token_amd.inputs.MqaCase."""
    return pa_mqa_problem(case.num_rows, case.num_heads, case.head_dim, case.page_size, case.num_blocks,
                          case.num_seqs, case.max_blocks_per_seq, case.out_stride)


def pa_mqa_logits_mxfp4(problem: pa_mqa_problem, q, q_scale, weights, k_cache, k_scale, block_tables, row_to_batch,
                        local_starts, local_ends, out, stream=None):
    """Enqueue the MXFP4 paged MQA logits on `stream`; writes only window positions of `out`.

    The tensors must have the shapes `problem` describes (checked here, since the
    C ABI sees only pointers): q [R, H, D/2], q_scale [R, H, D/32], weights [R, H],
    k_cache [NB, PG, D/2], k_scale [NB, PG, D/32], block_tables [B, W],
    row_to_batch / local_starts / local_ends [R], out [R, out_stride]."""
    p = problem
    R, H, D, NB, PG = p.num_rows, p.num_heads, p.head_dim, p.num_blocks, p.page_size
    for t, name, dt, shape in ((q, "q", torch.uint8, (R, H, D // 2)),
                               (q_scale, "q_scale", torch.uint8, (R, H, D // 32)),
                               (weights, "weights", torch.float32, (R, H)),
                               (k_cache, "k_cache", torch.uint8, (NB, PG, D // 2)),
                               (k_scale, "k_scale", torch.uint8, (NB, PG, D // 32)),
                               (block_tables, "block_tables", torch.int32, (p.num_seqs, p.max_blocks_per_seq)),
                               (row_to_batch, "row_to_batch", torch.int32, (R,)),
                               (local_starts, "local_starts", torch.int32, (R,)),
                               (local_ends, "local_ends", torch.int32, (R,)),
                               (out, "out", torch.float32, (R, p.out_stride))):
        if t.dtype != dt:
            raise ValueError("%s must be %s" % (name, dt))
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, the problem needs %s" % (name, tuple(t.shape), shape))
    st = lib().pa_mqa_logits_mxfp4(ctypes.byref(problem), _dev(q, "q"), _dev(q_scale, "q_scale"),
                                   _dev(weights, "weights"), _dev(k_cache, "k_cache"), _dev(k_scale, "k_scale"),
                                   _dev(block_tables, "block_tables"), _dev(row_to_batch, "row_to_batch"),
                                   _dev(local_starts, "local_starts"), _dev(local_ends, "local_ends"),
                                   _dev(out, "out"), ctypes.c_void_p(_stream_ptr(stream)))
    _check(st)
    return out
