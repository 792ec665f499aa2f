"""Paged-attention decode for MI355X (gfx950): a C-ABI HIP library (libpa.so)
with a thin ctypes binding. See include/pa.h for the contract."""
from .binding import (PaError, Plan, pa_decode, pa_decode_direct, pa_decode_static, pa_write_kv_mxfp4, pa_last_error, pa_plan,  # noqa: F401
                      pa_plan_host, pa_version, pa_kv_write_problem, pa_mqa_logits_mxfp4, pa_mqa_problem,
                      mqa_problem_of,
                      make_problem, problem_of, decode_case, device_tensors, lib, LIB_PATH, EXPORTS)
