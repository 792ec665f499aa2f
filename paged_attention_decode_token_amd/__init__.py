"""Paged-attention decode for MI355X (gfx950): a C-ABI HIP library (libpa.so)
with a thin ctypes binding. See include/pa.h for the contract."""
from .binding import (PaError, Plan, pa_decode, pa_decode_direct, pa_last_error, pa_plan, pa_plan_host, pa_version,  # noqa: F401
                      make_problem, problem_of, decode_case, device_tensors, lib, LIB_PATH, EXPORTS)
