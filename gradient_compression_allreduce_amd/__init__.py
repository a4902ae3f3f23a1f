"""INT8-compressed gradient AllReduce compute for AMD Instinct MI355X.

The package is a thin Python binding (``gq``) over libgq.so, a C-ABI library
of hand-written gfx950 HIP kernels (csrc/).  See include/gq.h for the
contract of every entry point.
"""
from . import gq  # noqa: F401
from .gq import (  # noqa: F401
    Chunker, GQError, Pipe, Units, gq_absmax, gq_chunker_create, gq_chunker_destroy,
    gq_chunker_plan, gq_chunker_predict, gq_chunker_update, gq_error_report, gq_last_error,
    gq_pipe_clear_faults, gq_pipe_create, gq_pipe_destroy, gq_pipe_faults, gq_pipe_slots,
    gq_pipe_step, gq_plan_chunks, gq_quantize, gq_reduce_dequant, gq_reduce_requantize, gq_requantize,
    gq_sum_f32, gq_units_clear_faults, gq_units_create, gq_units_destroy, gq_units_faults,
    gq_units_force_timeout, gq_units_info, gq_units_reduce_tile, gq_units_schedule, gq_version)
