"""INT8-compressed gradient AllReduce compute for AMD Instinct MI355X.

The package is a thin Python binding (``gq``) over libgq.so, a C-ABI library
of hand-written gfx950 HIP kernels (csrc/).  See include/gq.h for the
contract of every entry point.
"""
from . import gq  # noqa: F401
from .gq import (  # noqa: F401
    GQError, Units, gq_absmax, gq_last_error, gq_plan_chunks, gq_quantize,
    gq_reduce_dequant, gq_reduce_requantize, gq_requantize, gq_units_create,
    gq_units_destroy, gq_units_faults, gq_units_info, gq_units_schedule, gq_version)
