"""Seeded synthetic gradient workloads (shared input generators).

This package holds only random-number generation and the shapes of the
synthetic workloads.  It contains none of the compression method's
arithmetic (no chunk plan, no scale, no quantization, no reduction): both the
HIP library and the CPU oracle take their inputs from here, and each side
computes its own chunk plan and unit table.
"""
from .native import build, lib  # noqa: F401
from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
