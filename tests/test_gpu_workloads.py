"""GPU parity on the five synthetic workloads at full size, in the launch
shape the benchmark times (fused quantize for all ranks, fused
reduce + requantize without materializing the sum), plus a second reduce
that also writes the fp32 sum.

Every workload is compared with the oracle on every element.  Workloads 1,
2 and 5 run the oracle on the whole workload at once; workloads 3 and 4
(2.7 G and 4.3 G input elements) run it on ranges of whole units in
parallel host threads (units are independent, so a range's result is the
whole-workload result there)."""
import numpy as np
import pytest

from datagen import get_workload
from tests.gpu_util import (F16, F32, GpuStep, compare_step, compare_step_streamed, say,
                            to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from gradient_compression_allreduce_amd import gq as mod
    return mod


def unit_offsets(w, plan):
    """Unit table of a workload from a chunk planner (each side passes its
    own: gq_plan_chunks for the GPU, the oracle's planner for the oracle)."""
    if w.units == "tensor":
        return w.toff.copy()
    parts = [np.zeros(1, dtype=np.int64)]
    for t, size in enumerate(w.sizes):
        p = plan(int(size), w.elem_bytes)
        parts.append(p[1:] + w.toff[t])
    return np.concatenate(parts)


def _kind(w):
    return F32 if w.kind == "f32" else F16


@pytest.mark.parametrize("cfg", [1, 5, 2])
def test_workload_every_element(gq, oracle, cfg):
    w = get_workload(cfg)
    off = unit_offsets(w, gq.gq_plan_chunks)
    assert np.array_equal(off, unit_offsets(w, oracle.plan_chunks))
    say("workload", w.name, "W", w.W, "n", w.n, "units", off.size - 1)
    xs = [w.fill(r) for r in range(w.W)]
    want = oracle.allreduce_step(xs, _kind(w), off, w.in_mul)
    dx = [to_device(x) for x in xs]
    step = GpuStep(gq, off, w.W, _kind(w), w.n)
    # per-layer units take wide reduce tiles, the small-tensor set narrow ones;
    # the small-tensor set takes the chunk schedule, whole tensors the layer one
    assert gq.gq_units_reduce_tile(step.units) == (8192 if cfg == 5 else 16384)
    assert gq.gq_units_schedule(step.units, _kind(w)) == (
        gq.GQ_SCHED_CHUNK if cfg == 5 else gq.GQ_SCHED_LAYER)
    step.quantize(dx, w.in_mul)
    step.reduce(fused=True, with_r=False)
    compare_step(step.host(), want, w.W, check_r=False, label=w.name + "/bench")
    step.reduce(fused=True, with_r=True)
    compare_step(step.host(), want, w.W, check_r=True, label=w.name + "/with_r")
    plan = gq.gq_units_launch_plan(step.units, _kind(w), w.in_mul)
    form = gq.GQ_FORM_SHORT_UNITS if cfg == 5 else gq.GQ_FORM_PERSISTENT
    assert plan["q_form"] == plan["r_form"] == form, plan
    if cfg == 5:
        # the class structure of the small-tensor set really hits the edge rules
        zero_units = np.flatnonzero(want["scale"][0] == 0)
        assert zero_units.size >= 200
        assert np.any(~np.isfinite(want["scale_out"]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [3, 4])
def test_workload_every_element_large(gq, oracle, cfg):
    """The two largest workloads (2.7 G and 4.3 G input elements) at full
    size, every element compared: the GPU step runs once on the whole
    workload, the oracle on ranges of whole units in parallel host threads."""
    import torch
    w = get_workload(cfg)
    kind = _kind(w)
    off = unit_offsets(w, gq.gq_plan_chunks)
    assert np.array_equal(off, unit_offsets(w, oracle.plan_chunks))
    U = off.size - 1
    say("workload", w.name, "W", w.W, "n", w.n, "units", U)
    xs, dx = [], []
    for r in range(w.W):
        xs.append(w.fill(r))
        dx.append(to_device(xs[-1]))
        say("  rank", r, "generated and uploaded")
    step = GpuStep(gq, off, w.W, kind, w.n)
    assert gq.gq_units_schedule(step.units, kind) == gq.GQ_SCHED_CHUNK
    # 128 KiB fp32 chunks fill one chunk-wide reduce tile; 64 Ki-element
    # fp16 chunks span four wide ones
    assert gq.gq_units_reduce_tile(step.units) == (32768 if kind == F32 else 16384)
    # whole 128 KiB fp32 chunks fill 8 rows of a chunk quantize tile; the
    # fp16 table's 65,664-element chunks need 9
    assert gq.gq_units_quantize_tile(step.units, kind) == (32768 if kind == F32 else 73728)
    plan = gq.gq_units_launch_plan(step.units, kind, w.in_mul)
    assert plan["q_form"] == plan["r_form"] == gq.GQ_FORM_PERSISTENT, plan
    step.quantize(dx, w.in_mul)
    step.reduce(fused=True, with_r=False)          # the benchmark's launch shape
    torch.cuda.synchronize()
    q_out_bench = step.q_out.clone()
    s_out_bench = step.scale_out.clone()
    step.reduce(fused=True, with_r=True)           # the same, also writing the sum
    torch.cuda.synchronize()
    assert gq.gq_units_faults(step.units) == 0, "a bounded cross-group wait gave up"
    assert torch.equal(q_out_bench, step.q_out)
    assert torch.equal(s_out_bench.view(torch.int32), step.scale_out.view(torch.int32))
    del dx, q_out_bench, s_out_bench
    nb = compare_step_streamed(oracle, xs, kind, off, w.in_mul, step, w.W, w.name)
    say("  every element of", w.name, "bit-exact (%d unit ranges)" % nb)
