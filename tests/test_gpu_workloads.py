"""GPU parity on the five synthetic workloads at full size, in the launch
shape the benchmark times (fused quantize for all ranks, fused
reduce + requantize without materializing the sum), plus a second reduce
that also writes the fp32 sum.

Workloads 1, 2 and 5 are compared with the oracle on every element.
Workloads 3 and 4 (2.7 G and 4.3 G input elements) are compared on sampled
units, which the oracle computes one by one from regenerated inputs (units
are independent, so a sampled unit's result is its full-size result)."""
import numpy as np
import pytest

from datagen import get_workload
from tests.gpu_util import F16, F32, GpuStep, compare_step, same_f32, say, to_device

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
    if cfg == 5:
        # the class structure of the small-tensor set really hits the edge rules
        zero_units = np.flatnonzero(want["scale"][0] == 0)
        assert zero_units.size >= 200
        assert np.any(~np.isfinite(want["scale_out"]))


@pytest.mark.parametrize("cfg", [3, 4])
def test_workload_sampled_units(gq, oracle, cfg):
    import torch
    w = get_workload(cfg)
    kind = _kind(w)
    off = unit_offsets(w, gq.gq_plan_chunks)
    assert np.array_equal(off, unit_offsets(w, oracle.plan_chunks))
    U = off.size - 1
    say("workload", w.name, "W", w.W, "n", w.n, "units", U)
    dx = []
    for r in range(w.W):
        dx.append(to_device(w.fill(r)))
        say("  rank", r, "generated and uploaded")
    step = GpuStep(gq, off, w.W, kind, w.n)
    step.quantize(dx, w.in_mul)
    step.reduce(fused=True, with_r=False)
    torch.cuda.synchronize()
    q_out_bench = step.q_out.clone()
    s_out_bench = step.scale_out.clone()
    step.reduce(fused=True, with_r=True)
    torch.cuda.synchronize()
    assert torch.equal(q_out_bench, step.q_out)
    assert torch.equal(s_out_bench.view(torch.int32), step.scale_out.view(torch.int32))
    del dx

    # properties of every unit at full size (the formula's: the element of
    # largest magnitude codes to +-127, and with a normal scale no code is
    # -128), for every rank and for the requantized sum
    lo = np.float32(2.0 ** -126)

    def check_all_units(codes_dev, scale_host, label):
        q = codes_dev.cpu().numpy()
        amax = np.maximum.reduceat(np.abs(q.astype(np.int16)), off[:-1])
        normal = (scale_host >= lo) & np.isfinite(scale_host)
        assert np.all(amax[normal] == 127), (label, np.flatnonzero(amax[normal] != 127)[:5])
        has_min = np.maximum.reduceat((q == -128).astype(np.int8), off[:-1]) > 0
        assert not np.any(has_min & normal), (label, "code -128 with a normal scale")
        assert np.all(scale_host[~normal] == 0), (label, "non-normal scale")

    for r in range(w.W):
        check_all_units(step.codes[r], step.scales[r].cpu().numpy(), "rank %d" % r)
    check_all_units(step.q_out, step.scale_out.cpu().numpy(), "q_out")
    say("  every unit: max|code| = 127, no -128")

    rng = np.random.default_rng(cfg)
    sample = set(int(u) for u in rng.choice(U, 40, replace=False)) | {0, U - 1}
    if cfg == 3:
        sample |= {1, 475, 476, 477}  # word-embedding chunks (above 128 KiB) and the next tensor
    scales = [s.cpu().numpy() for s in step.scales]
    s_out = step.scale_out.cpu().numpy()
    for u in sorted(sample):
        a, b = int(off[u]), int(off[u + 1])
        xs = [w.fill(r, begin=a, end=b) for r in range(w.W)]
        want = oracle.allreduce_step(xs, kind, np.array([0, b - a], dtype=np.int64), w.in_mul)
        for r in range(w.W):
            assert same_f32(scales[r][u:u + 1], want["scale"][r]), (u, r)
            got_q = step.codes[r][a:b].cpu().numpy()
            assert np.array_equal(got_q, want["q"][r]), (u, r)
        assert same_f32(step.r[a:b].cpu().numpy(), want["r"]), u
        assert same_f32(s_out[u:u + 1], want["scale_out"]), u
        assert np.array_equal(step.q_out[a:b].cpu().numpy(), want["q_out"]), u
    say("  sampled units checked:", len(sample))
