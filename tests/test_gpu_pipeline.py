"""GPU parity of the two-stream bucket pipeline (the article's §2.1 pipeline
scheduling with double buffering, §4.2 pipeline depth 2) and of unit tables
that start past element 0 (which the pipeline's per-bucket tables use):
results equal the oracle's bit for bit, NaN compared by NaN-ness."""
import numpy as np
import pytest

from tests.gpu_util import F16, F32, GpuStep, compare_step, same_f32, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from gradient_compression_allreduce_amd import gq as mod
    return mod


def _grad(rng, n, kind):
    g = rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -1)
    g[rng.random(n) < 0.03] = 0.0
    if kind == F16:
        return (g * 65536.0).astype(np.float16).view(np.uint16)
    return g.astype(np.float32)


def greedy_buckets(unit_bytes, bucket_bytes):
    """Unit indices where buckets start (greedy in order, a unit that would
    overflow a non-empty bucket starts a new one), plus the end."""
    bounds = [0]
    acc = 0
    for u, b in enumerate(unit_bytes):
        if acc > 0 and acc + b > bucket_bytes:
            bounds.append(u)
            acc = 0
        acc += b
    bounds.append(len(unit_bytes))
    return np.array(bounds, dtype=np.int64)


def run_pipe(gq, pipe, xs, W, in_mul, n, U, reps=1, fresh=None):
    import torch
    se, su = gq.gq_pipe_slots(pipe)
    q_slots = [torch.full((se,), 99, dtype=torch.int8, device="cuda") for _ in range(2 * W)]
    s_slots = [torch.full((su,), float("nan"), device="cuda") for _ in range(2 * W)]
    s_out = torch.full((U,), float("nan"), device="cuda")
    q_out = torch.full((n,), 99, dtype=torch.int8, device="cuda")
    dx = [to_device(x) for x in xs]
    for rep in range(reps):
        if fresh is not None and rep > 0:
            for d, x in zip(dx, fresh):
                d.copy_(to_device(x))
        gq.gq_pipe_step(pipe, dx, q_slots, s_slots, s_out, q_out, in_mul=in_mul)
    torch.cuda.synchronize()
    assert gq.gq_pipe_faults(pipe) == 0
    gq.gq_pipe_clear_faults(pipe)
    assert gq.gq_pipe_faults(pipe) == 0
    return (s_out.cpu().numpy(), q_out.cpu().numpy(), [t.cpu().numpy() for t in q_slots],
            [t.cpu().numpy() for t in s_slots])


def check_pipe(gq, oracle, xs, kind, off, bounds, in_mul, label, fresh=None, mode=None,
               schedule=None):
    """Both modes (or `mode`) against the oracle; `schedule`, if given, is the
    schedule the overlap mode must take."""
    if mode is None:
        for m in (gq.GQ_PIPE_OVERLAP, gq.GQ_PIPE_SERIAL):
            check_pipe(gq, oracle, xs, kind, off, bounds, in_mul, label, fresh, m, schedule)
        return
    label = "%s/mode%d" % (label, mode)
    W = len(xs)
    n = int(off[-1])
    U = off.size - 1
    pipe = gq.gq_pipe_create(off, bounds, mode)
    sched = gq.gq_pipe_schedule(pipe, kind, in_mul)
    if mode == gq.GQ_PIPE_SERIAL:
        assert sched == gq.GQ_PIPE_SCHED_SERIAL, (label, sched)
    elif schedule is not None:
        assert sched == schedule, (label, sched)
    label = "%s/sched%d" % (label, sched)
    final = fresh if fresh is not None else xs
    want = oracle.allreduce_step(final, kind, off, in_mul)
    say("pipeline", label, "W", W, "n", n, "units", U, "buckets", bounds.size - 1)
    s_out, q_out, q_slots, s_slots = run_pipe(gq, pipe, xs, W, in_mul, n, U,
                                              reps=2 if fresh is not None else 1, fresh=fresh)
    assert same_f32(s_out, want["scale_out"]), (label, "scale_out")
    bad = np.flatnonzero(q_out != want["q_out"])
    assert bad.size == 0, (label, "q_out", bad[:5])
    # each slot holds the codes and scales of the last bucket that used it
    B = bounds.size - 1
    for b in range(max(0, B - 2), B):
        s = b % 2
        ua, ub = int(bounds[b]), int(bounds[b + 1])
        base = int(off[ua]) & ~15
        lo, hi = int(off[ua]), int(off[ub])
        for w in range(W):
            got_q = q_slots[s * W + w][lo - base:hi - base]
            assert np.array_equal(got_q, want["q"][w][lo:hi]), (label, "slot codes", b, w)
            assert same_f32(s_slots[s * W + w][:ub - ua], want["scale"][w][ua:ub]), (
                label, "slot scales", b, w)
    return pipe


def test_table_starting_past_zero(gq, oracle):
    """A unit table whose first unit starts at element 37: elements before it
    are neither read into a result nor written."""
    import torch
    rng = np.random.default_rng(401)
    start = 37
    lens = [5, 20_000, 1, 70_000, 333, 40_001]
    off = np.concatenate([[start], start + np.cumsum(lens)]).astype(np.int64)
    n = int(off[-1])
    for kind in (F32, F16):
        xs = [_grad(rng, n, kind) for _ in range(3)]
        for x in xs:   # junk before the first unit (NaN)
            x[:start] = np.nan if kind == F32 else 0x7e00
        in_mul = 2.0 ** -16 if kind == F16 else 1.0
        want = oracle.allreduce_step(xs, kind, off, in_mul)
        step = GpuStep(gq, off, 3, kind, n)
        for q in step.codes:
            q.fill_(99)
        step.q_out.fill_(99)
        step.r.fill_(-7.0)
        step.quantize([to_device(x) for x in xs], in_mul)
        step.reduce(fused=True, with_r=True)
        got = step.host()
        for key in ("q", "r", "q_out"):
            arrs = got[key] if key == "q" else [got[key]]
            for a in arrs:
                assert np.all(a[:start] == (99 if key != "r" else -7.0)), (kind, key)
        trim = lambda a: a[start:]
        got_t = dict(got, q=[trim(a) for a in got["q"]], r=trim(got["r"]),
                     q_out=trim(got["q_out"]))
        want_t = dict(want, q=[trim(a) for a in want["q"]], r=trim(want["r"]),
                      q_out=trim(want["q_out"]))
        compare_step(got_t, want_t, 3, check_r=True, label="offset_table_k%d" % kind)
        # the error report and the fp32 reference on the same table
        ref = oracle.sum_f32(xs, kind, in_mul)
        stats = torch.full((U_of(off) * gq.GQ_STATS,), float("nan"), dtype=torch.float64,
                           device="cuda")
        gq.gq_error_report(step.q_out, step.scale_out, torch.from_numpy(ref).cuda(), step.units,
                           stats)
        torch.cuda.synchronize()
        got_rep = stats.cpu().numpy().reshape(U_of(off), gq.GQ_STATS)
        want_rep = oracle.error_report(got["q_out"], got["scale_out"], ref, off)
        from tests.test_gpu_check import compare_report
        compare_report(got_rep, want_rep, got["q_out"], got["scale_out"], ref, off,
                       "offset_report_k%d" % kind)
    torch.cuda.synchronize()


def U_of(off):
    return off.size - 1


@pytest.mark.parametrize("kind", [F32, F16], ids=["f32", "f16"])
def test_pipeline_random_tensors(gq, oracle, kind):
    """Tensors of mixed sizes (unit boundaries off the 16-element grid),
    small buckets so that slots are reused many times."""
    rng = np.random.default_rng(410 + kind)
    sizes = [int(v) for v in rng.integers(1, 60_000, 60)] + [250_003, 7, 120_000]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    esz = 4 if kind == F32 else 2
    bounds = greedy_buckets([s * esz for s in sizes], 400_000)
    assert bounds.size - 1 >= 5
    xs = [_grad(rng, int(off[-1]), kind) for _ in range(4)]
    in_mul = 2.0 ** -16 if kind == F16 else 1.0
    check_pipe(gq, oracle, xs, kind, off, bounds, in_mul, "random_k%d" % kind)


def test_pipeline_chunk_units_and_single_bucket(gq, oracle):
    """Per-chunk units grouped into buckets of whole tensors; and one bucket
    holding everything (no overlap at all)."""
    rng = np.random.default_rng(420)
    sizes = [300_000, 65_536, 1_000, 500_001]
    parts, tensor_first_unit = [np.zeros(1, np.int64)], [0]
    base = 0
    for sz in sizes:
        p = gq.gq_plan_chunks(sz, 4)[1:] + base
        parts.append(p)
        tensor_first_unit.append(tensor_first_unit[-1] + p.size)
        base += sz
    off = np.concatenate(parts)
    xs = [_grad(rng, int(off[-1]), F32) for _ in range(3)]
    bounds = np.array([0, tensor_first_unit[1], tensor_first_unit[3], off.size - 1], np.int64)
    check_pipe(gq, oracle, xs, F32, off, bounds, 1.0, "chunk_units")
    check_pipe(gq, oracle, xs, F32, off, np.array([0, off.size - 1], np.int64), 1.0, "one_bucket")


def test_pipeline_two_steps_in_a_row(gq, oracle):
    """The second step (new inputs, same slots and plan) is not disturbed by
    the first."""
    rng = np.random.default_rng(430)
    sizes = [int(v) for v in rng.integers(1000, 80_000, 30)]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    bounds = greedy_buckets([s * 4 for s in sizes], 300_000)
    n = int(off[-1])
    xs = [_grad(rng, n, F32) * np.float32(1000) for _ in range(5)]
    fresh = [_grad(rng, n, F32) for _ in range(5)]
    check_pipe(gq, oracle, xs, F32, off, bounds, 1.0, "two_steps", fresh=fresh)


def test_pipeline_resnet152_buckets(gq, oracle):
    """The ResNet-152 gradient set (8 ranks, per-layer scales) in its 25 MiB
    buckets, every element against the oracle."""
    from datagen import get_workload
    w = get_workload(2)
    off = w.toff.copy()
    bounds = np.array([a for a, _ in w.buckets] + [len(w.sizes)], dtype=np.int64)
    xs = [w.fill(r) for r in range(w.W)]
    check_pipe(gq, oracle, xs, F32, off, bounds, w.in_mul, w.name,
               schedule=gq.GQ_PIPE_SCHED_ALTERNATE)


def test_pipeline_event_schedule(gq, oracle):
    """A plan whose buckets take the chunk quantize (one work group per
    compute unit) with a unit of several chunk tiles, so that quantize waits
    on its own work groups: the overlap mode then keeps the quantizes on the
    caller's stream and the reduces on the second stream after events, the
    reduce that meets a waiting quantize in its form that never waits."""
    rng = np.random.default_rng(450)
    sizes = [30_000] * 5 + [100_000] + [30_001] * 5 + [100_003] + [29_999] * 5
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    bounds = np.array([0, 6, 12, 17], dtype=np.int64)
    units = gq.gq_units_create(off[:7])
    assert gq.gq_units_schedule(units, gq.GQ_F32) == gq.GQ_SCHED_CHUNK
    xs = [_grad(rng, int(off[-1]), F32) for _ in range(3)]
    check_pipe(gq, oracle, xs, F32, off, bounds, 1.0, "event_schedule",
               schedule=gq.GQ_PIPE_SCHED_EVENTS)


def test_pipeline_tiny_and_odd_buckets(gq, oracle):
    """Buckets of one element, buckets that start and end inside a 16-byte
    slot, a bucket with a unit larger than any tile, and more buckets than
    slots can hold at once."""
    rng = np.random.default_rng(440)
    sizes = [1, 3, 17, 1, 40_000, 5, 1, 33, 100_001, 2, 7, 16, 16, 15]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    bounds = np.array([0, 1, 2, 4, 5, 6, 9, 10, 12, 13, 14], dtype=np.int64)
    for kind in (F32, F16):
        xs = [_grad(rng, int(off[-1]), kind) for _ in range(3)]
        in_mul = 2.0 ** -16 if kind == F16 else 1.0
        check_pipe(gq, oracle, xs, kind, off, bounds, in_mul, "tiny_odd_k%d" % kind)
