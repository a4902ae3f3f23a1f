"""GPU parity of the precision check with quantization switched off (the
pipelined HCCL AllReduce article, §5.2 gradient anomalies): the fp32
reference sum (bit-exact against the oracle) and the per-unit error report
(maxima bit-exact; sums within the bound that two summation orders of the
same binary64 terms can differ by).

Tolerance of the report's sums, derived from the arithmetic: every term
(|d - ref|, |ref|, d^2, ref^2, d*ref) is computed identically on both sides
(the products of binary32 values are exact in binary64, the difference is
rounded once), and a sum of m terms in any order lies within
gamma_{m-1} = (m-1) u / (1 - (m-1) u), u = 2^-53, times the sum of the
terms' magnitudes from the exact sum.  So the kernel's and the oracle's sums
differ by at most g = 2 gamma_{m-1} times that magnitude; the ratios by at
most 2g relative (plus their own rounding), and the cosine (whose numerator
magnitude is at most sqrt(sum_dd * sum_rr) by Cauchy-Schwarz) by 2g plus a
few ulps absolute."""
import numpy as np
import pytest

from datagen import get_workload
from tests.gpu_util import F16, F32, first_mismatch_f32, same_f32, say, to_device

pytestmark = pytest.mark.gpu

STATS = ("max_abs_err", "max_abs_ref", "max_rel_err", "sum_abs_err", "sum_abs_ref",
         "mean_rel_err", "sum_dd", "sum_rr", "sum_dr", "cos")
EXACT = ("max_abs_err", "max_abs_ref", "max_rel_err")


@pytest.fixture(scope="module")
def gq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from gradient_compression_allreduce_amd import gq as mod
    return mod


def _same_f64(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint64),
                                                     b[~nb].view(np.uint64))


def compare_report(got, want, q, scale, ref, off, label):
    """got, want: [U, 10] float64; q, scale, ref, off: the host inputs."""
    U = off.size - 1
    assert got.shape == want.shape == (U, len(STATS))
    for name in EXACT:
        k = STATS.index(name)
        assert _same_f64(got[:, k], want[:, k]), (label, name,
                                                  np.flatnonzero(got[:, k] != want[:, k])[:5])
    m = np.diff(off).astype(np.float64)
    u = 2.0 ** -53
    g = 2 * (m - 1) * u / (1 - (m - 1) * u)
    start = int(off[0])            # elements before the first unit take no part
    q, ref, off = q[start:int(off[-1])], ref[start:int(off[-1])], off - start
    seg = np.repeat(np.arange(U), np.diff(off))
    d = (q.astype(np.float32) * scale[seg]).astype(np.float64)
    r = ref.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        mag_dr = np.add.reduceat(np.abs(d * r), off[:-1]) if off[-1] > 0 else np.zeros(U)
    for name in STATS:
        if name in EXACT:
            continue
        k = STATS.index(name)
        a, b = got[:, k], want[:, k]
        nan_a, nan_b = np.isnan(a), np.isnan(b)
        assert np.array_equal(nan_a, nan_b), (label, name, "NaN-ness",
                                              np.flatnonzero(nan_a != nan_b)[:5])
        fin = np.isfinite(b) & ~nan_a
        inf = np.isinf(b)
        assert np.array_equal(a[inf], b[inf]), (label, name, "inf")
        if name in ("sum_abs_err", "sum_abs_ref", "sum_dd", "sum_rr"):
            tol = 1.01 * g * np.abs(b)
        elif name == "sum_dr":
            tol = 1.01 * g * mag_dr
        elif name == "mean_rel_err":
            tol = (2.1 * g + 2.0 ** -51) * np.abs(b)
        else:  # cos
            tol = 2.1 * g + 2.0 ** -50
        bad = fin & ~(np.abs(a - b) <= tol)
        assert not np.any(bad), (label, name, np.flatnonzero(bad)[:5], a[bad][:3], b[bad][:3],
                                 np.asarray(tol)[bad][:3] if np.ndim(tol) else tol)


def _offsets(rng, n, lo, hi):
    cuts = [0]
    while cuts[-1] < n:
        cuts.append(min(n, cuts[-1] + int(rng.integers(lo, hi))))
    return np.array(cuts, dtype=np.int64)


def _grads(rng, n, W, kind):
    xs = []
    for _ in range(W):
        g = rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0)
        g[rng.random(n) < 0.02] = 0.0
        if kind == F16:
            xs.append((g * 1024.0).astype(np.float16).view(np.uint16))
        else:
            xs.append(g.astype(np.float32))
    return xs


def _sum_on_gpu(gq, xs, kind, in_mul, mean):
    import torch
    n = xs[0].size
    dx = [to_device(x) for x in xs]
    r = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_sum_f32(dx, r, in_mul=in_mul, mean=mean)
    torch.cuda.synchronize()
    return r.cpu().numpy()


@pytest.mark.parametrize("kind", [F32, F16], ids=["f32", "f16"])
@pytest.mark.parametrize("W", [1, 3, 8, 13, 64])
def test_sum_f32_matches_oracle(gq, oracle, kind, W):
    """Bit-exact rank-order sums (and means) over lengths that end on and
    off a 16-byte slot, from one element to many work groups."""
    rng = np.random.default_rng(300 + W + 7 * kind)
    in_mul = 2.0 ** -10 if kind == F16 else 1.0
    for n in (1, 3, 8, 9, 1023, 4096 * 3 + 5, 250_007):
        xs = _grads(rng, n, W, kind)
        for mean in (False, True):
            say("sum_f32 kind", kind, "W", W, "n", n, "mean", mean)
            got = _sum_on_gpu(gq, xs, kind, in_mul, mean)
            want = oracle.sum_f32(xs, kind, in_mul, mean=mean)
            assert same_f32(got, want), (n, mean, first_mismatch_f32(got, want))


def test_sum_f32_special_values(gq, oracle):
    """-0, subnormals, infinities, NaN, rank-order overflow and cancellation;
    every binary16 pattern with an inexact multiplier."""
    tiny = np.float32(2.0 ** -149)
    base = np.array([0.0, -0.0, tiny, -tiny, 3e38, -3e38, np.inf, -np.inf, np.nan, 1.0,
                     2.0 ** 25, -2.0 ** 25, 1.5], dtype=np.float32)
    xs = [base.copy(), base[::-1].copy(), np.roll(base, 3), (base * np.float32(0.5))]
    for mean in (False, True):
        got = _sum_on_gpu(gq, xs, F32, 1.0, mean)
        assert same_f32(got, oracle.sum_f32(xs, F32, mean=mean))
    bits = np.arange(65536, dtype=np.uint16)
    xs = [bits.copy(), bits[::-1].copy(), np.roll(bits, 12345)]
    for mul in (1.0, 2.0 ** -16, 0.1):
        got = _sum_on_gpu(gq, xs, F16, mul, False)
        assert same_f32(got, oracle.sum_f32(xs, F16, mul)), mul


def _report_on_gpu(gq, units, q, scale, ref):
    import torch
    U = units.n_units
    out = torch.full((U * gq.GQ_STATS,), float("nan"), dtype=torch.float64, device="cuda")
    gq.gq_error_report(torch.from_numpy(q).cuda(), torch.from_numpy(scale).cuda(),
                       torch.from_numpy(ref).cuda(), units, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(U, gq.GQ_STATS)


def test_error_report_random_units(gq, oracle):
    """INT8 result of a real step against the fp32 sum, units from one
    element to several 8192-element tiles, offsets off the 16-byte slots."""
    rng = np.random.default_rng(310)
    n = 300_001
    off = _offsets(rng, n, 1, 40_000)
    extra = _offsets(rng, 3000, 1, 30) + n
    off = np.concatenate([off, extra[1:]])
    n = int(off[-1])
    W = 4
    xs = _grads(rng, n, W, F32)
    res = oracle.allreduce_step(xs, F32, off)
    ref = oracle.sum_f32(xs, F32)
    units = gq.gq_units_create(off)
    got = _report_on_gpu(gq, units, res["q_out"], res["scale_out"], ref)
    want = oracle.error_report(res["q_out"], res["scale_out"], ref, off)
    compare_report(got, want, res["q_out"], res["scale_out"], ref, off, "random")
    # the report repeats bit for bit
    again = _report_on_gpu(gq, units, res["q_out"], res["scale_out"], ref)
    assert _same_f64(got, again)


def test_error_report_chunk_wide_units(gq, oracle):
    """The report on a table of 128 KiB fp32 chunks, which takes chunk-wide
    reduce tiles of 32768 elements (one work group of the report per tile,
    so each group strides over four times its lanes): units of one, two and
    three such tiles and one element more and less, off the 16-byte slots."""
    rng = np.random.default_rng(312)
    lens = [int(v) for v in rng.integers(16385, 32769, 24)]
    for m in (1, 2, 3):
        lens += [32768 * m - 1, 32768 * m, 32768 * m + 1]
    rng.shuffle(lens)
    lens = [5] + lens
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(off[-1])
    W = 3
    xs = _grads(rng, n, W, F32)
    res = oracle.allreduce_step(xs, F32, off)
    ref = oracle.sum_f32(xs, F32)
    units = gq.gq_units_create(off)
    assert gq.gq_units_reduce_tile(units) == 32768
    got = _report_on_gpu(gq, units, res["q_out"], res["scale_out"], ref)
    want = oracle.error_report(res["q_out"], res["scale_out"], ref, off)
    compare_report(got, want, res["q_out"], res["scale_out"], ref, off, "chunk_wide")


def test_error_report_edge_units(gq, oracle):
    """All-zero units, zero codes against a nonzero reference, identical and
    negated vectors (cos exactly 1 and -1), a NaN and an inf reference, and
    an exact dequantized match across several tiles."""
    rng = np.random.default_rng(311)
    parts_q, parts_s, parts_r = [], [], []

    def unit(q, s, r):
        parts_q.append(np.asarray(q, np.int8))
        parts_s.append(np.float32(s))
        parts_r.append(np.asarray(r, np.float32))

    unit(np.zeros(37), 0.0, np.zeros(37))
    unit(np.zeros(20000), 0.5, rng.standard_normal(20000))
    q = rng.integers(-128, 128, 30000)
    s = np.float32(3e-4)
    d = (q.astype(np.float32) * s).astype(np.float32)
    unit(q, s, d)
    unit(q, s, -d)
    unit([1, 2, 3], 1.0, [np.nan, 2.0, 3.0])
    unit([1, 2, 3], 1.0, [np.inf, 2.0, 3.0])
    unit([5], 2.0 ** -140, [0.0])
    unit(q[:9000], np.float32(1e30), (q[:9000].astype(np.float32) * np.float32(1e30)))
    off = np.concatenate([[0], np.cumsum([p.size for p in parts_q])]).astype(np.int64)
    qq = np.concatenate(parts_q)
    ss = np.array(parts_s, np.float32)
    rr = np.concatenate(parts_r)
    units = gq.gq_units_create(off)
    got = _report_on_gpu(gq, units, qq, ss, rr)
    want = oracle.error_report(qq, ss, rr, off)
    compare_report(got, want, qq, ss, rr, off, "edges")
    cos = STATS.index("cos")
    assert got[2, cos] == 1.0 and got[3, cos] == -1.0 and got[0, cos] == 1.0
    assert got[1, cos] == 0.0 and np.isnan(got[4, cos])


@pytest.mark.parametrize("cfg", [2, 5])
def test_check_path_on_workload(gq, oracle, cfg):
    """The whole A/B on a full-size workload: INT8 step on the GPU, fp32 sum
    on the GPU (bit-exact), and the report of one against the other."""
    import torch
    from tests.test_gpu_workloads import unit_offsets
    w = get_workload(cfg)
    kind = F32 if w.kind == "f32" else F16
    off = unit_offsets(w, gq.gq_plan_chunks)
    say("workload", w.name, "W", w.W, "n", w.n)
    xs = [w.fill(r) for r in range(w.W)]
    dx = [to_device(x) for x in xs]
    units = gq.gq_units_create(off)
    U = off.size - 1
    scales = [torch.empty(U, dtype=torch.float32, device="cuda") for _ in range(w.W)]
    codes = [torch.empty(w.n, dtype=torch.int8, device="cuda") for _ in range(w.W)]
    s_out = torch.empty(U, dtype=torch.float32, device="cuda")
    q_out = torch.empty(w.n, dtype=torch.int8, device="cuda")
    ref = torch.empty(w.n, dtype=torch.float32, device="cuda")
    stats = torch.empty(U * gq.GQ_STATS, dtype=torch.float64, device="cuda")
    gq.gq_quantize(dx, units, scales, codes, in_mul=w.in_mul)
    gq.gq_reduce_requantize(codes, scales, units, s_out, q_out)
    gq.gq_sum_f32(dx, ref, in_mul=w.in_mul)
    gq.gq_error_report(q_out, s_out, ref, units, stats)
    torch.cuda.synchronize()
    assert gq.gq_units_faults(units) == 0
    ref_h = ref.cpu().numpy()
    want_ref = oracle.sum_f32(xs, kind, w.in_mul)
    assert same_f32(ref_h, want_ref), first_mismatch_f32(ref_h, want_ref)
    q_h, s_h = q_out.cpu().numpy(), s_out.cpu().numpy()
    want = oracle.allreduce_step(xs, kind, off, w.in_mul)
    assert np.array_equal(q_h, want["q_out"]) and same_f32(s_h, want["scale_out"])
    got = stats.cpu().numpy().reshape(U, gq.GQ_STATS)
    compare_report(got, oracle.error_report(q_h, s_h, ref_h, off), q_h, s_h, ref_h, off,
                   w.name)
    fin = np.isfinite(got[:, STATS.index("cos")])
    say("  worst max_rel_err %.3e, mean of mean_rel_err %.3e, min cos %.6f" % (
        np.nanmax(got[:, STATS.index("max_rel_err")]),
        np.nanmean(got[:, STATS.index("mean_rel_err")]),
        np.min(got[fin, STATS.index("cos")])))
