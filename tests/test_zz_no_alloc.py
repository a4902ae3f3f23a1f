"""gq_quantize_noalloc (no unit table, maxima in the library's fixed device
array) against gq_quantize with computed maxima through a unit table: bit
for bit on two calls in a row, the second on a smaller input, so that
anything the first call left in the shared array would show; also against
the oracle.  Called through the C ABI (the binding only marshals)."""
import numpy as np
import pytest

from tests.gpu_util import F16, F32, first_mismatch_f32, same_f32, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from gradient_compression_allreduce_amd import gq as mod
    return mod


def _case(rng, W, kind, units, first, sigma):
    """W gradients of one unit table: unit lengths `units`, the first unit at
    element `first` (the elements before it belong to no unit); a few units
    all zero, subnormal, or holding inf / NaN."""
    off = (first + np.concatenate([[0], np.cumsum(units)])).astype(np.int64)
    n = int(off[-1])
    xs = []
    for w in range(W):
        g = (rng.standard_normal(n) * sigma).astype(np.float32)
        U = len(units)
        for u in rng.choice(U, min(U, 6), replace=False):
            a, b = off[u], off[u + 1]
            kindu = int(rng.integers(0, 4))
            if kindu == 0:
                g[a:b] = 0.0
            elif kindu == 1:
                g[a:b] = (rng.integers(-300, 300, b - a) * 2.0 ** -149).astype(np.float32)
            elif kind == F32 and kindu == 2:
                g[a + (b - a) // 2] = np.inf
            elif kind == F32:
                g[a] = np.nan
        if kind == F16:
            xs.append((g * 65536.0).astype(np.float16).view(np.uint16))
        else:
            xs.append(g)
    return off, xs


def _both(gq, oracle, off, xs, kind, in_mul, label):
    import torch
    W = len(xs)
    n, U = int(off[-1]), off.size - 1
    say("case", label, "W", W, "n", n, "units", U, "first", int(off[0]))
    dx = [to_device(x) for x in xs]
    d_off = torch.from_numpy(off.copy()).cuda()
    units = gq.gq_units_create(off)
    sc_ref = [torch.full((U,), 7.0, device="cuda") for _ in range(W)]
    q_ref = [torch.full((n,), 99, dtype=torch.int8, device="cuda") for _ in range(W)]
    sc = [torch.full((U,), -5.0, device="cuda") for _ in range(W)]
    q = [torch.full((n,), 99, dtype=torch.int8, device="cuda") for _ in range(W)]
    gq.gq_quantize(dx, units, sc_ref, q_ref, in_mul=in_mul)
    gq.gq_quantize_noalloc(dx, off, d_off, sc, q, in_mul=in_mul)
    torch.cuda.synchronize()
    assert gq.gq_units_faults(units) == 0
    h0 = int(off[0])
    for w in range(W):
        a, b = sc[w].cpu().numpy(), sc_ref[w].cpu().numpy()
        assert same_f32(a, b), (label, "scale", w, first_mismatch_f32(a, b))
        qa, qb = q[w].cpu().numpy(), q_ref[w].cpu().numpy()
        bad = np.flatnonzero(qa != qb)
        assert bad.size == 0, (label, "codes", w, int(bad[0]), int(qa[bad[0]]), int(qb[bad[0]]))
        assert np.all(qa[:h0] == 99), (label, "wrote before the first unit")
        # and the definition, by the oracle (on the unit range)
        _, s_o, q_o = oracle.quantize_units(xs[w][h0:], kind, off - h0, in_mul)
        assert same_f32(a, s_o), (label, "oracle scale", w, first_mismatch_f32(a, s_o))
        assert np.array_equal(qa[h0:], q_o), (label, "oracle codes", w)


def test_noalloc_matches_quantize_two_calls(gq, oracle):
    """Call 1 at the array's full size (W * n_units = 2^20, units of 1 to 40
    elements, first unit at element 3, values of scale 1); call 2 right
    after on a smaller input whose units reuse the first ones' words with
    values a thousand times smaller (a word the first call left behind
    would show as a wrong scale)."""
    rng = np.random.default_rng(910)
    W1 = 4
    U1 = gq.GQ_NOALLOC_MAX_MAXIMA // W1
    units1 = rng.integers(1, 41, U1)
    off1, xs1 = _case(rng, W1, F32, units1, 3, 1.0)
    _both(gq, oracle, off1, xs1, F32, 1.0, "full_array")
    units2 = np.concatenate([rng.integers(1, 20, 3000), [40000, 5, 100_003, 17]])
    off2, xs2 = _case(rng, 3, F32, units2, 0, 1e-3)
    _both(gq, oracle, off2, xs2, F32, 1.0, "smaller_after")


def test_noalloc_fp16_and_long_units(gq, oracle):
    """fp16 with the 2^-16 unscale, units much longer and much shorter than
    a work group's range, starting at every offset modulo 16."""
    rng = np.random.default_rng(911)
    units = np.concatenate([[1, 2, 3, 5, 7, 8, 9, 15, 16, 17], [8191, 8192, 8193],
                            rng.integers(1, 300, 200), [1_000_000, 70_001], rng.integers(1, 9, 50)])
    off, xs = _case(rng, 5, F16, units, 13, 1e-2)
    _both(gq, oracle, off, xs, F16, 2.0 ** -16, "fp16_mixed")
    off, xs = _case(rng, 64, F32, np.array([33_333, 1, 4096 * 3]), 0, 1.0)
    _both(gq, oracle, off, xs, F32, 1.0, "sixty_four_ranks")


def test_noalloc_rejects_too_many_maxima(gq):
    import torch
    W = 2
    U = gq.GQ_NOALLOC_MAX_MAXIMA // W + 1
    off = np.arange(U + 1, dtype=np.int64)
    d_off = torch.from_numpy(off).cuda()
    xs = [torch.zeros(U, device="cuda") for _ in range(W)]
    sc = [torch.full((U,), 7.0, device="cuda") for _ in range(W)]
    q = [torch.full((U,), 5, dtype=torch.int8, device="cuda") for _ in range(W)]
    with pytest.raises(gq.GQError) as e:
        gq.gq_quantize_noalloc(xs, off, d_off, sc, q)
    assert e.value.status == gq.GQ_ERR_INVALID and "limit" in str(e.value)
    torch.cuda.synchronize()
    assert float(sc[0][0]) == 7.0 and int(q[1][-1]) == 5
