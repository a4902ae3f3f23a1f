"""Host logic of the benchmark's parity pass and of the tests' streamed
comparison, checked on the CPU: the outputs stand in for a GPU step's (they
are the oracle's own whole-workload outputs, then copies with planted
differences), so these tests need no device."""
import types

import numpy as np
import pytest

from datagen import get_workload


def _small_case(oracle, T=120, W=3):
    w = get_workload(5)
    off = w.toff[:T + 1].copy()
    n = int(off[-1])
    xs = [w.fill(r, begin=0, end=n) for r in range(W)]
    want = oracle.allreduce_step(xs, 0, off)
    wl = types.SimpleNamespace(W=W, n=n, elem_bytes=4, in_mul=1.0)
    return wl, xs, off, want


def _got(want, W):
    codes = [q.copy() for q in want["q"]]
    r = want["r"].copy()
    q_out = want["q_out"].copy()
    return {"scale": [s.copy() for s in want["scale"]],
            "scale_out": want["scale_out"].copy(),
            "codes": lambda w, a, b: codes[w][a:b],
            "r": lambda a, b: r[a:b],
            "q_out": lambda a, b: q_out[a:b],
            "_codes": codes, "_r": r, "_q_out": q_out}


def test_unit_batches_cover_every_unit_once():
    import bench
    from tests.gpu_util import unit_batches
    rng = np.random.default_rng(4)
    off = np.concatenate([[0], np.cumsum(rng.integers(1, 5000, 777))]).astype(np.int64)
    for fn in (bench.unit_batches, unit_batches):
        for min_elems in (1, 100, 4096, 100_000, 1 << 40):
            b = fn(off, min_elems)
            assert b[0][0] == 0 and b[-1][1] == off.size - 1
            assert all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
            assert all(ub > ua for ua, ub in b)
            assert all(off[ub] - off[ua] >= min_elems for ua, ub in b[:-1])


def test_bench_parity_pass_exact_and_planted(oracle):
    import bench
    wl, xs, off, want = _small_case(oracle)
    got = _got(want, wl.W)
    parity, base = bench.oracle_check(wl, xs, off, 0, got, min_seconds=0.0, batch_elems=5000)
    assert parity["bit_exact"] and parity["first_mismatch"] is None
    assert parity["unit_batches"] > 5
    U = off.size - 1
    assert parity["compared"] == {"codes": wl.W * wl.n, "scales": wl.W * U, "r": wl.n,
                                  "scale_out": U, "q_out": wl.n}
    assert base["cores"] == 1 and base["kind"] == "oracle" and base["value"] > 0

    # one wrong code of rank 2, one sum of different sign, one scale off by
    # one ulp: each counted once, the first range named
    i = int(off[77]) + 3
    got["_codes"][2][i] ^= 1
    got["_r"][5] = -got["_r"][5] if got["_r"][5] != 0 else np.float32(1e-30)
    got["scale_out"][100] = np.nextafter(got["scale_out"][100], np.float32(np.inf))
    parity, _ = bench.oracle_check(wl, xs, off, 0, got, min_seconds=0.0, batch_elems=5000)
    assert not parity["bit_exact"]
    assert parity["mismatches"] == {"codes": 1, "scales": 0, "r": 1, "scale_out": 1, "q_out": 0}
    assert parity["first_mismatch"]["units"][0] == 0


def test_bench_parity_nan_by_nan_ness():
    import bench
    a = np.array([np.nan, 1.0, -0.0], np.float32)
    b = np.array([-np.nan, 1.0, -0.0], np.float32)
    assert bench.f32_mismatches(a, b) == 0
    b[2] = 0.0
    assert bench.f32_mismatches(a, b) == 1
    b[0] = 1.0
    assert bench.f32_mismatches(a, b) == 2


def test_streamed_comparison_exact_and_planted(oracle):
    import torch
    from tests.gpu_util import compare_step_streamed
    wl, xs, off, want = _small_case(oracle, T=200, W=4)
    step = types.SimpleNamespace(
        scales=[torch.from_numpy(s.copy()) for s in want["scale"]],
        codes=[torch.from_numpy(q.copy()) for q in want["q"]],
        r=torch.from_numpy(want["r"].copy()),
        scale_out=torch.from_numpy(want["scale_out"].copy()),
        q_out=torch.from_numpy(want["q_out"].copy()))
    nb = compare_step_streamed(oracle, xs, 0, off, 1.0, step, wl.W, "cpu", batch_elems=3000,
                               threads=3)
    assert nb > 10
    step.codes[3][int(off[150])] += 1
    with pytest.raises(AssertionError, match="codes"):
        compare_step_streamed(oracle, xs, 0, off, 1.0, step, wl.W, "cpu", batch_elems=3000,
                              threads=3)
    step.codes[3][int(off[150])] -= 1
    step.q_out[-1] += 1
    with pytest.raises(AssertionError, match="q_out"):
        compare_step_streamed(oracle, xs, 0, off, 1.0, step, wl.W, "cpu", batch_elems=3000,
                              threads=3)


def test_input_checksums_are_per_rank_fnv1a():
    import bench
    w = get_workload(1)
    xs = [w.fill(r, begin=0, end=4096) for r in range(3)]
    cs = bench.input_checksums(w, xs)
    assert len(cs) == 3 and len(set(cs)) == 3
    # FNV-1a 64 of the bytes, from its published definition
    h = 0xcbf29ce484222325
    for byte in xs[1].tobytes():
        h = ((h ^ byte) * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    assert cs[1] == "%016x" % h
