"""The C ABI driven from C++ alone (tests/c_abi/abi_step.cpp: hipMalloc'd
buffers, its own hipStream_t, no Python tensor library), checked bit for bit
against the oracle: chunk plans, every rank's scales and codes, and the
requantized rank-order sum."""
import ctypes
import os

import numpy as np
import pytest

from tests.conftest import ROOT
from tests.gpu_util import same_f32, say

pytestmark = pytest.mark.gpu

SO = os.path.join(ROOT, "tests", "c_abi", "libabi_step.so")


@pytest.fixture(scope="module")
def drv():
    assert os.path.exists(SO), "tests/c_abi/libabi_step.so is not built (run the build)"
    L = ctypes.CDLL(SO)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.abi_plan.restype = i64
    L.abi_plan.argtypes = [i64, i32, vp, i64]
    L.abi_step.restype = ctypes.c_int
    L.abi_step.argtypes = [vp, i32, i64, vp, i64, vp, vp, vp, vp]
    return L


def test_c_abi_step(drv, oracle):
    rng = np.random.default_rng(501)
    sizes = [300_001, 70_000, 1, 4096, 131_072, 17]
    parts, base = [np.zeros(1, np.int64)], 0
    for sz in sizes:
        cap = sz // 32768 + 8
        off_t = np.empty(cap, dtype=np.int64)
        k = drv.abi_plan(sz, 4, off_t.ctypes.data, cap)
        assert k >= 1
        assert np.array_equal(off_t[:k + 1], oracle.plan_chunks(sz, 4))
        parts.append(off_t[1:k + 1] + base)
        base += sz
    off = np.concatenate(parts)
    n, U, W = int(off[-1]), off.size - 1, 4
    xs = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -1)).astype(np.float32)
          for _ in range(W)]
    xs[1][:1000] = 0.0
    x = np.ascontiguousarray(np.stack(xs))
    scales = np.empty((W, U), np.float32)
    codes = np.empty((W, n), np.int8)
    s_out = np.empty(U, np.float32)
    q_out = np.empty(n, np.int8)
    say("C ABI step: W", W, "n", n, "units", U)
    rc = drv.abi_step(x.ctypes.data, W, n, off.ctypes.data, U, scales.ctypes.data,
                      codes.ctypes.data, s_out.ctypes.data, q_out.ctypes.data)
    assert rc == 0, rc
    want = oracle.allreduce_step(xs, 0, off)
    for w in range(W):
        assert same_f32(scales[w], want["scale"][w]), w
        assert np.array_equal(codes[w], want["q"][w]), w
    assert same_f32(s_out, want["scale_out"])
    assert np.array_equal(q_out, want["q_out"])
