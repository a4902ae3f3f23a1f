"""The binding's argument guards, on the CPU: every tensor's device,
dtype, contiguity and size, and every list's length, are checked before
the library is called, so a short or mistyped buffer can never become an
out-of-bounds device access.  Tensors are stand-ins with the attributes the
guards read; the library is replaced by a stub that fails the test if it is
reached (except where a valid call is meant to reach it)."""
import ctypes
import types

import pytest
import torch


class Reached(Exception):
    pass


class StubLib:
    """Any entry point called raises Reached (records the name)."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*a):
            self.calls.append(name)
            raise Reached(name)
        return f


class Fake:
    """What the guards read of a tensor."""

    def __init__(self, numel, dtype, cuda=True, contiguous=True, device=0):
        self._n, self.dtype, self.is_cuda, self._c = numel, dtype, cuda, contiguous
        self.device = types.SimpleNamespace(index=device if cuda else None)

    def numel(self):
        return self._n

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return 0x10000

    def get_device(self):
        return self.device.index if self.is_cuda else -1


@pytest.fixture()
def env(monkeypatch):
    from gradient_compression_allreduce_amd import gq
    stub = StubLib()
    monkeypatch.setattr(gq, "lib", stub)
    monkeypatch.setattr(gq, "_current_device", lambda: 0)
    monkeypatch.setattr(gq, "_stream", lambda s: ctypes.c_void_p(0))
    units = gq.Units.__new__(gq.Units)
    units.handle, units.n, units.n_units = ctypes.c_void_p(1), 1000, 10
    pipe = gq.Pipe.__new__(gq.Pipe)
    pipe.handle, pipe.n, pipe.n_units, pipe.n_buckets = ctypes.c_void_p(1), 1000, 10, 2
    monkeypatch.setattr(gq, "gq_pipe_slots", lambda p: (600, 6))
    yield gq, stub, units, pipe
    units.handle = ctypes.c_void_p()   # never destroyed through the real library
    pipe.handle = ctypes.c_void_p()


F32, F16, I8, I32, F64 = torch.float32, torch.float16, torch.int8, torch.int32, torch.float64


def _q_args(W=3, n=1000, U=10):
    return ([Fake(n, F32) for _ in range(W)], [Fake(U, F32) for _ in range(W)],
            [Fake(n, I8) for _ in range(W)])


def test_valid_calls_reach_the_library(env):
    gq, stub, units, pipe = env
    xs, sc, cd = _q_args()
    calls = [
        lambda: gq.gq_quantize(xs, units, sc, cd),
        lambda: gq.gq_quantize(xs, units, sc, cd, amax_bits=Fake(30, I32)),
        lambda: gq.gq_absmax(xs, units, Fake(30, torch.uint32)),
        lambda: gq.gq_reduce_dequant(cd, sc, units, Fake(1000, F32)),
        lambda: gq.gq_requantize(Fake(1000, F32), units, Fake(10, F32), Fake(1000, I8)),
        lambda: gq.gq_reduce_requantize(cd, sc, units, Fake(10, F32), Fake(1000, I8)),
        lambda: gq.gq_reduce_requantize(cd, sc, units, Fake(10, F32), Fake(1000, I8),
                                        r_out=Fake(1000, F32)),
        lambda: gq.gq_sum_f32(xs, Fake(1000, F32)),
        lambda: gq.gq_error_report(Fake(1000, I8), Fake(10, F32), Fake(1000, F32), units,
                                   Fake(100, F64)),
        lambda: gq.gq_pipe_step(pipe, xs, [Fake(600, I8) for _ in range(6)],
                                [Fake(6, F32) for _ in range(6)], Fake(10, F32),
                                Fake(1000, I8)),
    ]
    for c in calls:
        with pytest.raises(Reached):
            c()
    assert len(stub.calls) == len(calls)


BAD = {
    # quantize inputs
    "x short": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32), Fake(999, F32)], u, [Fake(10, F32)] * 2, [Fake(1000, I8)] * 2),
    "x mixed dtypes": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32), Fake(1000, F16)], u, [Fake(10, F32)] * 2, [Fake(1000, I8)] * 2),
    "x integer": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, I32)], u, [Fake(10, F32)], [Fake(1000, I8)]),
    "x not contiguous": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32, contiguous=False)], u, [Fake(10, F32)], [Fake(1000, I8)]),
    "x on the host": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32, cuda=False)], u, [Fake(10, F32)], [Fake(1000, I8)]),
    "x on another device": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32, device=1)], u, [Fake(10, F32)], [Fake(1000, I8)]),
    "no ranks": lambda gq, u, p: gq.gq_quantize([], u, [], []),
    "65 ranks": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)] * 65, u, [Fake(10, F32)] * 65, [Fake(1000, I8)] * 65),
    "scales list short": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)] * 3, u, [Fake(10, F32)] * 2, [Fake(1000, I8)] * 3),
    "codes list long": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)] * 3, u, [Fake(10, F32)] * 3, [Fake(1000, I8)] * 4),
    "scale short": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)], u, [Fake(9, F32)], [Fake(1000, I8)]),
    "scale float64": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)], u, [Fake(10, F64)], [Fake(1000, I8)]),
    "codes uint8": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)], u, [Fake(10, F32)], [Fake(1000, torch.uint8)]),
    "codes short": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)], u, [Fake(10, F32)], [Fake(999, I8)]),
    "amax short": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)] * 2, u, [Fake(10, F32)] * 2, [Fake(1000, I8)] * 2,
        amax_bits=Fake(19, I32)),
    "amax float": lambda gq, u, p: gq.gq_absmax([Fake(1000, F32)], u, Fake(10, F32)),
    "dead table": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)], gq.Units.__new__(gq.Units), [Fake(10, F32)], [Fake(1000, I8)]),
    "not a table": lambda gq, u, p: gq.gq_quantize(
        [Fake(1000, F32)], object(), [Fake(10, F32)], [Fake(1000, I8)]),
    # reduce inputs and outputs
    "reduce scales list short": lambda gq, u, p: gq.gq_reduce_dequant(
        [Fake(1000, I8)] * 4, [Fake(10, F32)] * 3, u, Fake(1000, F32)),
    "reduce codes short": lambda gq, u, p: gq.gq_reduce_requantize(
        [Fake(1000, I8), Fake(10, I8)], [Fake(10, F32)] * 2, u, Fake(10, F32),
        Fake(1000, I8)),
    "r_out short": lambda gq, u, p: gq.gq_reduce_dequant(
        [Fake(1000, I8)], [Fake(10, F32)], u, Fake(999, F32)),
    "r_out float16": lambda gq, u, p: gq.gq_reduce_requantize(
        [Fake(1000, I8)], [Fake(10, F32)], u, Fake(10, F32), Fake(1000, I8),
        r_out=Fake(1000, F16)),
    "scale_out short": lambda gq, u, p: gq.gq_reduce_requantize(
        [Fake(1000, I8)], [Fake(10, F32)], u, Fake(9, F32), Fake(1000, I8)),
    "q_out float": lambda gq, u, p: gq.gq_reduce_requantize(
        [Fake(1000, I8)], [Fake(10, F32)], u, Fake(10, F32), Fake(1000, F32)),
    "requantize r int8": lambda gq, u, p: gq.gq_requantize(
        Fake(1000, I8), u, Fake(10, F32), Fake(1000, I8)),
    # precision check and pipeline
    "sum second rank short": lambda gq, u, p: gq.gq_sum_f32(
        [Fake(1000, F32), Fake(500, F32)], Fake(1000, F32)),
    "sum r_out short": lambda gq, u, p: gq.gq_sum_f32([Fake(1000, F32)], Fake(999, F32)),
    "report stats float32": lambda gq, u, p: gq.gq_error_report(
        Fake(1000, I8), Fake(10, F32), Fake(1000, F32), u, Fake(100, F32)),
    "report ref short": lambda gq, u, p: gq.gq_error_report(
        Fake(1000, I8), Fake(10, F32), Fake(999, F32), u, Fake(100, F64)),
    "pipe slots W instead of 2W": lambda gq, u, p: gq.gq_pipe_step(
        p, [Fake(1000, F32)] * 3, [Fake(600, I8)] * 3, [Fake(6, F32)] * 6, Fake(10, F32),
        Fake(1000, I8)),
    "pipe slot short": lambda gq, u, p: gq.gq_pipe_step(
        p, [Fake(1000, F32)], [Fake(600, I8), Fake(599, I8)], [Fake(6, F32)] * 2,
        Fake(10, F32), Fake(1000, I8)),
    "pipe scale slot float16": lambda gq, u, p: gq.gq_pipe_step(
        p, [Fake(1000, F32)], [Fake(600, I8)] * 2, [Fake(6, F16)] * 2, Fake(10, F32),
        Fake(1000, I8)),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_bad_argument_raises_before_the_library(env, case):
    gq, stub, units, pipe = env
    with pytest.raises((TypeError, ValueError)):
        BAD[case](gq, units, pipe)
    assert stub.calls == [], "the library was called: %s" % stub.calls


def test_live_handles_are_released_at_exit_once():
    """A handle still alive at interpreter exit is destroyed by the
    binding's exit hook (before torch's and the HIP runtime's teardown),
    exactly once, and nothing is reported from the destructors."""
    import subprocess
    import sys
    from tests.conftest import ROOT
    code = (
        "from gradient_compression_allreduce_amd import gq\n"
        "real = gq.lib.gq_chunker_destroy\n"
        "def wrapped(h):\n"
        "    print('destroyed', flush=True)\n"
        "    return real(h)\n"
        "gq.lib.gq_chunker_destroy = wrapped\n"
        "keep = [gq.gq_chunker_create(), gq.gq_chunker_create()]\n"
        "print('alive', flush=True)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["alive", "destroyed", "destroyed"]
    # and the owners' destructors, run after the module's globals are gone,
    # stay silent
    assert "Exception ignored" not in out.stderr, out.stderr
