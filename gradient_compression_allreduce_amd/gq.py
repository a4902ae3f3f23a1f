"""Thin Python binding of libgq.so (argument marshalling only).

Every function has the name and the meaning of the C entry point declared in
include/gq.h; tensors are torch tensors on the current HIP device, and the
work is enqueued on torch's current stream unless a stream is given.  All
arithmetic runs in the library's gfx950 kernels; if the library is missing
the import fails (there is no fallback).
"""
import atexit
import ctypes
import os
import sys
import weakref

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "_lib", "libgq.so")

GQ_OK, GQ_ERR_INVALID, GQ_ERR_ALIGN, GQ_ERR_CAPACITY, GQ_ERR_HIP, GQ_ERR_DEVICE = range(6)
GQ_F32, GQ_F16 = 0, 1
GQ_SCHED_LAYER, GQ_SCHED_CHUNK = 0, 1
GQ_PIPE_OVERLAP, GQ_PIPE_SERIAL = 0, 1
GQ_FORM_PERSISTENT, GQ_FORM_TWO_PASS, GQ_FORM_SHORT_UNITS = 0, 1, 2
GQ_PIPE_SCHED_ALTERNATE, GQ_PIPE_SCHED_EVENTS, GQ_PIPE_SCHED_SERIAL = 0, 1, 2
GQ_MAX_RANKS = 64
GQ_MAX_TILES = 1 << 22
GQ_NOALLOC_MAX_MAXIMA = 1 << 20
CHUNK_BYTES, ALIGN_BYTES = 131072, 64

EXPORTS = ("gq_last_error", "gq_version", "gq_plan_chunks", "gq_units_create",
           "gq_units_destroy", "gq_units_info", "gq_units_schedule", "gq_units_quantize_tile", "gq_units_reduce_tile", "gq_units_faults",
           "gq_units_faults_async", "gq_units_launch_plan", "gq_units_clear_faults", "gq_units_force_timeout",
           "gq_absmax", "gq_quantize", "gq_quantize_noalloc",
           "gq_reduce_dequant", "gq_requantize", "gq_reduce_requantize",
           "gq_sum_f32", "gq_error_report", "gq_pipe_create", "gq_pipe_destroy",
           "gq_pipe_slots", "gq_pipe_schedule", "gq_pipe_faults", "gq_pipe_clear_faults", "gq_pipe_step", "gq_chunker_create",
           "gq_chunker_destroy", "gq_chunker_update", "gq_chunker_predict", "gq_chunker_plan")
GQ_STATS = 10
STATS = ("max_abs_err", "max_abs_ref", "max_rel_err", "sum_abs_err", "sum_abs_ref",
         "mean_rel_err", "sum_dd", "sum_rr", "sum_dr", "cos")


class GQError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


def _load():
    if not os.path.exists(SO):
        raise ImportError("libgq.so is not built (%s); build it with "
                          "python gradient_compression_allreduce_amd/build.py" % SO)
    L = ctypes.CDLL(SO)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    st = ctypes.c_int
    L.gq_last_error.restype = ctypes.c_char_p
    L.gq_last_error.argtypes = []
    L.gq_version.restype = ctypes.c_char_p
    L.gq_version.argtypes = []
    L.gq_plan_chunks.restype = st
    L.gq_plan_chunks.argtypes = [i64, i32, i64, i32, vp, i64, ctypes.POINTER(i64)]
    L.gq_units_create.restype = st
    L.gq_units_create.argtypes = [vp, i64, ctypes.POINTER(vp)]
    L.gq_units_destroy.restype = st
    L.gq_units_destroy.argtypes = [vp]
    L.gq_units_info.restype = st
    L.gq_units_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.gq_units_schedule.restype = st
    L.gq_units_schedule.argtypes = [vp, i32, ctypes.POINTER(i32)]
    L.gq_units_quantize_tile.restype = st
    L.gq_units_quantize_tile.argtypes = [vp, i32, ctypes.POINTER(i64)]
    L.gq_units_reduce_tile.restype = st
    L.gq_units_reduce_tile.argtypes = [vp, ctypes.POINTER(i64)]
    L.gq_units_faults.restype = st
    L.gq_units_faults.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64)]
    L.gq_units_faults_async.restype = st
    L.gq_units_faults_async.argtypes = [vp, vp, vp]
    L.gq_units_launch_plan.restype = st
    L.gq_units_launch_plan.argtypes = [vp, i32, f32, ctypes.POINTER(i64), ctypes.POINTER(i32),
                                       ctypes.POINTER(i64), ctypes.POINTER(i32)]
    L.gq_units_clear_faults.restype = st
    L.gq_units_clear_faults.argtypes = [vp]
    L.gq_units_force_timeout.restype = st
    L.gq_units_force_timeout.argtypes = [vp]
    L.gq_absmax.restype = st
    L.gq_absmax.argtypes = [vp, i32, i32, f32, vp, vp, vp]
    L.gq_quantize.restype = st
    L.gq_quantize.argtypes = [vp, i32, i32, f32, vp, vp, vp, vp, vp]
    L.gq_quantize_noalloc.restype = st
    L.gq_quantize_noalloc.argtypes = [vp, i32, i32, f32, vp, vp, i64, vp, vp, vp]
    L.gq_reduce_dequant.restype = st
    L.gq_reduce_dequant.argtypes = [vp, vp, i32, vp, vp, vp]
    L.gq_requantize.restype = st
    L.gq_requantize.argtypes = [vp, vp, vp, vp, vp]
    L.gq_reduce_requantize.restype = st
    L.gq_reduce_requantize.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp]
    L.gq_pipe_create.restype = st
    L.gq_pipe_create.argtypes = [vp, i64, vp, i64, i32, ctypes.POINTER(vp)]
    L.gq_pipe_destroy.restype = st
    L.gq_pipe_destroy.argtypes = [vp]
    L.gq_pipe_slots.restype = st
    L.gq_pipe_slots.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.gq_pipe_schedule.restype = st
    L.gq_pipe_schedule.argtypes = [vp, i32, ctypes.c_float, ctypes.POINTER(i32)]
    L.gq_pipe_faults.restype = st
    L.gq_pipe_faults.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64)]
    L.gq_pipe_clear_faults.restype = st
    L.gq_pipe_clear_faults.argtypes = [vp]
    L.gq_pipe_step.restype = st
    L.gq_pipe_step.argtypes = [vp, vp, i32, i32, f32, vp, vp, vp, vp, vp]
    L.gq_chunker_create.restype = st
    L.gq_chunker_create.argtypes = [i32, ctypes.c_double, i64, ctypes.POINTER(vp)]
    L.gq_chunker_destroy.restype = st
    L.gq_chunker_destroy.argtypes = [vp]
    L.gq_chunker_update.restype = st
    L.gq_chunker_update.argtypes = [vp, i64, ctypes.c_double]
    L.gq_chunker_predict.restype = st
    L.gq_chunker_predict.argtypes = [vp, ctypes.POINTER(i64)]
    L.gq_chunker_plan.restype = st
    L.gq_chunker_plan.argtypes = [vp, i64, i32, vp, i64, ctypes.POINTER(i64)]
    L.gq_sum_f32.restype = st
    L.gq_sum_f32.argtypes = [vp, i32, i32, f32, i64, i32, vp, vp]
    L.gq_error_report.restype = st
    L.gq_error_report.argtypes = [vp, vp, vp, vp, vp, vp]
    return L


lib = _load()

# Tables, plans and chunkers still alive when the interpreter exits are
# freed here, in an exit hook registered after torch was imported, so it
# runs before torch's own exit hooks and long before the HIP runtime's
# teardown at process exit; after it, and whenever the interpreter is
# already finalizing, the owners' destructors free nothing.
_live = weakref.WeakSet()
_closed = False


def _release_at_exit():
    global _closed
    objs = list(_live)
    if objs and "torch" in sys.modules:
        try:
            torch = sys.modules["torch"]
            if torch.cuda.is_initialized():
                torch.cuda.synchronize()
        except Exception:
            pass
    for o in objs:
        try:
            o.close()
        except Exception:
            pass
    _closed = True


def _register_exit_hook():
    try:
        import torch  # noqa: F401  (its exit hooks must run after ours)
    except ImportError:
        pass
    atexit.register(_release_at_exit)


_register_exit_hook()


def _finalizing():
    return _closed or sys.is_finalizing()


def _check(status):
    if status != GQ_OK:
        raise GQError(status, lib.gq_last_error().decode())


def gq_last_error():
    return lib.gq_last_error().decode()


def gq_version():
    return lib.gq_version().decode()


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _current_device():
    import torch
    return torch.cuda.current_device()


def _why(name, t, numel, dtypes, dev):
    """The error for a tensor that fails its guard (None if it passes)."""
    if not getattr(t, "is_cuda", False):
        return ValueError("%s must be a tensor on the HIP device" % name)
    if t.dtype not in dtypes:
        return TypeError("%s must be of dtype %s, got %s"
                         % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if not t.is_contiguous():
        return ValueError("%s must be contiguous" % name)
    if t.numel() < numel:
        return ValueError("%s holds %d elements, needs at least %d" % (name, t.numel(), numel))
    if t.get_device() != dev:
        return ValueError("%s is on device %d, the current device is %d"
                          % (name, t.get_device(), dev))
    return None


def _need(name, t, numel, dtypes, dev):
    """Host-side guard, checked before anything is enqueued: a contiguous
    tensor on the current HIP device `dev`, of one of `dtypes`, holding at
    least numel elements (the library reads and writes exactly what the
    call's sizes say, so a short or mistyped buffer would be overrun)."""
    e = _why(name, t, numel, dtypes, dev)
    if e is not None:
        raise e


def _need_list(name, ts, W, numel, dtypes, dev):
    """W tensors, each passing _need (one short-circuit test per tensor; the
    reason is worked out only for a tensor that fails it)."""
    if not isinstance(ts, (list, tuple)):
        raise TypeError("%s must be a list of tensors" % name)
    if len(ts) != W:
        raise ValueError("%s holds %d tensors for %d ranks" % (name, len(ts), W))
    for i, t in enumerate(ts):
        if not (getattr(t, "is_cuda", False) and t.dtype in dtypes and t.numel() >= numel
                and t.is_contiguous() and t.get_device() == dev):
            raise _why("%s[%d]" % (name, i), t, numel, dtypes, dev) or ValueError(name)


def _ranks(name, xs):
    """Number of ranks of a list of rank buffers (1 .. GQ_MAX_RANKS)."""
    if not isinstance(xs, (list, tuple)):
        raise TypeError("%s must be a list of tensors, one per rank" % name)
    if not 1 <= len(xs) <= GQ_MAX_RANKS:
        raise ValueError("%s: %d ranks, must be 1 .. %d" % (name, len(xs), GQ_MAX_RANKS))
    return len(xs)


_TORCH = {}


def _dt():
    """(float32, float16, int8, int32, uint32, int64, float64) torch dtypes."""
    if not _TORCH:
        import torch
        _TORCH["f32"] = (torch.float32,)
        _TORCH["f16"] = (torch.float16,)
        _TORCH["grad"] = (torch.float32, torch.float16)
        _TORCH["i8"] = (torch.int8,)
        _TORCH["bits"] = (torch.int32, torch.uint32)
        _TORCH["i64"] = (torch.int64,)
        _TORCH["f64"] = (torch.float64,)
    return _TORCH


def _grads(xs, numel, dev):
    """Gradient inputs: 1 .. GQ_MAX_RANKS tensors of one element type
    (float32 or float16), each of at least numel elements; returns (W,
    dtype code)."""
    T = _dt()
    W = _ranks("xs", xs)
    dt = getattr(xs[0], "dtype", None)
    if dt not in T["grad"]:
        raise TypeError("gradient elements must be float32 or float16, got %s" % dt)
    _need_list("xs", xs, W, numel, (dt,), dev)
    return W, (GQ_F32 if dt == T["f32"][0] else GQ_F16)


def _table(units):
    if not isinstance(units, Units) or not getattr(units, "handle", None):
        raise ValueError("units must be a live unit table (gq_units_create)")
    return units


_PTR_ARRAYS = {}


def _ptrs(tensors):
    """A host array of the tensors' device addresses: (its address, the
    array, which must stay alive until the call returns)."""
    n = len(tensors)
    t = _PTR_ARRAYS.get(n)
    if t is None:
        t = _PTR_ARRAYS[n] = ctypes.c_uint64 * n
    arr = t(*[x.data_ptr() for x in tensors])
    return ctypes.addressof(arr), arr


def gq_plan_chunks(numel, elem_bytes, chunk_bytes=CHUNK_BYTES, align_bytes=ALIGN_BYTES):
    """Chunk offsets (int64 numpy array of count+1 entries) of §2.1's
    dynamic_chunk for a tensor of numel elements of elem_bytes each."""
    cnt = ctypes.c_int64(0)
    st = lib.gq_plan_chunks(numel, elem_bytes, chunk_bytes, align_bytes, None, 0,
                            ctypes.byref(cnt))
    if st != GQ_ERR_CAPACITY:
        _check(st)
    off = np.empty(cnt.value + 1, dtype=np.int64)
    _check(lib.gq_plan_chunks(numel, elem_bytes, chunk_bytes, align_bytes,
                              off.ctypes.data, off.size, ctypes.byref(cnt)))
    return off


class Units:
    """Owner of a gq_units handle (destroyed with the object)."""

    def __init__(self, offsets):
        off = np.ascontiguousarray(offsets, dtype=np.int64)
        h = ctypes.c_void_p()
        _check(lib.gq_units_create(off.ctypes.data, off.size - 1, ctypes.byref(h)))
        self.handle = h
        self.offsets = off
        self.n = int(off[-1])
        self.n_units = off.size - 1
        _live.add(self)

    @property
    def _as_parameter_(self):
        return self.handle

    def close(self):
        if getattr(self, "handle", None):
            _check(lib.gq_units_destroy(self.handle))
            self.handle = ctypes.c_void_p()

    def __del__(self):
        # (at interpreter shutdown this module's globals may already be
        # None; the exit hook has freed the handle by then)
        try:
            if not _finalizing():
                self.close()
        except Exception:
            pass


def gq_units_create(offsets):
    return Units(offsets)


def gq_units_destroy(units):
    units.close()


def gq_units_info(units):
    n, u = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib.gq_units_info(units.handle, ctypes.byref(n), ctypes.byref(u)))
    return n.value, u.value


def gq_units_schedule(units, dtype_code=GQ_F32):
    """GQ_SCHED_LAYER or GQ_SCHED_CHUNK: the fused quantize schedule chosen
    for this table and element type."""
    v = ctypes.c_int32(-1)
    _check(lib.gq_units_schedule(units.handle, dtype_code, ctypes.byref(v)))
    return v.value


def gq_units_quantize_tile(units, dtype_code=GQ_F32):
    """Elements of the given type per work-group tile of the table's fused
    quantize, chosen when the table was created."""
    v = ctypes.c_int64(0)
    _check(lib.gq_units_quantize_tile(units.handle, dtype_code, ctypes.byref(v)))
    return v.value


def gq_units_reduce_tile(units):
    """Elements per work-group tile of the table's reduce (8192, 16384 or
    32768), chosen when the table was created."""
    v = ctypes.c_int64(0)
    _check(lib.gq_units_reduce_tile(units.handle, ctypes.byref(v)))
    return v.value


def gq_units_faults(units):
    """Bounded waits that gave up on this table since it was created or its
    count was cleared (synchronizes; 0 expected)."""
    c = ctypes.c_uint64(0)
    _check(lib.gq_units_faults(units.handle, ctypes.byref(c)))
    return c.value


def gq_units_faults_async(units, count_out, stream=None):
    """Enqueue a copy of the table's fault count into count_out (a device
    int32/uint32 tensor of at least one element) on the stream, without
    synchronizing; nonzero after the stream's sync means the outputs since
    the count was last cleared are invalid."""
    _table(units)
    _need("count_out", count_out, 1, _dt()["bits"], _current_device())
    _check(lib.gq_units_faults_async(units.handle, count_out.data_ptr(), _stream(stream)))


def gq_units_launch_plan(units, dtype_code=GQ_F32, in_mul=1.0):
    """{"q_groups", "q_form", "r_groups", "r_form"}: the resident work
    groups of the table's persistent quantize and reduce kernels on the
    current device, and the form each fused stage takes (GQ_FORM_*)."""
    _table(units)
    qg, rg = ctypes.c_int64(0), ctypes.c_int64(0)
    qf, rf = ctypes.c_int32(-1), ctypes.c_int32(-1)
    _check(lib.gq_units_launch_plan(units.handle, dtype_code, in_mul, ctypes.byref(qg),
                                    ctypes.byref(qf), ctypes.byref(rg), ctypes.byref(rf)))
    return {"q_groups": qg.value, "q_form": qf.value, "r_groups": rg.value, "r_form": rf.value}


def gq_units_clear_faults(units):
    """Set the table's fault count to zero, so that its waits wait normally
    again (synchronizes)."""
    _check(lib.gq_units_clear_faults(units.handle))


def gq_units_force_timeout(units):
    """Testing aid: make the fault count nonzero, so that the table's
    persistent launches take every wait not satisfied at its first look as
    timed out (counted; outputs may be invalid) until the count is cleared.
    Synchronizes."""
    _check(lib.gq_units_force_timeout(units.handle))


def gq_absmax(xs, units, amax_bits, in_mul=1.0, stream=None):
    """amax_bits: int32/uint32 tensor of W*n_units (rank-major), overwritten
    with the bit patterns of max|x*in_mul| per unit."""
    _table(units)
    dev = _current_device()
    W, dt = _grads(xs, units.n, dev)
    _need("amax_bits", amax_bits, W * units.n_units, _dt()["bits"], dev)
    px, keep = _ptrs(xs)
    _check(lib.gq_absmax(px, W, dt, in_mul, units.handle, amax_bits.data_ptr(),
                         _stream(stream)))


def gq_quantize(xs, units, scales, codes, in_mul=1.0, amax_bits=None, stream=None):
    """Per-unit scales (float32, n_units each) and int8 codes (n each) of W
    gradients xs."""
    _table(units)
    dev = _current_device()
    T = _dt()
    W, dt = _grads(xs, units.n, dev)
    _need_list("scales", scales, W, units.n_units, T["f32"], dev)
    _need_list("codes", codes, W, units.n, T["i8"], dev)
    if amax_bits is not None:
        _need("amax_bits", amax_bits, W * units.n_units, T["bits"], dev)
    px, k1 = _ptrs(xs)
    ps, k2 = _ptrs(scales)
    pq, k3 = _ptrs(codes)
    am = amax_bits.data_ptr() if amax_bits is not None else None
    _check(lib.gq_quantize(px, W, dt, in_mul, units.handle, am, ps, pq, _stream(stream)))


def gq_quantize_noalloc(xs, h_off, d_off, scales, codes, in_mul=1.0, stream=None):
    """gq_quantize with computed maxima and no unit table, for callers that
    cannot allocate device memory: h_off is the host array (int64, numpy) of
    n_units+1 unit offsets and d_off a device int64 tensor holding the same
    values.  The library keeps the maxima in a fixed array of its own
    (W * n_units <= GQ_NOALLOC_MAX_MAXIMA), shared by every call on the
    device: calls on one device must be ordered."""
    off = np.ascontiguousarray(h_off, dtype=np.int64)
    if off.ndim != 1 or off.size < 2:
        raise ValueError("h_off must hold n_units + 1 >= 2 offsets")
    U = off.size - 1
    dev = _current_device()
    T = _dt()
    W, dt = _grads(xs, int(off[-1]), dev)
    _need("d_off", d_off, U + 1, T["i64"], dev)
    _need_list("scales", scales, W, U, T["f32"], dev)
    _need_list("codes", codes, W, int(off[-1]), T["i8"], dev)
    px, k1 = _ptrs(xs)
    ps, k2 = _ptrs(scales)
    pq, k3 = _ptrs(codes)
    _check(lib.gq_quantize_noalloc(px, W, dt, in_mul, off.ctypes.data, d_off.data_ptr(), U,
                                   ps, pq, _stream(stream)))


def _reduce_inputs(codes, scales, units, dev):
    _table(units)
    T = _dt()
    W = _ranks("codes", codes)
    _need_list("codes", codes, W, units.n, T["i8"], dev)
    _need_list("scales", scales, W, units.n_units, T["f32"], dev)
    return W


def gq_reduce_dequant(codes, scales, units, r_out, stream=None):
    dev = _current_device()
    W = _reduce_inputs(codes, scales, units, dev)
    _need("r_out", r_out, units.n, _dt()["f32"], dev)
    pq, k1 = _ptrs(codes)
    ps, k2 = _ptrs(scales)
    _check(lib.gq_reduce_dequant(pq, ps, W, units.handle, r_out.data_ptr(), _stream(stream)))


def gq_requantize(r, units, scale_out, q_out, stream=None):
    _table(units)
    dev = _current_device()
    T = _dt()
    _need("r", r, units.n, T["f32"], dev)
    _need("scale_out", scale_out, units.n_units, T["f32"], dev)
    _need("q_out", q_out, units.n, T["i8"], dev)
    _check(lib.gq_requantize(r.data_ptr(), units.handle, scale_out.data_ptr(),
                             q_out.data_ptr(), _stream(stream)))


def gq_reduce_requantize(codes, scales, units, scale_out, q_out, r_out=None, stream=None):
    dev = _current_device()
    T = _dt()
    W = _reduce_inputs(codes, scales, units, dev)
    _need("scale_out", scale_out, units.n_units, T["f32"], dev)
    _need("q_out", q_out, units.n, T["i8"], dev)
    if r_out is not None:
        _need("r_out", r_out, units.n, T["f32"], dev)
    pq, k1 = _ptrs(codes)
    ps, k2 = _ptrs(scales)
    rp = r_out.data_ptr() if r_out is not None else None
    _check(lib.gq_reduce_requantize(pq, ps, W, units.handle, rp, scale_out.data_ptr(),
                                    q_out.data_ptr(), _stream(stream)))


def gq_sum_f32(xs, r_out, in_mul=1.0, mean=False, stream=None):
    """fp32 rank-order sum of the unquantized gradients xs (divided by W if
    mean) into r_out (float32, n)."""
    _ranks("xs", xs)
    dev = _current_device()
    n = xs[0].numel()
    W, dt = _grads(xs, n, dev)
    _need("r_out", r_out, n, _dt()["f32"], dev)
    px, keep = _ptrs(xs)
    _check(lib.gq_sum_f32(px, W, dt, in_mul, n, 1 if mean else 0, r_out.data_ptr(),
                          _stream(stream)))


def gq_error_report(q, scale, ref, units, stats_out, stream=None):
    """Per-unit binary64 error statistics of the INT8 result (q, scale)
    against ref; stats_out: float64 tensor of n_units * GQ_STATS, columns
    named by STATS."""
    _table(units)
    dev = _current_device()
    T = _dt()
    _need("q", q, units.n, T["i8"], dev)
    _need("scale", scale, units.n_units, T["f32"], dev)
    _need("ref", ref, units.n, T["f32"], dev)
    _need("stats_out", stats_out, units.n_units * GQ_STATS, T["f64"], dev)
    _check(lib.gq_error_report(q.data_ptr(), scale.data_ptr(), ref.data_ptr(), units.handle,
                               stats_out.data_ptr(), _stream(stream)))


class Pipe:
    """Owner of a gq_pipe plan (destroyed with the object)."""

    def __init__(self, offsets, bucket_units, mode=GQ_PIPE_OVERLAP):
        off = np.ascontiguousarray(offsets, dtype=np.int64)
        bu = np.ascontiguousarray(bucket_units, dtype=np.int64)
        h = ctypes.c_void_p()
        _check(lib.gq_pipe_create(off.ctypes.data, off.size - 1, bu.ctypes.data, bu.size - 1,
                                  mode, ctypes.byref(h)))
        self.handle = h
        self.n = int(off[-1])
        self.n_units = off.size - 1
        self.n_buckets = bu.size - 1
        _live.add(self)

    def close(self):
        if getattr(self, "handle", None):
            _check(lib.gq_pipe_destroy(self.handle))
            self.handle = ctypes.c_void_p()

    def __del__(self):
        # (at interpreter shutdown this module's globals may already be
        # None; the exit hook has freed the handle by then)
        try:
            if not _finalizing():
                self.close()
        except Exception:
            pass


def gq_pipe_create(offsets, bucket_units, mode=GQ_PIPE_OVERLAP):
    return Pipe(offsets, bucket_units, mode)


def gq_pipe_destroy(pipe):
    pipe.close()


def gq_pipe_slots(pipe):
    """(slot_elems, slot_units) of one code/scale slot per rank."""
    e, u = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib.gq_pipe_slots(pipe.handle, ctypes.byref(e), ctypes.byref(u)))
    return e.value, u.value


def gq_pipe_schedule(pipe, dtype_code=GQ_F32, in_mul=1.0):
    """The schedule gq_pipe_step runs for this plan on the current device:
    GQ_PIPE_SCHED_ALTERNATE, GQ_PIPE_SCHED_EVENTS or GQ_PIPE_SCHED_SERIAL."""
    v = ctypes.c_int32(-1)
    _check(lib.gq_pipe_schedule(pipe.handle, int(dtype_code), float(in_mul), ctypes.byref(v)))
    return v.value


def gq_pipe_faults(pipe):
    c = ctypes.c_uint64(0)
    _check(lib.gq_pipe_faults(pipe.handle, ctypes.byref(c)))
    return c.value


def gq_pipe_clear_faults(pipe):
    """gq_units_clear_faults on each of the plan's tables (synchronizes)."""
    _check(lib.gq_pipe_clear_faults(pipe.handle))


def gq_pipe_step(pipe, xs, q_slots, scale_slots, scale_out, q_out, in_mul=1.0, stream=None):
    """Pipelined step over the plan's buckets.  q_slots / scale_slots: lists
    of 2*W tensors (slot s of rank w at index s*W + w)."""
    if not isinstance(pipe, Pipe) or not getattr(pipe, "handle", None):
        raise ValueError("pipe must be a live plan (gq_pipe_create)")
    dev = _current_device()
    T = _dt()
    W, dt = _grads(xs, pipe.n, dev)
    se, su = gq_pipe_slots(pipe)
    _need_list("q_slots", q_slots, 2 * W, se, T["i8"], dev)
    _need_list("scale_slots", scale_slots, 2 * W, su, T["f32"], dev)
    _need("scale_out", scale_out, pipe.n_units, T["f32"], dev)
    _need("q_out", q_out, pipe.n, T["i8"], dev)
    px, k1 = _ptrs(xs)
    pq, k2 = _ptrs(q_slots)
    ps, k3 = _ptrs(scale_slots)
    _check(lib.gq_pipe_step(pipe.handle, px, W, dt, in_mul, pq, ps, scale_out.data_ptr(),
                            q_out.data_ptr(), _stream(stream)))


class Chunker:
    """Owner of a gq_chunker (adaptive chunk size)."""

    def __init__(self, capacity=100, alpha=0.25, default_bytes=CHUNK_BYTES):
        h = ctypes.c_void_p()
        _check(lib.gq_chunker_create(capacity, alpha, default_bytes, ctypes.byref(h)))
        self.handle = h
        _live.add(self)

    def close(self):
        if getattr(self, "handle", None):
            _check(lib.gq_chunker_destroy(self.handle))
            self.handle = ctypes.c_void_p()

    def __del__(self):
        # (at interpreter shutdown this module's globals may already be
        # None; the exit hook has freed the handle by then)
        try:
            if not _finalizing():
                self.close()
        except Exception:
            pass


def gq_chunker_create(capacity=100, alpha=0.25, default_bytes=CHUNK_BYTES):
    return Chunker(capacity, alpha, default_bytes)


def gq_chunker_destroy(chunker):
    chunker.close()


def gq_chunker_update(chunker, chunk_bytes, latency):
    _check(lib.gq_chunker_update(chunker.handle, int(chunk_bytes), float(latency)))


def gq_chunker_predict(chunker):
    v = ctypes.c_int64(0)
    _check(lib.gq_chunker_predict(chunker.handle, ctypes.byref(v)))
    return v.value


def gq_chunker_plan(chunker, numel, elem_bytes):
    """Chunk offsets of dynamic_chunk with the predicted chunk size."""
    cnt = ctypes.c_int64(0)
    st = lib.gq_chunker_plan(chunker.handle, numel, elem_bytes, None, 0, ctypes.byref(cnt))
    if st != GQ_ERR_CAPACITY:
        _check(st)
    off = np.empty(cnt.value + 1, dtype=np.int64)
    _check(lib.gq_chunker_plan(chunker.handle, numel, elem_bytes, off.ctypes.data, off.size,
                               ctypes.byref(cnt)))
    return off
