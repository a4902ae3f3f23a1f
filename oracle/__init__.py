"""CPU oracle for the INT8-compressed gradient AllReduce compute.

TEST INFRASTRUCTURE ONLY: only tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its binding) never calls it.

A thin ctypes wrapper over liboracle.so (oracle.c, plain single-threaded C,
built with -O2 -ffp-contract=off).  Each function follows one step of the
pipelined HCCL AllReduce article (bjdmk.com.cn/news/6235379): §2.1 chunk
plan, §2.2.1 absmax scale / int8 codes / INT8 AllReduce reduction, §6.1
unscale on load, §5.2's check with quantization switched off (the fp32
reference sum and the per-unit error report), and §6.2's adaptive chunk
size.
"""
import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
SO = os.path.join(HERE, "liboracle.so")

F32, F16 = 0, 1
STATS = ("max_abs_err", "max_abs_ref", "max_rel_err", "sum_abs_err", "sum_abs_ref",
         "mean_rel_err", "sum_dd", "sum_rr", "sum_dr", "cos")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]

_lock = threading.Lock()
_lib = None


def build(src=SRC, out=SO, extra=()):
    """Compile the oracle in place (or a variant of it, for the mutation
    tests)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, *extra, "-I", HERE, "-o", tmp, src, "-lm"],
                   check=True)
    os.replace(tmp, out)


def _declare(L):
    i64, i32, u32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    vp, i8 = ctypes.c_void_p, ctypes.c_int8
    L.oracle_plan_chunks.restype = ctypes.c_int
    L.oracle_plan_chunks.argtypes = [i64, i32, i64, i32, vp, i64, ctypes.POINTER(i64)]
    L.oracle_half_to_float.restype = f32
    L.oracle_half_to_float.argtypes = [ctypes.c_uint16]
    L.oracle_load.restype = None
    L.oracle_load.argtypes = [vp, i32, f32, i64, vp]
    L.oracle_absmax_bits.restype = u32
    L.oracle_absmax_bits.argtypes = [vp, i64]
    L.oracle_scale.restype = f32
    L.oracle_scale.argtypes = [u32]
    L.oracle_code.restype = i8
    L.oracle_code.argtypes = [f32, f32]
    L.oracle_quantize_units.restype = None
    L.oracle_quantize_units.argtypes = [vp, i32, f32, i64, vp, i64, vp, vp, vp]
    L.oracle_quantize_with_amax.restype = None
    L.oracle_quantize_with_amax.argtypes = [vp, i32, f32, i64, vp, i64, vp, vp, vp]
    L.oracle_reduce_dequant.restype = None
    L.oracle_reduce_dequant.argtypes = [vp, vp, i32, i64, vp, i64, vp]
    L.oracle_requantize.restype = None
    L.oracle_requantize.argtypes = [vp, i64, vp, i64, vp, vp]
    L.oracle_chunker_predict.restype = i64
    L.oracle_chunker_predict.argtypes = [vp, vp, i64, i32, ctypes.c_double, i64]
    L.oracle_sum_f32.restype = None
    L.oracle_sum_f32.argtypes = [vp, i32, f32, i32, i64, i32, vp]
    L.oracle_error_report.restype = None
    L.oracle_error_report.argtypes = [vp, vp, vp, i64, vp, i64, vp]
    return L


def load(path=SO):
    """Load an oracle shared object (the default one, built if missing)."""
    return _declare(ctypes.CDLL(path))


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(SO):
                build()
            _lib = load(SO)
    return _lib


class Oracle:
    """numpy-level interface over one loaded oracle library."""

    def __init__(self, L=None):
        self.L = L if L is not None else lib()

    def plan_chunks(self, numel, elem_bytes, chunk_bytes=131072, align_bytes=64):
        cnt = ctypes.c_int64(0)
        rc = self.L.oracle_plan_chunks(numel, elem_bytes, chunk_bytes, align_bytes,
                                       None, 0, ctypes.byref(cnt))
        if rc < 0:
            raise ValueError("oracle_plan_chunks: bad arguments")
        off = np.empty(cnt.value + 1, dtype=np.int64)
        rc = self.L.oracle_plan_chunks(numel, elem_bytes, chunk_bytes, align_bytes,
                                       off.ctypes.data, off.size, ctypes.byref(cnt))
        assert rc == 0
        return off

    def half_to_float(self, h):
        return np.float32(self.L.oracle_half_to_float(int(h)))

    def load(self, x, kind, in_mul=1.0):
        x = np.ascontiguousarray(x)
        g = np.empty(x.size, dtype=np.float32)
        self.L.oracle_load(x.ctypes.data, kind, in_mul, x.size, g.ctypes.data)
        return g

    def absmax_bits(self, g):
        g = np.ascontiguousarray(g, dtype=np.float32)
        return int(self.L.oracle_absmax_bits(g.ctypes.data, g.size))

    def scale(self, amax_bits):
        return np.float32(self.L.oracle_scale(int(amax_bits)))

    def code(self, g, s):
        return int(self.L.oracle_code(float(np.float32(g)), float(np.float32(s))))

    def quantize_units(self, x, kind, off, in_mul=1.0):
        """-> (amax_bits[U] uint32, scale[U] float32, q[n] int8)"""
        x = np.ascontiguousarray(x)
        off = np.ascontiguousarray(off, dtype=np.int64)
        U = off.size - 1
        n = int(off[-1])
        assert x.size >= n
        amax = np.empty(U, dtype=np.uint32)
        sc = np.empty(U, dtype=np.float32)
        q = np.empty(n, dtype=np.int8)
        self.L.oracle_quantize_units(x.ctypes.data, kind, in_mul, n, off.ctypes.data,
                                     U, amax.ctypes.data, sc.ctypes.data, q.ctypes.data)
        return amax, sc, q

    def quantize_with_amax(self, x, kind, off, amax, in_mul=1.0):
        x = np.ascontiguousarray(x)
        off = np.ascontiguousarray(off, dtype=np.int64)
        amax = np.ascontiguousarray(amax, dtype=np.uint32)
        U = off.size - 1
        n = int(off[-1])
        sc = np.empty(U, dtype=np.float32)
        q = np.empty(n, dtype=np.int8)
        self.L.oracle_quantize_with_amax(x.ctypes.data, kind, in_mul, n, off.ctypes.data,
                                         U, amax.ctypes.data, sc.ctypes.data, q.ctypes.data)
        return sc, q

    def reduce_dequant(self, qs, ss, off):
        """qs: list of W int8 arrays (n); ss: list of W float32 arrays (U)."""
        off = np.ascontiguousarray(off, dtype=np.int64)
        W = len(qs)
        qs = [np.ascontiguousarray(a, dtype=np.int8) for a in qs]
        ss = [np.ascontiguousarray(a, dtype=np.float32) for a in ss]
        qp = (ctypes.c_void_p * W)(*[a.ctypes.data for a in qs])
        sp = (ctypes.c_void_p * W)(*[a.ctypes.data for a in ss])
        n = int(off[-1])
        r = np.empty(n, dtype=np.float32)
        self.L.oracle_reduce_dequant(ctypes.cast(qp, ctypes.c_void_p),
                                     ctypes.cast(sp, ctypes.c_void_p), W, n,
                                     off.ctypes.data, off.size - 1, r.ctypes.data)
        return r

    def requantize(self, r, off):
        r = np.ascontiguousarray(r, dtype=np.float32)
        off = np.ascontiguousarray(off, dtype=np.int64)
        U = off.size - 1
        n = int(off[-1])
        sc = np.empty(U, dtype=np.float32)
        q = np.empty(n, dtype=np.int8)
        self.L.oracle_requantize(r.ctypes.data, n, off.ctypes.data, U, sc.ctypes.data,
                                 q.ctypes.data)
        return sc, q

    def allreduce_step(self, xs, kind, off, in_mul=1.0):
        """The whole per-device path for W ranks: each rank's codes and
        scales, the rank-order fp32 sum, and its requantized codes."""
        per = [self.quantize_units(x, kind, off, in_mul) for x in xs]
        qs = [p[2] for p in per]
        ss = [p[1] for p in per]
        r = self.reduce_dequant(qs, ss, off)
        s2, q2 = self.requantize(r, off)
        return {"amax": [p[0] for p in per], "scale": ss, "q": qs, "r": r,
                "scale_out": s2, "q_out": q2}

    def sum_f32(self, xs, kind, in_mul=1.0, mean=False):
        """fp32 rank-order sum of the loaded gradients (÷W if mean)."""
        xs = [np.ascontiguousarray(x) for x in xs]
        W = len(xs)
        n = xs[0].size
        assert all(x.size == n for x in xs)
        xp = (ctypes.c_void_p * W)(*[x.ctypes.data for x in xs])
        r = np.empty(n, dtype=np.float32)
        self.L.oracle_sum_f32(ctypes.cast(xp, ctypes.c_void_p), kind, in_mul, W, n,
                              1 if mean else 0, r.ctypes.data)
        return r

    def error_report(self, q, scale, ref, off):
        """-> float64 array [U, 10], columns named by STATS."""
        q = np.ascontiguousarray(q, dtype=np.int8)
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        ref = np.ascontiguousarray(ref, dtype=np.float32)
        off = np.ascontiguousarray(off, dtype=np.int64)
        U = off.size - 1
        n = int(off[-1])
        assert q.size >= n and ref.size >= n and scale.size >= U
        out = np.empty((U, len(STATS)), dtype=np.float64)
        self.L.oracle_error_report(q.ctypes.data, scale.ctypes.data, ref.ctypes.data, n,
                                   off.ctypes.data, U, out.ctypes.data)
        return out

    def chunker_predict(self, sizes, lat, capacity=100, alpha=0.25, default_bytes=131072):
        """Predicted chunk size after the observations (sizes[i], lat[i])."""
        sizes = np.ascontiguousarray(sizes, dtype=np.int64)
        lat = np.ascontiguousarray(lat, dtype=np.float64)
        assert sizes.size == lat.size
        return int(self.L.oracle_chunker_predict(sizes.ctypes.data, lat.ctypes.data, sizes.size,
                                                 capacity, alpha, default_bytes))
