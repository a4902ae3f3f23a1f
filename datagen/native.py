"""ctypes loader for libdatagen.so (built with gcc + OpenMP)."""
import ctypes
import os
import subprocess
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "datagen.c")
SO = os.path.join(HERE, "libdatagen.so")

_lock = threading.Lock()
_lib = None


def build(force=True):
    """Compile libdatagen.so in place."""
    tmp = SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, SO)


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(SO):
                build()
            L = ctypes.CDLL(SO)
            u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
            vp = ctypes.c_void_p
            L.dg_key.restype = u64
            L.dg_key.argtypes = [u64, u64, u64, u64, u64]
            L.dg_u64.restype = u64
            L.dg_u64.argtypes = [u64, u64]
            L.dg_uniform.restype = dbl
            L.dg_uniform.argtypes = [u64, u64]
            L.dg_normal.restype = dbl
            L.dg_normal.argtypes = [u64, u64]
            L.dg_fill_normal_f32.restype = None
            L.dg_fill_normal_f32.argtypes = [u64, u64, dbl, u64, i64, dbl, vp]
            L.dg_fill_student_t3_f32.restype = None
            L.dg_fill_student_t3_f32.argtypes = [u64, u64, i64, dbl, vp]
            L.dg_fill_normal_f16.restype = None
            L.dg_fill_normal_f16.argtypes = [u64, u64, i64, dbl, dbl, vp]
            L.dg_fill_denormal_f32.restype = None
            L.dg_fill_denormal_f32.argtypes = [u64, u64, u64, i64, dbl, vp]
            L.dg_checksum.restype = u64
            L.dg_checksum.argtypes = [vp, i64]
            _lib = L
    return _lib
