"""gq_quantize_noalloc's host checks, without a GPU: every argument error,
the size limit of the library's fixed maxima array included, is returned
before the device is touched."""
import ctypes

import numpy as np


def _arr(vals):
    a = (ctypes.c_void_p * len(vals))(*vals)
    return ctypes.cast(a, ctypes.c_void_p)


def test_noalloc_argument_errors_before_any_device_call():
    from gradient_compression_allreduce_amd import gq
    L = gq.lib
    good = 0x10000
    W = 4
    x, s, q = _arr([good] * W), _arr([good] * W), _arr([good] * W)
    off = np.array([0, 10, 20, 35], dtype=np.int64)
    h = off.ctypes.data
    ok_args = (x, W, gq.GQ_F32, 1.0, h, good, 3, s, q, None)

    def call(**kw):
        names = ("x", "W", "dt", "in_mul", "h_off", "d_off", "n_units", "s", "q", "stream")
        args = dict(zip(names, ok_args))
        args.update(kw)
        return L.gq_quantize_noalloc(*(args[k] for k in names))

    assert call(W=0) == gq.GQ_ERR_INVALID
    assert call(W=65) == gq.GQ_ERR_INVALID
    assert call(dt=3) == gq.GQ_ERR_INVALID
    assert call(in_mul=float("nan")) == gq.GQ_ERR_INVALID
    assert call(x=_arr([good, good, good + 8, good])) == gq.GQ_ERR_ALIGN
    assert call(s=_arr([good, 0, good, good])) == gq.GQ_ERR_INVALID
    assert call(q=_arr([good, good, good, good + 4])) == gq.GQ_ERR_ALIGN
    assert call(d_off=None) == gq.GQ_ERR_INVALID
    assert call(d_off=good + 4) == gq.GQ_ERR_ALIGN
    assert call(h_off=None) == gq.GQ_ERR_INVALID
    assert call(n_units=0) == gq.GQ_ERR_INVALID
    bad = np.array([0, 10, 10, 35], dtype=np.int64)
    assert call(h_off=bad.ctypes.data) == gq.GQ_ERR_INVALID
    assert "strictly increasing" in gq.gq_last_error()
    neg = np.array([-1, 10, 20, 35], dtype=np.int64)
    assert call(h_off=neg.ctypes.data) == gq.GQ_ERR_INVALID
    huge = np.array([0, 10, 20, (1 << 40) + 1], dtype=np.int64)
    assert call(h_off=huge.ctypes.data) == gq.GQ_ERR_INVALID
    # the limit: W * n_units maxima in the fixed array
    lim = gq.GQ_NOALLOC_MAX_MAXIMA
    big = np.arange(lim // W + 2, dtype=np.int64)
    assert call(h_off=big.ctypes.data, n_units=lim // W + 1) == gq.GQ_ERR_INVALID
    assert "limit" in gq.gq_last_error()
    one = _arr([good])
    assert L.gq_quantize_noalloc(one, 1, gq.GQ_F32, 1.0, big.ctypes.data, good, lim + 1, one,
                                 one, None) == gq.GQ_ERR_INVALID
    assert "limit" in gq.gq_last_error()
