"""The five synthetic gradient workloads.

Each workload is W simulated data-parallel ranks holding the same list of
gradient tensors (the same model on every rank), packed back to back in one
flat buffer per rank, declaration order, no padding.  Tensor-level properties
(size, standard deviation, value class) are drawn once and shared by all
ranks; element values are drawn per rank.

They stand in for real training gradients (ResNet-152 and BERT-Large on the
pages), which would need datasets, weights and training runs.

Element streams are keyed by (seed, workload, rank, tensor, purpose), so any
element range of any rank can be regenerated on its own.
"""
import math

import numpy as np

from .native import lib

SHARED = 0xFFFF  # "rank" index of the tensor-level (rank-shared) streams

# stream purposes
P_VALUES, P_ZEROS, P_SIGMA, P_HUGE, P_DENORM, P_CLASS, P_SIZE = range(7)

# value classes (workload 5)
C_NORMAL, C_ZERO, C_DENORMAL, C_HUGE = range(4)

HUGE_VALUE = np.float32(3.0e38)


def resnet152_shapes():
    """Parameter tensors of ResNet-152 (torchvision layout), in declaration
    order: 467 tensors, 60,192,808 elements."""
    shapes = [("conv1.weight", (64, 3, 7, 7)), ("bn1.weight", (64,)),
              ("bn1.bias", (64,))]
    inplanes = 64
    for li, (planes, blocks) in enumerate([(64, 3), (128, 8), (256, 36), (512, 3)]):
        for b in range(blocks):
            p = "layer%d.%d." % (li + 1, b)
            cin = inplanes if b == 0 else planes * 4
            shapes += [
                (p + "conv1.weight", (planes, cin, 1, 1)),
                (p + "bn1.weight", (planes,)), (p + "bn1.bias", (planes,)),
                (p + "conv2.weight", (planes, planes, 3, 3)),
                (p + "bn2.weight", (planes,)), (p + "bn2.bias", (planes,)),
                (p + "conv3.weight", (planes * 4, planes, 1, 1)),
                (p + "bn3.weight", (planes * 4,)), (p + "bn3.bias", (planes * 4,)),
            ]
            if b == 0:
                shapes += [
                    (p + "downsample.0.weight", (planes * 4, inplanes, 1, 1)),
                    (p + "downsample.1.weight", (planes * 4,)),
                    (p + "downsample.1.bias", (planes * 4,)),
                ]
        inplanes = planes * 4
    shapes += [("fc.weight", (1000, 2048)), ("fc.bias", (1000,))]
    return shapes


def bert_large_shapes(vocab=30522, hidden=1024, layers=24, ffn=4096,
                      positions=512, types=2):
    """Parameter tensors of BERT-Large with a pooler, in declaration order:
    391 tensors, 335,141,888 elements."""
    h = hidden
    shapes = [("embeddings.word", (vocab, h)), ("embeddings.position", (positions, h)),
              ("embeddings.token_type", (types, h)), ("embeddings.ln.weight", (h,)),
              ("embeddings.ln.bias", (h,))]
    for i in range(layers):
        p = "layer%d." % i
        for m in ("query", "key", "value"):
            shapes += [(p + m + ".weight", (h, h)), (p + m + ".bias", (h,))]
        shapes += [(p + "attn_out.weight", (h, h)), (p + "attn_out.bias", (h,)),
                   (p + "attn_ln.weight", (h,)), (p + "attn_ln.bias", (h,)),
                   (p + "ffn_in.weight", (ffn, h)), (p + "ffn_in.bias", (ffn,)),
                   (p + "ffn_out.weight", (h, ffn)), (p + "ffn_out.bias", (h,)),
                   (p + "out_ln.weight", (h,)), (p + "out_ln.bias", (h,))]
    shapes += [("pooler.weight", (h, h)), ("pooler.bias", (h,))]
    return shapes


def _numel(shape):
    n = 1
    for d in shape:
        n *= d
    return n


class Workload:
    """One synthetic workload.

    Attributes:
      cfg        workload number 1..5
      W          simulated ranks
      kind       'f32' or 'f16' (stored gradient element type)
      elem_bytes 4 or 2
      in_mul     multiplier applied on load (1/S for the loss-scaled fp16 set)
      sizes      int64 array of tensor element counts
      toff       int64 array, tensor offsets in the flat buffer (len T+1)
      n          elements per rank
      units      'tensor' (one scale per tensor) or 'chunk' (one per chunk of
                 each tensor's chunk plan); the plan itself is not computed here
      buckets    list of (first_tensor, end_tensor) bucket ranges or None
    """

    def __init__(self, cfg, name, W, kind, sizes, units, seed=0, in_mul=1.0,
                 loss_scale=1.0, classes=None, sigmas=None, value_law="normal",
                 p_zero=0.0, bucket_bytes=None, description=""):
        self.cfg, self.name, self.W, self.kind = cfg, name, W, kind
        self.elem_bytes = 4 if kind == "f32" else 2
        self.sizes = np.asarray(sizes, dtype=np.int64)
        self.toff = np.zeros(len(self.sizes) + 1, dtype=np.int64)
        np.cumsum(self.sizes, out=self.toff[1:])
        self.n = int(self.toff[-1])
        self.units, self.seed = units, seed
        self.in_mul, self.loss_scale = in_mul, loss_scale
        self.classes = classes if classes is not None else np.zeros(len(sizes), np.int8)
        self.sigmas = sigmas
        self.value_law, self.p_zero = value_law, p_zero
        self.description = description
        self.buckets = None
        if bucket_bytes:
            self.buckets = []
            start, acc = 0, 0
            for t, s in enumerate(self.sizes):
                b = int(s) * self.elem_bytes
                if acc > 0 and acc + b > bucket_bytes:
                    self.buckets.append((start, t))
                    start, acc = t, 0
                acc += b
            self.buckets.append((start, len(self.sizes)))

    @property
    def np_dtype(self):
        return np.float32 if self.kind == "f32" else np.uint16

    def key(self, rank, tensor, purpose):
        return lib().dg_key(self.seed, self.cfg, rank, tensor, purpose)

    def _fill_tensor(self, rank, t, first, count, out):
        """Fill elements [first, first+count) of tensor t of a rank."""
        L = lib()
        ptr = out.ctypes.data
        cls = int(self.classes[t])
        if self.value_law == "normal_f16":
            L.dg_fill_normal_f16(self.key(rank, t, P_VALUES), first, count,
                                 float(self.sigmas[t]), float(self.loss_scale), ptr)
            return
        if self.value_law == "student_t3":
            L.dg_fill_student_t3_f32(self.key(rank, t, P_VALUES), first, count,
                                     float(self.sigmas[t]), ptr)
            return
        if cls == C_ZERO:
            out[:] = 0
            return
        sigma = float(self.sigmas[t])
        if cls == C_DENORMAL:
            L.dg_fill_denormal_f32(self.key(rank, t, P_VALUES),
                                   self.key(rank, t, P_DENORM), first, count,
                                   sigma, ptr)
            return
        L.dg_fill_normal_f32(self.key(rank, t, P_VALUES), self.key(rank, t, P_ZEROS),
                             float(self.p_zero), first, count, sigma, ptr)
        if cls == C_HUGE:
            size = int(self.sizes[t])
            z = L.dg_u64(self.key(rank, t, P_HUGE), 0)
            pos = int(z % size)
            if first <= pos < first + count:
                out[pos - first] = -HUGE_VALUE if (z >> 63) else HUGE_VALUE

    def fill(self, rank, out=None, begin=0, end=None):
        """Elements [begin, end) of rank's flat gradient buffer, as a numpy
        array of float32 (f32) or uint16 binary16 bit patterns (f16)."""
        if end is None:
            end = self.n
        if out is None:
            out = np.empty(end - begin, dtype=self.np_dtype)
        assert out.dtype == self.np_dtype and out.size == end - begin
        t0 = int(np.searchsorted(self.toff, begin, side="right") - 1)
        t = t0
        while t < len(self.sizes) and self.toff[t] < end:
            a = max(begin, int(self.toff[t]))
            b = min(end, int(self.toff[t + 1]))
            if b > a:
                self._fill_tensor(rank, t, a - int(self.toff[t]), b - a,
                                  out[a - begin:b - begin])
            t += 1
        return out

    def checksum(self, arr):
        return int(lib().dg_checksum(arr.ctypes.data, arr.nbytes))

    def input_bytes(self):
        return self.W * self.n * self.elem_bytes

    def summary(self):
        return {"workload": self.name, "W": self.W, "dtype": self.kind,
                "tensors": int(len(self.sizes)), "elements_per_rank": self.n,
                "scale_unit": self.units, "seed": self.seed}


def _log_uniform_sigmas(cfg, seed, count, lo, hi):
    L = lib()
    out = np.empty(count, dtype=np.float64)
    for t in range(count):
        u = L.dg_uniform(L.dg_key(seed, cfg, SHARED, t, P_SIGMA), 0)
        out[t] = 10.0 ** (math.log10(lo) + u * (math.log10(hi) - math.log10(lo)))
    return out


def _make(cfg, seed=0):
    if cfg == 1:
        return Workload(1, "w4_1m_fp32_per_tensor", 4, "f32", [1 << 20], "tensor",
                        seed=seed, sigmas=np.array([1e-3]), p_zero=0.05,
                        description="W=4, one fp32 tensor of 1,048,576 elements, "
                        "N(0,1e-3) with 5% exact zeros, per-tensor scale")
    if cfg == 2:
        shapes = resnet152_shapes()
        sizes = [_numel(s) for _, s in shapes]
        return Workload(2, "resnet152_w8_fp32_per_layer", 8, "f32", sizes, "tensor",
                        seed=seed, sigmas=_log_uniform_sigmas(2, seed, len(sizes), 1e-5, 1e-2),
                        bucket_bytes=25 * 1024 * 1024,
                        description="W=8, ResNet-152 parameter shapes (467 tensors, "
                        "60,192,808 elements), N(0, sigma_t), sigma_t log-uniform in "
                        "[1e-5, 1e-2], one scale per layer tensor, 25 MiB buckets")
    if cfg == 3:
        shapes = bert_large_shapes()
        sizes = [_numel(s) for _, s in shapes]
        return Workload(3, "bert_large_w8_fp16_per_chunk", 8, "f16", sizes, "chunk",
                        seed=seed, in_mul=2.0 ** -16, loss_scale=65536.0,
                        sigmas=_log_uniform_sigmas(3, seed, len(sizes), 1e-5, 1e-2),
                        value_law="normal_f16",
                        description="W=8, BERT-Large parameter shapes (391 tensors, "
                        "335,141,888 elements) stored as fp16 times loss scale 65536, "
                        "unscaled by 2^-16 on load, one scale per 128 KB chunk")
    if cfg == 4:
        return Workload(4, "w16_256m_fp32_student_t_per_chunk", 16, "f32", [1 << 28],
                        "chunk", seed=seed, sigmas=np.array([1e-3]),
                        value_law="student_t3",
                        description="W=16, one fp32 tensor of 268,435,456 elements, "
                        "1e-3 * Student-t(3), one scale per 128 KB chunk")
    if cfg == 5:
        L = lib()
        T = 10000
        sizes = np.array([1 + int(L.dg_u64(L.dg_key(seed, 5, SHARED, t, P_SIZE), 0) % 4096)
                          for t in range(T)], dtype=np.int64)
        order = sorted(range(T), key=lambda t: L.dg_u64(L.dg_key(seed, 5, SHARED, t, P_CLASS), 0))
        classes = np.full(T, C_NORMAL, dtype=np.int8)
        for t in order[:200]:
            classes[t] = C_ZERO
        for t in order[200:300]:
            classes[t] = C_DENORMAL
        for t in order[300:400]:
            classes[t] = C_HUGE
        return Workload(5, "w8_10k_small_fp32_per_tensor", 8, "f32", sizes, "tensor",
                        seed=seed, sigmas=np.full(T, 1e-3), classes=classes,
                        description="W=8, 10,000 fp32 tensors of 1..4096 elements; "
                        "200 all-zero, 100 denormal-rich, 100 holding one +-3e38 per "
                        "rank, the rest N(0,1e-3); one scale per tensor")
    raise ValueError("unknown workload %r" % (cfg,))


_cache = {}


def get_workload(cfg, seed=0):
    k = (cfg, seed)
    if k not in _cache:
        _cache[k] = _make(cfg, seed)
    return _cache[k]


WORKLOADS = (1, 2, 3, 4, 5)
