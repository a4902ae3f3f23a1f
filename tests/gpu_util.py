"""Helpers shared by the GPU parity tests: run the HIP path through the
C ABI on host arrays, run the oracle on the same arrays, compare."""
import sys

import numpy as np

F32, F16 = 0, 1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(arr):
    import torch
    if arr.dtype == np.uint16:
        arr = arr.view(np.float16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def same_f32(a, b):
    """Bitwise equality of float32 arrays, NaNs compared by NaN-ness."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    if a.shape != b.shape:
        return False
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def first_mismatch_f32(a, b):
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    bad = (na != nb) | (~na & ~nb & (a.view(np.uint32) != b.view(np.uint32)))
    idx = np.flatnonzero(bad)
    return (int(idx[0]), a[idx[0]], b[idx[0]], int(idx.size)) if idx.size else None


class GpuStep:
    """The HIP path for W ranks sharing one unit table, on device tensors."""

    def __init__(self, gq, offsets, W, kind, n):
        import torch
        self.gq, self.W, self.kind, self.n = gq, W, kind, n
        self.units = gq.gq_units_create(offsets)
        U = len(offsets) - 1
        self.U = U
        dev = torch.device("cuda")
        self.scales = [torch.empty(U, dtype=torch.float32, device=dev) for _ in range(W)]
        self.codes = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(W)]
        self.amax = torch.empty(W * U, dtype=torch.int32, device=dev)
        self.r = torch.empty(n, dtype=torch.float32, device=dev)
        self.scale_out = torch.empty(U, dtype=torch.float32, device=dev)
        self.q_out = torch.empty(n, dtype=torch.int8, device=dev)

    def quantize(self, xs, in_mul, two_step=False):
        if two_step:
            self.gq.gq_absmax(xs, self.units, self.amax, in_mul=in_mul)
            self.gq.gq_quantize(xs, self.units, self.scales, self.codes, in_mul=in_mul,
                                amax_bits=self.amax)
        else:
            self.gq.gq_quantize(xs, self.units, self.scales, self.codes, in_mul=in_mul)

    def reduce(self, fused=True, with_r=True):
        if fused:
            self.gq.gq_reduce_requantize(self.codes, self.scales, self.units, self.scale_out,
                                         self.q_out, r_out=self.r if with_r else None)
        else:
            self.gq.gq_reduce_dequant(self.codes, self.scales, self.units, self.r)
            self.gq.gq_requantize(self.r, self.units, self.scale_out, self.q_out)

    def host(self):
        import torch
        torch.cuda.synchronize()
        assert self.gq.gq_units_faults(self.units) == 0, "a bounded cross-group wait gave up"
        return {
            "scale": [s.cpu().numpy() for s in self.scales],
            "q": [q.cpu().numpy() for q in self.codes],
            "amax": self.amax.cpu().numpy().view(np.uint32).reshape(self.W, self.U),
            "r": self.r.cpu().numpy(),
            "scale_out": self.scale_out.cpu().numpy(),
            "q_out": self.q_out.cpu().numpy(),
        }


def compare_step(got, want, W, check_r=True, check_amax=False, label=""):
    """Element-by-element comparison of a whole step (bit-exact; NaN by
    NaN-ness)."""
    for w in range(W):
        assert same_f32(got["scale"][w], want["scale"][w]), (
            label, "scale", w, first_mismatch_f32(got["scale"][w], want["scale"][w]))
        bad = np.flatnonzero(got["q"][w] != want["q"][w])
        assert bad.size == 0, (label, "codes", w, int(bad[0]), int(got["q"][w][bad[0]]),
                               int(want["q"][w][bad[0]]), bad.size)
        if check_amax:
            # NaN maxima carry the input's NaN payload: compared by NaN-ness
            assert same_f32(np.asarray(got["amax"][w], np.uint32).view(np.float32),
                            np.asarray(want["amax"][w], np.uint32).view(np.float32)), (
                label, "amax", w)
    if check_r:
        assert same_f32(got["r"], want["r"]), (label, "r", first_mismatch_f32(got["r"], want["r"]))
    assert same_f32(got["scale_out"], want["scale_out"]), (
        label, "scale_out", first_mismatch_f32(got["scale_out"], want["scale_out"]))
    bad = np.flatnonzero(got["q_out"] != want["q_out"])
    assert bad.size == 0, (label, "q_out", int(bad[0]), int(got["q_out"][bad[0]]),
                           int(want["q_out"][bad[0]]), bad.size)


def unit_batches(off, min_elems):
    """Consecutive ranges [ua, ub) of whole units, at least min_elems
    elements each (the last may be shorter)."""
    U = off.size - 1
    out, ua = [], 0
    while ua < U:
        ub = int(np.searchsorted(off, off[ua] + min_elems, side="left"))
        ub = min(max(ub, ua + 1), U)
        out.append((ua, ub))
        ua = ub
    return out


def compare_step_streamed(oracle, xs, kind, off, in_mul, step, W, label, batch_elems=1 << 23,
                          threads=16):
    """Every element of a GPU step (every rank's scales and codes, the fp32
    sum, the requantized scales and codes) against the oracle, which runs
    on ranges of whole units in parallel host threads.  Units are
    independent, so the oracle's result on a range of whole units is its
    whole-workload result there.  step.r must hold the sum."""
    from concurrent.futures import ThreadPoolExecutor
    batches = unit_batches(off, batch_elems)
    scales = [s.cpu().numpy() for s in step.scales]
    s_out = step.scale_out.cpu().numpy()

    def run(ua, ub):
        a, b = int(off[ua]), int(off[ub])
        return oracle.allreduce_step([x[a:b] for x in xs], kind, off[ua:ub + 1] - a, in_mul)

    done = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        # a bounded window of batches in flight keeps host memory small
        window = 2 * threads
        futs = {}
        for i in range(min(window, len(batches))):
            futs[i] = ex.submit(run, *batches[i])
        for i, (ua, ub) in enumerate(batches):
            want = futs.pop(i).result()
            if i + window < len(batches):
                futs[i + window] = ex.submit(run, *batches[i + window])
            a, b = int(off[ua]), int(off[ub])
            where = (label, "units", ua, ub)
            for r in range(W):
                assert same_f32(scales[r][ua:ub], want["scale"][r]), where + (
                    "scale", r, first_mismatch_f32(scales[r][ua:ub], want["scale"][r]))
                got_q = step.codes[r][a:b].cpu().numpy()
                bad = np.flatnonzero(got_q != want["q"][r])
                assert bad.size == 0, where + ("codes", r, a + int(bad[0]), bad.size)
            got_r = step.r[a:b].cpu().numpy()
            assert same_f32(got_r, want["r"]), where + ("r", first_mismatch_f32(got_r, want["r"]))
            assert same_f32(s_out[ua:ub], want["scale_out"]), where + (
                "scale_out", first_mismatch_f32(s_out[ua:ub], want["scale_out"]))
            got_q = step.q_out[a:b].cpu().numpy()
            bad = np.flatnonzero(got_q != want["q_out"])
            assert bad.size == 0, where + ("q_out", a + int(bad[0]), bad.size)
            done += b - a
            if (i + 1) % 8 == 0 or i + 1 == len(batches):
                say("  compared units [0, %d) of %d (%d elements per rank)"
                    % (ub, off.size - 1, done))
    return len(batches)
