"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch,
so that the same list runs against the real oracle (test_oracle_pins.py) and
against deliberately broken copies of it (test_oracle_mutants.py).

Method source: the pipelined HCCL AllReduce article
(bjdmk.com.cn/news/6235379): §2.1 dynamic_chunk, §2.2.1 quantize_gradient
and the INT8 AllReduce, §6.1 unscale before quantizing, §5.2 the precision
check with quantization switched off (fp32 reference sum, error report),
§6.2 the adaptive chunk size.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.json")

F32, F16 = 0, 1
TINY = np.float32(2.0 ** -149)
NORMAL_MIN_SCALE = np.float32(2.0 ** -126)


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def _bits(f):
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0])


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _pow2(m, e):
    return np.float32(math.ldexp(m, e)) if m != "inf" else np.float32(np.inf)


# --------------------------------------------------------------------------
# §2.1 chunk plan


def _torch_chunk_offsets(n, k):
    sizes = [c.numel() for c in torch.chunk(torch.empty(n, dtype=torch.uint8), k)]
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def pin_plan_matches_torch_chunk(o):
    """Library routine: the plan's pieces are exactly torch.chunk's, for the
    chunk count of §2.1 (byte size // (131072 - 131072 % 64), at least 1)."""
    rng = np.random.default_rng(1)
    ns = list(range(1, 300)) + [int(v) for v in rng.integers(1, 4_000_000, 400)]
    ns += [32767, 32768, 32769, 65535, 65536, 65537, 1 << 20, (1 << 20) + 3,
           2359296, 2048000, 31254528, 4194304]
    for e in (4, 2, 1):
        for n in ns:
            k = max(1, (n * e) // (131072 - 131072 % 64))
            want = _torch_chunk_offsets(n, k)
            got = o.plan_chunks(n, e)
            assert np.array_equal(got, want), (n, e, got[:4], want[:4])


def pin_plan_invariants(o):
    """Closed form: all pieces have ceil(n/k) elements except a shorter last
    one, they tile [0, n), and there are exactly k of them whenever
    k(k-1) < n (always true below 2^30 elements for 4-byte data)."""
    rng = np.random.default_rng(2)
    for n in [int(v) for v in rng.integers(1, 50_000_000, 300)] + [1, 2, 268435456]:
        for e in (4, 2):
            off = o.plan_chunks(n, e)
            k = max(1, n * e // 131072)
            c = -(-n // k)
            lens = np.diff(off)
            assert off[0] == 0 and off[-1] == n
            assert np.all(lens[:-1] == c) and 0 < lens[-1] <= c
            if k * (k - 1) < n:
                assert len(lens) == k, (n, e, len(lens), k)


def pin_plan_alignment_term(o):
    """§2.1: the divisor is the chunk size rounded down to the alignment.
    With chunk 1000 B and alignment 64 B the divisor is 960 B."""
    for n, e, want_k in [(960, 1, 1), (1919, 1, 1), (1920, 1, 2), (2879, 1, 2),
                         (2880, 1, 3), (480, 4, 2), (479, 4, 1), (1000, 1, 1)]:
        off = o.plan_chunks(n, e, chunk_bytes=1000, align_bytes=64)
        assert len(off) - 1 == want_k, (n, e, len(off) - 1, want_k)
    # with the article's constants the alignment term vanishes: 131072 % 64 == 0
    assert len(o.plan_chunks(32768, 4)) - 1 == 1
    assert len(o.plan_chunks(65536, 4)) - 1 == 2
    assert len(o.plan_chunks(65535, 4)) - 1 == 1


# --------------------------------------------------------------------------
# §6.1 load + unscale


def pin_half_to_float_all_patterns(o):
    """Library routine: every binary16 pattern converts as numpy does
    (NaNs compared by NaN-ness)."""
    bits = np.arange(65536, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = o.load(bits, F16, 1.0)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def pin_load_unscale_exact(o):
    """Unscaling by 2^-16 is exact for every finite binary16 value (the
    product stays >= 2^-40, a normal binary32): compare with the float64
    product, which is exact too."""
    bits = np.arange(65536, dtype=np.uint16)
    h = bits.view(np.float16)
    fin = np.isfinite(h)
    got = o.load(bits, F16, 2.0 ** -16)
    want = (h[fin].astype(np.float64) * 2.0 ** -16).astype(np.float32)
    assert np.array_equal(got[fin].view(np.uint32), want.view(np.uint32))
    # fp32 input with a general multiplier: one binary32 rounding (numpy)
    rng = np.random.default_rng(3)
    x = rng.standard_normal(5000).astype(np.float32)
    m = np.float32(0.1)
    assert np.array_equal(o.load(x, F32, float(m)).view(np.uint32),
                          (x * m).astype(np.float32).view(np.uint32))


def pin_golden_load_f16(o):
    for ex in _golden()["load_f16"]:
        bits = np.array(ex["bits"], dtype=np.uint16)
        got = o.load(bits, F16, 2.0 ** -16)
        for i, (m, e) in enumerate(zip(ex["g_mult"], ex["g_exp2"])):
            assert got[i] == np.float32(math.ldexp(m, e)), (ex["name"], i)
            assert bool(np.signbit(got[i])) == (ex["negative_zero"][i] or m < 0)


# --------------------------------------------------------------------------
# §2.2.1 absmax and scale


def pin_absmax_matches_numpy(o):
    """Library routine: max|g| as numpy computes it, NaN propagating."""
    rng = np.random.default_rng(4)
    for trial in range(40):
        g = (rng.standard_normal(rng.integers(1, 3000)) *
             10.0 ** rng.uniform(-44, 30)).astype(np.float32)
        if trial % 5 == 0:
            g[rng.integers(0, g.size)] = -0.0
        want = np.max(np.abs(g))
        got = _f32(o.absmax_bits(g))
        assert got == want, (trial, got, want)
    g = np.array([1.0, np.nan, -np.inf], dtype=np.float32)
    assert np.isnan(_f32(o.absmax_bits(g)))
    g = np.array([1.0, -np.inf, 3.0], dtype=np.float32)
    assert _f32(o.absmax_bits(g)) == np.inf
    g = np.array([-0.0, -0.0], dtype=np.float32)
    assert o.absmax_bits(g) == 0


def _round_rational_to_f32(x):
    """Nearest binary32 to the rational x, ties to even (exact search)."""
    c = np.float32(float(x))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = None
    for f in cands:
        if not np.isfinite(f):
            continue
        d = abs(Fraction(float(f)) - x)
        key = (d, _bits(f) & 1)
        if best is None or key < best[0]:
            best = (key, f)
    return best[1]


def pin_scale_correctly_rounded(o):
    """s is the binary32 nearest to M/127: checked by exact rational search
    on a sample, and against a float64 quotient rounded once more to binary32
    (double rounding is harmless for a quotient of two binary32 values since
    53 >= 2*24 + 2) on many random bit patterns, subnormals included."""
    rng = np.random.default_rng(5)
    pats = rng.integers(0, 0x7f800000, 200000, dtype=np.uint32)
    pats[:64] = np.arange(64, dtype=np.uint32) * 3
    for p in pats[:400]:
        assert o.scale(int(p)) == _round_rational_to_f32(Fraction(float(_f32(p))) / 127)
    ref = (pats.view(np.float32).astype(np.float64) / 127.0).astype(np.float32)
    got = np.array([o.scale(int(p)) for p in pats[:20000]], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref[:20000].view(np.uint32))
    assert o.scale(_bits(np.float32(np.inf))) == np.inf
    assert np.isnan(o.scale(0x7fc00000))


# --------------------------------------------------------------------------
# §2.2.1 int8 codes


def _units(n, rng, max_len=700):
    cuts = [0]
    while cuts[-1] < n:
        cuts.append(min(n, cuts[-1] + int(rng.integers(1, max_len))))
    return np.array(cuts, dtype=np.int64)


def _random_grad(rng, n):
    g = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 3)
    g[rng.random(n) < 0.05] = 0.0
    return g.astype(np.float32)


def pin_codes_match_torch_formula(o):
    """Library routine: the article's quantize_gradient evaluated by torch on
    the CPU, unit by unit, wherever its scale is a normal, finite, non-zero
    number (elsewhere the article's formula is undefined or NaN)."""
    rng = np.random.default_rng(6)
    n = 60000
    g = _random_grad(rng, n)
    off = _units(n, rng)
    amax, sc, q = o.quantize_units(g, F32, off)
    for u in range(off.size - 1):
        a, b = off[u], off[u + 1]
        grad = torch.from_numpy(g[a:b].copy())
        scale = torch.max(torch.abs(grad)) / 127.0
        if not (scale.item() >= float(NORMAL_MIN_SCALE)):
            continue
        want = torch.clamp(torch.round(grad / scale), -128, 127).to(torch.int8)
        assert sc[u] == np.float32(scale.item()), u
        assert np.array_equal(q[a:b], want.numpy()), u


def pin_codes_brute_force(o):
    """Brute force: the code is the argmin over all 256 int8 values of
    |fl(g/s) - c|, ties to the even code, then clamped (the quotient is the
    IEEE binary32 quotient numpy computes)."""
    rng = np.random.default_rng(7)
    cands = np.arange(-128, 128, dtype=np.float64)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        g = _random_grad(rng, n)
        if trial % 7 == 0:
            # force exact half-integer quotients
            k = rng.integers(-127, 127, n)
            g = ((k + 0.5) * 2.0 ** -8).astype(np.float32)
            g[0] = np.float32(127 * 2.0 ** -8)
        off = np.array([0, n], dtype=np.int64)
        _, sc, q = o.quantize_units(g, F32, off)
        s = sc[0]
        if s == 0:
            assert np.all(q == 0)
            continue
        t = (g / s).astype(np.float64)
        d = np.abs(t[:, None] - cands[None, :])
        best = d.min(axis=1, keepdims=True)
        ties = d == best
        want = []
        for i in range(n):
            c = cands[ties[i]]
            if c.size > 1:
                c = c[(c % 2) == 0]
            want.append(int(c[0]))
        assert list(q) == want, (trial, g, s, list(q), want)


def pin_code_error_bound_exact(o):
    """|g - q*s| <= s*(1/2 + 2^-17) in exact rational arithmetic, for units
    with a normal scale (the 2^-17 covers the rounding of g/s for
    |g/s| <= 128)."""
    rng = np.random.default_rng(8)
    n = 4000
    g = _random_grad(rng, n)
    off = _units(n, rng, 300)
    _, sc, q = o.quantize_units(g, F32, off)
    bound = Fraction(1, 2) + Fraction(1, 2 ** 17)
    for u in range(off.size - 1):
        s = sc[u]
        if not s >= NORMAL_MIN_SCALE:
            continue
        S = Fraction(float(s))
        for i in range(off[u], off[u + 1]):
            err = abs(Fraction(float(g[i])) - int(q[i]) * S)
            assert err <= bound * S, (u, i)


def pin_code_invariants(o):
    """Max element -> +-127; no -128 with a normal scale; odd symmetry;
    invariance under scaling by powers of two; zeros -> 0."""
    rng = np.random.default_rng(9)
    n = 50000
    g = _random_grad(rng, n)
    off = _units(n, rng)
    amax, sc, q = o.quantize_units(g, F32, off)
    _, sc_neg, q_neg = o.quantize_units(-g, F32, off)
    assert np.array_equal(q_neg, -q.astype(np.int16))
    assert np.array_equal(sc_neg, sc)
    g2 = (g * np.float32(2.0 ** 5)).astype(np.float32)
    _, sc2, q2 = o.quantize_units(g2, F32, off)
    for u in range(off.size - 1):
        a, b = off[u], off[u + 1]
        if sc[u] >= NORMAL_MIN_SCALE:
            m = np.abs(g[a:b]) == _f32(amax[u])
            assert np.all(np.abs(q[a:b][m]) == 127), u
            assert np.all(q[a:b] != -128), u
            assert sc2[u] == sc[u] * np.float32(32.0)
            assert np.array_equal(q2[a:b], q[a:b])
        assert np.all(q[a:b][g[a:b] == 0] == 0)


def pin_golden_quantize(o):
    for ex in _golden()["quantize"]:
        g = np.array([math.ldexp(m, ex["g_exp2"]) for m in ex["g_mult"]], dtype=np.float32)
        off = np.array([0, g.size], dtype=np.int64)
        _, sc, q = o.quantize_units(g, F32, off)
        assert sc[0] == _pow2(ex["scale_mult"], ex["scale_exp2"]), ex["name"]
        assert list(q) == ex["q"], (ex["name"], list(q))


def pin_subnormal_scales(o):
    """s = 0 exactly when M <= 63*2^-149; 64*2^-149 <= M < 191*2^-149 gives
    s = 2^-149 (values checked against the rational nearest), and codes
    follow the clamp."""
    for k in (1, 2, 62, 63):
        g = np.array([k, -1], dtype=np.float32) * TINY
        _, sc, q = o.quantize_units(g, F32, np.array([0, 2]))
        assert sc[0] == 0 and np.all(q == 0), k
    for k in (64, 100, 190):
        g = np.array([k, -k], dtype=np.float32) * TINY
        _, sc, q = o.quantize_units(g, F32, np.array([0, 2]))
        assert sc[0] == TINY, k
        assert list(q) == [min(k, 127), max(-k, -128)], (k, list(q))
    # torch's CPU formula agrees on the subnormal, non-zero scales
    for k in (64, 190, 8388607):
        g = torch.tensor([k, -k, 3], dtype=torch.float32) * float(TINY)
        s = torch.max(torch.abs(g)) / 127.0
        want = torch.clamp(torch.round(g / s), -128, 127).to(torch.int8)
        _, sc, q = o.quantize_units(g.numpy(), F32, np.array([0, 3]))
        assert sc[0] == np.float32(s.item()) and list(q) == want.tolist(), k


def pin_non_finite_units(o):
    """A unit holding inf gets s = inf and codes 0 (finite/inf = 0, and
    inf/inf = NaN -> 0); a unit holding NaN gets a NaN scale and codes 0;
    finite units beside them are unaffected."""
    g = np.array([1.0, -np.inf, 2.0, 0.5, np.nan, 3.0, 0.25, -0.5], dtype=np.float32)
    off = np.array([0, 3, 6, 8], dtype=np.int64)
    _, sc, q = o.quantize_units(g, F32, off)
    assert sc[0] == np.inf and np.all(q[0:3] == 0)
    assert np.isnan(sc[1]) and np.all(q[3:6] == 0)
    assert sc[2] == np.float32(0.5) / np.float32(127.0)
    assert list(q[6:8]) == [64, -127]


def pin_quantize_with_given_max(o):
    """Codes from a max taken separately (numpy's max|g|) equal the torch
    formula's codes, unit by unit."""
    rng = np.random.default_rng(14)
    n = 30000
    g = _random_grad(rng, n)
    off = _units(n, rng)
    amax = np.array([_bits(np.max(np.abs(g[off[u]:off[u + 1]])))
                     for u in range(off.size - 1)], dtype=np.uint32)
    sc, q = o.quantize_with_amax(g, F32, off, amax)
    for u in range(off.size - 1):
        a, b = off[u], off[u + 1]
        grad = torch.from_numpy(g[a:b].copy())
        scale = torch.max(torch.abs(grad)) / 127.0
        if not (scale.item() >= float(NORMAL_MIN_SCALE)):
            continue
        want = torch.clamp(torch.round(grad / scale), -128, 127).to(torch.int8)
        assert sc[u] == np.float32(scale.item()), u
        assert np.array_equal(q[a:b], want.numpy()), u


# --------------------------------------------------------------------------
# §2.2.1 INT8 AllReduce, one-device reduction


def pin_reduce_single_rank(o):
    """W = 1: r = fl(q * s), the binary32 product numpy computes."""
    rng = np.random.default_rng(10)
    n = 20000
    off = _units(n, rng)
    q = rng.integers(-128, 128, n).astype(np.int8)
    s = (rng.random(off.size - 1) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
    r = o.reduce_dequant([q], [s], off)
    su = np.repeat(s, np.diff(off))
    assert np.array_equal(r.view(np.uint32), (q.astype(np.float32) * su).view(np.uint32))


def pin_reduce_closed_form(o):
    """Closed form (all-reduce of known per-rank values): with
    g_w[i] = (i mod 255 - 127) * 2^e_w and units longer than 255 elements,
    M = 127*2^e_w, s = 2^e_w, codes are i mod 255 - 127, and the rank sum
    sum_w (i mod 255 - 127) * 2^e_w is exact in binary32."""
    n = 255 * 40
    off = np.array([0, 255 * 3, 255 * 17, n], dtype=np.int64)
    i = np.arange(n)
    base = (i % 255 - 127).astype(np.float64)
    es = [-3, -10, -5, -7, -4]
    xs = [(base * 2.0 ** e).astype(np.float32) for e in es]
    per = [o.quantize_units(x, F32, off) for x in xs]
    for (_, sc, q), e in zip(per, es):
        assert np.all(sc == np.float32(2.0 ** e))
        assert np.array_equal(q.astype(np.int64), base.astype(np.int64))
    r = o.reduce_dequant([p[2] for p in per], [p[1] for p in per], off)
    want = base * sum(2.0 ** e for e in es)
    assert np.array_equal(r, want.astype(np.float32))


def pin_reduce_error_bound(o):
    """|r - sum_w q_w s_w| <= gamma_W * sum_w |q_w s_w| in exact rational
    arithmetic, gamma_W = W u / (1 - W u), u = 2^-24."""
    rng = np.random.default_rng(11)
    W, n = 7, 600
    off = _units(n, rng, 200)
    qs = [rng.integers(-128, 128, n).astype(np.int8) for _ in range(W)]
    ss = [(rng.random(off.size - 1) * 2.0 ** -12).astype(np.float32) for _ in range(W)]
    r = o.reduce_dequant(qs, ss, off)
    u = Fraction(1, 2 ** 24)
    gamma = W * u / (1 - W * u)
    unit_of = np.repeat(np.arange(off.size - 1), np.diff(off))
    for i in range(n):
        terms = [int(qs[w][i]) * Fraction(float(ss[w][unit_of[i]])) for w in range(W)]
        exact = sum(terms)
        assert abs(Fraction(float(r[i])) - exact) <= gamma * sum(abs(t) for t in terms), i


def pin_reduce_torch_rank_order(o):
    """Library routine: torch on the CPU, acc = acc + q_w.float() * s_w, one
    separate multiply and add per rank, ranks in order 0..W-1."""
    rng = np.random.default_rng(12)
    W, n = 16, 30000
    off = _units(n, rng)
    qs = [rng.integers(-128, 128, n).astype(np.int8) for _ in range(W)]
    ss = [(rng.random(off.size - 1) * 1e-3).astype(np.float32) for _ in range(W)]
    r = o.reduce_dequant(qs, ss, off)
    lens = torch.from_numpy(np.diff(off))
    acc = torch.zeros(n, dtype=torch.float32)
    for w in range(W):
        su = torch.repeat_interleave(torch.from_numpy(ss[w]), lens)
        acc = acc + torch.from_numpy(qs[w]).float() * su
    assert np.array_equal(r.view(np.uint32), acc.numpy().view(np.uint32))


def pin_golden_reduce(o):
    for ex in _golden()["reduce"]:
        W = len(ex["q"])
        qs = [np.array(row, dtype=np.int8) for row in ex["q"]]
        if "scale" in ex:
            ss = [np.array([v], dtype=np.float32) for v in ex["scale"]]
        else:
            ss = [np.array([_pow2(m, e)], dtype=np.float32)
                  for m, e in zip(ex["scale_mult"], ex["scale_exp2"])]
        off = np.array([0, qs[0].size], dtype=np.int64)
        r = o.reduce_dequant(qs, ss, off)
        want_r = np.array([np.inf if v == "inf" else v for v in ex["r"]], dtype=np.float32)
        assert np.array_equal(r, want_r), (ex["name"], r)
        sc, q = o.requantize(r, off)
        want_s = np.float32(np.inf) if ex["scale_out"] == "inf" else np.float32(ex["scale_out"])
        assert sc[0] == want_s, (ex["name"], sc)
        assert list(q) == ex["q_out"], (ex["name"], list(q))
        assert W == len(ss)


def pin_requantize_is_quantize_of_sum(o):
    """Requantize follows the same pins as quantize: torch formula on the
    reduced sum, unit by unit."""
    rng = np.random.default_rng(13)
    W, n = 5, 20000
    off = _units(n, rng)
    xs = [_random_grad(rng, n) for _ in range(W)]
    res = o.allreduce_step(xs, F32, off)
    r = res["r"]
    for u in range(off.size - 1):
        a, b = off[u], off[u + 1]
        t = torch.from_numpy(r[a:b].copy())
        s = torch.max(torch.abs(t)) / 127.0
        if not (s.item() >= float(NORMAL_MIN_SCALE)):
            continue
        want = torch.clamp(torch.round(t / s), -128, 127).to(torch.int8)
        assert res["scale_out"][u] == np.float32(s.item())
        assert np.array_equal(res["q_out"][a:b], want.numpy())



# --------------------------------------------------------------------------
# §5.2 precision check: the unquantized fp32 sum and the error report


def pin_sum_f32_single_rank(o):
    """W = 1 without the mean: the sum is the loaded gradient itself (+0
    plus g is g, except -0 which becomes +0)."""
    rng = np.random.default_rng(20)
    x = _random_grad(rng, 5000)
    x[:3] = [0.0, -0.0, np.float32(2.0 ** -149)]
    r = o.sum_f32([x], F32)
    want = x.copy()
    want[1] = 0.0
    assert np.array_equal(r.view(np.uint32), want.view(np.uint32))
    h = np.arange(0, 65536, 7, dtype=np.uint16)
    h = h[np.isfinite(h.view(np.float16))]
    r = o.sum_f32([h], F16, 2.0 ** -16)
    want = (h.view(np.float16).astype(np.float64) * 2.0 ** -16).astype(np.float32) + np.float32(0)
    assert np.array_equal(r, want)


def pin_sum_f32_closed_form(o):
    """Closed form: integer-valued gradients below 2^20 sum exactly in
    binary32 in any order; W = 4 makes the mean an exact scaling by 1/4."""
    rng = np.random.default_rng(21)
    n, W = 4000, 4
    ints = [rng.integers(-2 ** 20, 2 ** 20, n) for _ in range(W)]
    xs = [a.astype(np.float32) for a in ints]
    total = np.sum(ints, axis=0)
    assert np.array_equal(o.sum_f32(xs, F32), total.astype(np.float32))
    assert np.array_equal(o.sum_f32(xs, F32, mean=True), (total / 4.0).astype(np.float32))


def pin_sum_f32_torch_rank_order(o):
    """Library routine: torch on the CPU, acc = acc + g_w in rank order, then
    acc / W (a binary32 division) for the mean."""
    rng = np.random.default_rng(22)
    W, n = 7, 30000
    xs = [_random_grad(rng, n) * np.float32(10.0 ** rng.uniform(-3, 3)) for _ in range(W)]
    acc = torch.zeros(n, dtype=torch.float32)
    for x in xs:
        acc = acc + torch.from_numpy(x)
    assert np.array_equal(o.sum_f32(xs, F32).view(np.uint32), acc.numpy().view(np.uint32))
    mean = acc / W
    assert np.array_equal(o.sum_f32(xs, F32, mean=True).view(np.uint32),
                          mean.numpy().view(np.uint32))
    hs = [(x * np.float32(300)).astype(np.float16).view(np.uint16) for x in xs]
    acc = torch.zeros(n, dtype=torch.float32)
    for h in hs:
        acc = acc + torch.from_numpy(h.view(np.float16)).float() * 0.5
    assert np.array_equal(o.sum_f32(hs, F16, 0.5).view(np.uint32), acc.numpy().view(np.uint32))


def pin_golden_sum_f32(o):
    for ex in _golden()["sum_f32"]:
        if "x" in ex:
            xs = [np.array(row, dtype=np.float32) for row in ex["x"]]
            r = o.sum_f32(xs, F32)
            assert np.array_equal(r, np.array(ex["r"], dtype=np.float32)), (ex["name"], r)
            m = o.sum_f32(xs, F32, mean=True)
            want = np.array([_pow2(a, b) for a, b in zip(ex["mean_r_mult"], ex["mean_r_exp2"])],
                            dtype=np.float32)
            assert np.array_equal(m, want), (ex["name"], m)
        else:
            hs = [np.array(row, dtype=np.uint16) for row in ex["bits"]]
            r = o.sum_f32(hs, F16, 2.0 ** -16)
            want = np.array([_pow2(a, b) for a, b in zip(ex["r_mult"], ex["r_exp2"])],
                            dtype=np.float32)
            assert np.array_equal(r, want), (ex["name"], r)


def _stat(o_row, name):
    from oracle import STATS
    return o_row[STATS.index(name)]


def _golden_value(v):
    if isinstance(v, list):
        return v[0] / v[1]
    return float(v)


def pin_golden_error_report(o):
    from oracle import STATS
    for ex in _golden()["error_report"]:
        q = np.array(ex["q"], dtype=np.int8)
        if "scale" in ex:
            s = np.float32(ex["scale"])
        else:
            s = _pow2(ex["scale_mult"], ex["scale_exp2"])
        ref = np.array([np.nan if v == "nan" else v for v in ex["ref"]], dtype=np.float32)
        off = np.array([0, q.size], dtype=np.int64)
        row = o.error_report(q, np.array([s], np.float32), ref, off)[0]
        for name, v in ex["stats"].items():
            assert row[STATS.index(name)] == _golden_value(v), (ex["name"], name, row)
        for name in ex.get("nan_stats", []):
            assert np.isnan(row[STATS.index(name)]), (ex["name"], name, row)


def _exact_d(q, s):
    """float(q) * s rounded once to binary32 (numpy's binary32 product)."""
    return (q.astype(np.float32) * np.float32(s)).astype(np.float32)


def pin_error_report_identical_and_negated(o):
    """Closed forms: against itself the INT8 result has zero error and
    cos = 1 exactly (sqrt of a rounded square returns the value); against
    its negation the error is twice the values, mean_rel_err = 2 and
    cos = -1 exactly."""
    rng = np.random.default_rng(23)
    n = 20000
    off = _units(n, rng)
    q = rng.integers(-128, 128, n).astype(np.int8)
    sc = (rng.random(off.size - 1) * 1e-3 + 1e-6).astype(np.float32)
    d = np.concatenate([_exact_d(q[off[u]:off[u + 1]], sc[u]) for u in range(off.size - 1)])
    rep = o.error_report(q, sc, d, off)
    for u in range(off.size - 1):
        row = rep[u]
        nz = np.any(d[off[u]:off[u + 1]] != 0)
        assert _stat(row, "max_abs_err") == 0 and _stat(row, "sum_abs_err") == 0, u
        assert _stat(row, "max_rel_err") == 0 and _stat(row, "mean_rel_err") == 0, u
        assert _stat(row, "sum_dd") == _stat(row, "sum_rr") == _stat(row, "sum_dr"), u
        assert _stat(row, "cos") == 1.0, (u, nz)
    rep = o.error_report(q, sc, -d, off)
    for u in range(off.size - 1):
        row = rep[u]
        seg = d[off[u]:off[u + 1]].astype(np.float64)
        if not np.any(seg != 0):
            continue
        assert _stat(row, "max_abs_err") == 2 * np.max(np.abs(seg)), u
        assert _stat(row, "max_abs_ref") == np.max(np.abs(seg)), u
        assert _stat(row, "max_rel_err") == 2.0, u
        assert _stat(row, "mean_rel_err") == 2.0, u
        assert _stat(row, "cos") == -1.0, u


def pin_error_report_exact_rational(o):
    """Brute force in exact rational arithmetic on small units: the maxima
    are the exact maxima rounded to binary64 (rounding is monotone), and
    every sum lies within gamma_{m+1} * (sum of |terms|) of the exact sum,
    gamma_k = k u / (1 - k u), u = 2^-53, m the unit length."""
    rng = np.random.default_rng(24)
    n = 400
    off = _units(n, rng, 60)
    q = rng.integers(-128, 128, n).astype(np.int8)
    sc = (rng.random(off.size - 1) * 2.0 ** rng.uniform(-20, 20, off.size - 1)).astype(np.float32)
    ref = np.concatenate([_exact_d(q[off[u]:off[u + 1]], sc[u]) for u in range(off.size - 1)])
    ref = (ref * (1 + rng.standard_normal(n).astype(np.float32) * np.float32(0.01))
           + rng.standard_normal(n).astype(np.float32) * np.float32(1e-4)).astype(np.float32)
    rep = o.error_report(q, sc, ref, off)
    u53 = Fraction(1, 2 ** 53)
    for u in range(off.size - 1):
        a, b = int(off[u]), int(off[u + 1])
        m = b - a
        gamma = (m + 1) * u53 / (1 - (m + 1) * u53)
        d = [Fraction(float(v)) for v in _exact_d(q[a:b], sc[u])]
        r = [Fraction(float(v)) for v in ref[a:b]]
        err = [abs(x - y) for x, y in zip(d, r)]
        row = rep[u]
        assert _stat(row, "max_abs_err") == float(max(err)), u
        assert _stat(row, "max_abs_ref") == float(max(abs(y) for y in r)), u
        exact = {"sum_abs_err": (sum(err), sum(err)),
                 "sum_abs_ref": (sum(abs(y) for y in r), sum(abs(y) for y in r)),
                 "sum_dd": (sum(x * x for x in d), sum(x * x for x in d)),
                 "sum_rr": (sum(y * y for y in r), sum(y * y for y in r)),
                 "sum_dr": (sum(x * y for x, y in zip(d, r)), sum(abs(x * y) for x, y in zip(d, r)))}
        for name, (val, mag) in exact.items():
            assert abs(Fraction(_stat(row, name)) - val) <= gamma * mag, (u, name)
        cos_exact = float(exact["sum_dr"][0]) / math.sqrt(float(exact["sum_dd"][0]) *
                                                          float(exact["sum_rr"][0]))
        assert abs(_stat(row, "cos") - cos_exact) <= 8 * (m + 4) * 2.0 ** -53, u
        assert abs(_stat(row, "mean_rel_err") - float(exact["sum_abs_err"][0] /
                                                       exact["sum_abs_ref"][0])) <= \
            4 * (m + 2) * 2.0 ** -53 * _stat(row, "mean_rel_err"), u


def pin_error_report_numpy_scipy(o):
    """Library routines on larger units: numpy's binary64 max / sum / dot and
    scipy's cosine distance (1 - cos), within the summation-order bound."""
    from scipy.spatial.distance import cosine
    rng = np.random.default_rng(25)
    W, n = 4, 60000
    off = _units(n, rng, 9000)
    xs = [_random_grad(rng, n) for _ in range(W)]
    res = o.allreduce_step(xs, F32, off)
    ref = o.sum_f32(xs, F32)
    rep = o.error_report(res["q_out"], res["scale_out"], ref, off)
    for u in range(off.size - 1):
        a, b = off[u], off[u + 1]
        m = b - a
        d = _exact_d(res["q_out"][a:b], res["scale_out"][u]).astype(np.float64)
        r = ref[a:b].astype(np.float64)
        row = rep[u]
        tol = 4 * (m + 2) * 2.0 ** -53
        assert _stat(row, "max_abs_err") == np.max(np.abs(d - r)), u
        assert _stat(row, "max_abs_ref") == np.max(np.abs(r)), u
        assert abs(_stat(row, "sum_abs_err") - np.sum(np.abs(d - r))) <= tol * np.sum(np.abs(d - r)), u
        assert abs(_stat(row, "sum_dr") - np.dot(d, r)) <= tol * np.dot(np.abs(d), np.abs(r)), u
        assert abs(_stat(row, "sum_rr") - np.dot(r, r)) <= tol * np.dot(r, r), u
        if np.any(d != 0) and np.any(r != 0):
            assert abs((1 - _stat(row, "cos")) - cosine(d, r)) <= 1e-12, u
        # the INT8 result differs from the fp32 sum by at most half a code
        # step of every rank's quantization and of the requantization, plus
        # the sums' own rounding: a sanity bound a wrong unit would break
        steps = res["scale_out"][u] + sum(res["scale"][w][u] for w in range(W))
        mag = np.max(np.sum([np.abs(x[a:b].astype(np.float64)) for x in xs], axis=0))
        assert _stat(row, "max_abs_err") <= 0.5 * (1 + 2.0 ** -16) * steps + \
            2 * W * 2.0 ** -23 * mag, u


# --------------------------------------------------------------------------
# §6.2 adaptive chunk size


def pin_golden_chunker(o):
    for ex in _golden()["chunker"]:
        if "predict" in ex:
            for a, want in ex["predict"].items():
                got = o.chunker_predict(ex["sizes"], ex["lat"], alpha=float(a))
                assert got == want, (ex["name"], a, got)
        for cap, want in ex.get("predict_capacity", {}).items():
            got = o.chunker_predict(ex["sizes"], ex["lat"], capacity=int(cap), alpha=ex["alpha"])
            assert got == want, (ex["name"], cap, got)


def pin_chunker_defaults_and_single_size(o):
    """No observation gives the default; a single observed size is always
    the prediction, whatever its latencies."""
    assert o.chunker_predict([], []) == 131072
    assert o.chunker_predict([], [], default_bytes=4096) == 4096
    rng = np.random.default_rng(30)
    for _ in range(20):
        k = int(rng.integers(1, 150))
        c = int(rng.integers(1, 1 << 22))
        assert o.chunker_predict([c] * k, rng.random(k) * 10 + 1e-3) == c


def pin_chunker_constant_costs(o):
    """Closed form: when every observation of a size costs the same per
    byte, its average is that cost, so the prediction is the size with the
    smallest cost (ties to the larger size), for any alpha and any order."""
    rng = np.random.default_rng(31)
    for _ in range(40):
        m = int(rng.integers(2, 7))
        sizes = [int(v) for v in rng.choice(np.arange(1, 64), m, replace=False) * 16384]
        cost = {c: float(rng.integers(1, 6)) * 2.0 ** -20 for c in sizes}   # exact values
        seq = [sizes[int(i)] for i in rng.integers(0, m, 80)]
        lat = [cost[c] * c for c in seq]
        present = set(seq)
        want = min(present, key=lambda c: (cost[c], -c))
        for alpha in (0.25, 0.5, 1.0, 0.1):
            assert o.chunker_predict(seq, lat, alpha=alpha) == want


def pin_chunker_exact_closed_form(o):
    """Brute force in exact rational arithmetic: the average of a size with
    costs x_1..x_k (oldest first) is (1-a)^(k-1) x_1 + sum_{j>=2} a (1-a)^(k-j) x_j;
    the exact minimiser must be the prediction whenever it is not within
    1e-9 of the runner-up (a gap no rounding of these short sums reaches)."""
    rng = np.random.default_rng(32)
    checked = 0
    for _ in range(300):
        m = int(rng.integers(1, 5))
        sizes = [int(v) * 4096 for v in rng.choice(np.arange(1, 40), m, replace=False)]
        n_obs = int(rng.integers(1, 25))
        cap = int(rng.integers(1, 30))
        seq = [sizes[int(i)] for i in rng.integers(0, m, n_obs)]
        lat = [float(v) for v in rng.random(n_obs) * 5 + 0.01]
        alpha = [0.25, 0.5, 0.1, 0.75][int(rng.integers(0, 4))]
        a = Fraction(alpha)
        hist = list(zip(seq, lat))[-cap:]
        avg = {}
        for c in dict.fromkeys(s for s, _ in hist):
            xs = [Fraction(l) / c for s, l in hist if s == c]
            k = len(xs)
            avg[c] = (1 - a) ** (k - 1) * xs[0] + sum(a * (1 - a) ** (k - j) * xs[j - 1]
                                                      for j in range(2, k + 1))
        ranked = sorted(avg.items(), key=lambda kv: (kv[1], -kv[0]))
        if len(ranked) > 1 and abs(ranked[1][1] - ranked[0][1]) <= Fraction(1, 10 ** 9) * ranked[0][1]:
            continue
        assert o.chunker_predict(seq, lat, capacity=cap, alpha=alpha) == ranked[0][0], (seq, lat, cap)
        checked += 1
    assert checked > 200

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
