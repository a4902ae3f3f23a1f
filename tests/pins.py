"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch,
so that the same list runs against the real oracle (test_oracle_pins.py) and
against deliberately broken copies of it (test_oracle_mutants.py).

Method source: the pipelined HCCL AllReduce article
(bjdmk.com.cn/news/6235379): §2.1 dynamic_chunk, §2.2.1 quantize_gradient
and the INT8 AllReduce, §6.1 unscale before quantizing.
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


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
