"""Pins of oracle/producers.py (fused SwiGLU / RMSNorm -> FP8) against values fixed by
the mathematics and by independent implementations: an fp64 math.exp evaluation of silu
over every bf16 input, exact rational bounds for the RMS reciprocal, torch's bf16
multiply, closed forms and invariants."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import producers as P
from oracle import quantize as OQ
from oracle.fp8_formats import round_to_bf16
import workloads as W


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    v = (b << 16).view(np.float32)
    ok = np.isfinite(v)
    return b[ok], v[ok]


def _bf16_grid_step(a: float) -> float:
    """Spacing of the bf16 values around the magnitude a (fixed 2^-133 below 2^-126)."""
    if a < 2.0 ** -126:
        return 2.0 ** -133
    return math.ldexp(1.0, math.frexp(a)[1] - 8)


def _tie_side_of_grid(a: float) -> float:
    """Relative distance of a > 0 to the nearest midpoint between bf16 neighbours."""
    step = _bf16_grid_step(a)
    lo = math.floor(a / step) * step
    return abs(a - (lo + step / 2)) / a


def test_silu_table_matches_independent_fp64_evaluation():
    """For every finite bf16 g with |g| >= 2^-100: the table equals the bf16 rounding of an
    fp64 evaluation through math.exp (another library, another arrangement of the formula),
    and that fp64 value is never within 2^-40 (relative) of a bf16 rounding midpoint, so
    the rounding is unambiguous."""
    bits, g = _all_finite_bf16()
    tab = P.silu_bf16_table()[bits]
    n = 0
    for b, gv, t in zip(bits.tolist(), g.astype(np.float64).tolist(), tab.tolist()):
        if abs(gv) < 2.0 ** -100:
            continue
        if gv >= 0:
            s = gv / (1.0 + math.exp(-gv))
        else:
            e = math.exp(gv)
            s = gv * e / (1.0 + e)
        if s != 0.0:
            assert _tie_side_of_grid(abs(s)) > 2.0 ** -40, (hex(b), gv, s)
        a = abs(s)
        step = _bf16_grid_step(a) if a > 0 else 1.0
        r = math.floor(a / step + 0.5) * step if a > 0 else 0.0          # no ties, by the assert above
        r = -r if (s < 0 or (s == 0 and gv < 0)) else r
        assert t == r and (t != 0 or math.copysign(1, t) == math.copysign(1, r)), (hex(b), gv, t, r)
        n += 1
    assert n > 55000


def test_silu_table_tiny_inputs_closed_form():
    """|g| < 2^-100: silu(g) = g/2 + g^2/4 + O(g^3), so bf16(silu(g)) is g/2 rounded to bf16,
    where a tie (g/2 exactly halfway between two bf16 values, which happens for |g| < 2^-125)
    goes up in magnitude for g > 0 and down for g < 0 (the g^2/4 term decides)."""
    bits, g = _all_finite_bf16()
    tab = P.silu_bf16_table()[bits]
    ties = 0
    for gv, t in zip(g.astype(np.float64).tolist(), tab.tolist()):
        if abs(gv) >= 2.0 ** -100 or gv == 0:
            continue
        half = abs(gv) / 2                                   # exact
        step = _bf16_grid_step(half)
        k = half / step
        if k == math.floor(k) + 0.5:
            ties += 1
            mag = (math.floor(k) + (1 if gv > 0 else 0)) * step
        else:
            mag = math.floor(k + 0.5) * step
        assert abs(t) == mag and math.copysign(1, t) == math.copysign(1, gv), (gv, t, mag)
    assert ties > 100


def test_silu_identity_and_closed_forms():
    # silu(x) - silu(-x) = x on the exact values
    for x in [0.5, 1.0, 3.0, 7.25, 20.0, 1e-3, 100.0]:
        d = P.silu_exact(x) - P.silu_exact(-x)
        assert abs(float(d) - x) <= 1e-40 * max(1.0, x)
    tab = P.silu_bf16_table()
    assert tab[0x0000] == 0.0 and not np.signbit(tab[0x0000])
    assert tab[0x8000] == 0.0 and np.signbit(tab[0x8000])
    # sigmoid(0) = 1/2: silu(2^-k) = 2^-(k+1) + ... rounds to bf16(2^-k / 2 * (1 + 2^-k / 2)); k = 20 -> 2^-21 exactly
    assert tab[np.array([2.0 ** -20], np.float32).view(np.uint32)[0] >> 16] == np.float32(2.0 ** -21)
    # large g: silu(g) rounds to g; very negative g: rounds to -0
    for g in [64.0, 1000.0, 3.0e38]:
        b = np.array([g], np.float32)
        b = round_to_bf16(b).view(np.uint32)[0] >> 16
        assert tab[b] == round_to_bf16(np.float32(g))
    b = round_to_bf16(np.array([-200.0], np.float32)).view(np.uint32)[0] >> 16
    assert tab[b] == 0.0 and np.signbit(tab[b])
    # silu(-1) = -1/(1+e): -0.26894142 -> bf16 -0.26953125 (neighbours -0.267578125 / -0.26953125)
    assert tab[0xBF80] == np.float32(-0.26953125)


def test_swiglu_layout_and_product_rounding():
    rng = np.random.default_rng(0)
    M, F = 8, 256
    g = W.bf16_round(rng.standard_normal((M, F)).astype(np.float32) * 2)
    u = W.bf16_round(rng.standard_normal((M, F)).astype(np.float32) * 2)
    h = P.swiglu_bf16(np.concatenate([g, u], 1))
    s = P.silu_bf16_table()[(g.view(np.uint32) >> 16).astype(np.int64)]
    # torch: bf16 * bf16 computes the fp32 product and rounds it to bf16
    ref = (torch.from_numpy(s).to(torch.bfloat16) * torch.from_numpy(u).to(torch.bfloat16)).float().numpy()
    assert np.array_equal(h.view(np.uint32), ref.view(np.uint32))
    # gate first: up = 1 gives silu(gate); a large positive gate gives up
    ones = np.ones_like(g)
    assert np.array_equal(P.swiglu_bf16(np.concatenate([g, ones], 1)), s)
    big = np.full_like(g, 64.0)
    assert np.array_equal(P.swiglu_bf16(np.concatenate([big, u], 1)), round_to_bf16(64.0 * u))
    with pytest.raises(ValueError):
        P.swiglu_bf16(np.concatenate([g, u], 1) + np.float32(1e-3))         # not bf16 values


def test_swiglu_quant_is_the_quantizer_on_h():
    rng = np.random.default_rng(1)
    gu = W.bf16_round(rng.standard_normal((256, 512)).astype(np.float32))
    q, s, qt, st = P.swiglu_quant_1x128(gu, colwise=True)
    h = P.swiglu_bf16(gu)
    rq, rs = OQ.quant_act_1x128(h)
    rqt, rst = OQ.quant_act_128x1(h)
    assert np.array_equal(q, rq) and np.array_equal(s, rs) and np.array_equal(qt, rqt) and np.array_equal(st, rst)


def _exact_r_check(row, eps, r32):
    """r32 is the fp32 value whose rounding interval contains 1/sqrt(v), v = mean(x^2) + eps:
    with m1 < m2 the midpoints to its neighbours, m1^2 v < 1 < m2^2 v (exact rationals)."""
    v = sum(Fraction(float(a)) ** 2 for a in row) / len(row) + Fraction(float(np.float32(eps)))
    r = Fraction(float(r32))
    up = Fraction(float(np.nextafter(r32, np.float32(np.inf))))
    dn = Fraction(float(np.nextafter(r32, np.float32(0))))
    m1, m2 = (r + dn) / 2, (r + up) / 2
    return m1 * m1 * v < 1 < m2 * m2 * v


def test_rms_reciprocal_exact_bounds():
    rng = np.random.default_rng(2)
    x = W.bf16_round(rng.standard_normal((24, 384)).astype(np.float32) * np.float32(3.0))
    x[3] *= np.float32(2.0 ** -60)
    x[4] = W.bf16_round(x[4] * np.float32(2.0 ** 60))
    x[5, ::2] = 0.0
    r, amb = P.rms_rstd(x, 1e-6)
    assert not amb.any()
    for m in range(x.shape[0]):
        assert _exact_r_check(x[m], 1e-6, r[m]), m


def test_rmsnorm_closed_form_and_scale_invariance():
    K = 256
    gamma = W.bf16_round(1.0 + np.random.default_rng(3).standard_normal(K).astype(np.float32) * np.float32(0.1))
    x = np.full((2, K), 4.0, np.float32)
    x[1, ::3] = -4.0
    y, r, _ = P.rmsnorm_bf16(x, gamma, 0.0)
    assert np.all(r == np.float32(0.25))
    assert np.array_equal(y, np.sign(x) * gamma[None, :])
    rng = np.random.default_rng(4)
    x = W.bf16_round(rng.standard_normal((6, K)).astype(np.float32))
    y0, r0, _ = P.rmsnorm_bf16(x, gamma, 0.0)
    for j in (-20, -3, 5, 30):
        yj, rj, _ = P.rmsnorm_bf16(x * np.float32(2.0 ** j), gamma, 0.0)
        assert np.array_equal(yj, y0)
        assert np.array_equal(rj, r0 * np.float32(2.0 ** -j))


def test_rmsnorm_close_to_plain_fp64_and_quant_composition():
    rng = np.random.default_rng(5)
    x = W.bf16_round(rng.standard_normal((128, 512)).astype(np.float32))
    gamma = W.bf16_round(1.0 + rng.standard_normal(512).astype(np.float32) * np.float32(0.1))
    y, r, _ = P.rmsnorm_bf16(x, gamma, 1e-6)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt(np.mean(x64 ** 2, axis=1, keepdims=True) + float(np.float32(1e-6))) * gamma
    assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2.0 ** -7     # two bf16 roundings
    q, s, qt, st, r2, _ = P.rmsnorm_quant_1x128(x, gamma, 1e-6, colwise=True)
    rq, rs = OQ.quant_act_1x128(y)
    rqt, rst = OQ.quant_act_128x1(y)
    assert np.array_equal(q, rq) and np.array_equal(s, rs) and np.array_equal(qt, rqt) and np.array_equal(st, rst)
    assert np.array_equal(r, r2)
    qp, sp = P.rmsnorm_quant_1x128(x, gamma, 1e-6, pow2=True)[:2]
    rqp, rsp = OQ.quant_act_1x128_pow2(y)
    assert np.array_equal(qp, rqp) and np.array_equal(sp, rsp)


def _round_binary(fr: Fraction, p: int, emin: int) -> Fraction:
    """Exact round-to-nearest-even of a rational to a binary format with p significant bits
    whose smallest normal binade is 2^emin (subnormals below it); integer arithmetic only."""
    if fr == 0:
        return Fraction(0)
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, emin) - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return (fl * quantum) if fr > 0 else -(fl * quantum)


def _f32r(fr):
    return _round_binary(fr, 24, -126)


def _bf16r(fr):
    return _round_binary(fr, 8, -126)


def test_rmsnorm_exact_rational_brute_force():
    """y = bf16(fl32(gamma * bf16(fl32(x * r)))) recomputed in exact rationals from r (itself
    checked against the exact reciprocal square root). The rows and gamma are such that each
    plausible mis-reading changes y somewhere: dropping the inner bf16 rounding, multiplying
    by gamma before r, or rounding the whole product once."""
    rng = np.random.default_rng(6)
    M, K = 8, 128
    x = W.bf16_round(rng.standard_normal((M, K)).astype(np.float32) * np.float32(1.7))
    x[1] = W.bf16_round(x[1] * np.float32(2.0 ** -20))
    x[2, ::5] = 0.0
    gamma = W.bf16_round(1.0 + rng.standard_normal(K).astype(np.float32) * np.float32(0.3))
    y, r, amb = P.rmsnorm_bf16(x, gamma, 1e-6)
    assert not amb.any()
    miss = {"no_inner_bf16": 0, "gamma_first": 0, "single_rounding": 0}
    for m in range(M):
        assert _exact_r_check(x[m], 1e-6, r[m]), m
        rf = Fraction(float(r[m]))
        for k in range(K):
            xf, gf = Fraction(float(x[m, k])), Fraction(float(gamma[k]))
            t = _bf16r(_f32r(xf * rf))
            want = _bf16r(_f32r(gf * t))
            assert Fraction(float(y[m, k])) == want, (m, k)
            miss["no_inner_bf16"] += _bf16r(_f32r(gf * _f32r(xf * rf))) != want
            miss["gamma_first"] += _bf16r(_f32r(_f32r(gf * xf) * rf)) != want
            miss["single_rounding"] += _bf16r(gf * xf * rf) != want
    assert all(v > 0 for v in miss.values()), miss
