"""Fused FP8 producers: SwiGLU(gate, up) -> FP8 and RMSNorm -> FP8.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Jet-RL] "Quantization scheme": the activations a linear layer consumes are produced in
FP8 by the operator before it (the elementwise activation, the normalisation), fused
with the quantization, so no bf16 copy goes through memory; [SkyRL-FP8] "Performance
analysis" counts the cost of the separate quantize passes this removes. The pages give
no formula for either operator. Readings (the usual bf16 framework definitions, evaluated
exactly and rounded where that framework rounds):

* SwiGLU. The fused gate/up output GU[M][2F] holds the gate in columns [0, F) and the up
  projection in columns [F, 2F). silu(g) = g / (1 + exp(-g)) is rounded once to bf16
  (from its exact value), then multiplied by u in fp32 (round to nearest even) and
  rounded to bf16: h = bf16(fl32(bf16(silu(g)) * u)). h is then quantized exactly like
  any bf16 activation (1x128 groups, optionally 128x1).
* RMSNorm. r = fl32(1 / sqrt(mean(x^2) + eps)) per row, the fp32 rounding of the exact
  value (mean over the K entries of the row, eps the given fp32 value); then
  t = bf16(fl32(x * r)) and y = bf16(fl32(gamma * t)). y is quantized like any bf16
  activation; r is returned too (the backward pass keeps it).

Exactness. bf16(silu(g)) depends on the 65536 bf16 values of g only: the table below
holds, for every finite bf16 g, the correctly rounded bf16 of silu(g), computed with
60-digit decimal arithmetic (no libm). For RMSNorm, the row's r is computed in fp64 (an
exactly rounded sum of the exact squares, then one division, sqrt and reciprocal);
`rmsnorm_bf16` also reports the rows whose exact r could lie within 2**-38 (relative)
of an fp32 rounding midpoint, where an fp64 evaluation in another order could round the
other way. Everything after r is exact fp32/bf16 arithmetic.

Pinned by tests/test_oracle_producers.py: the silu table against an independent fp64
evaluation through math.exp for all 65536 inputs, the identity silu(x) - silu(-x) = x on
the exact values, closed forms (silu(0) = 0; silu(g) rounds to g for large g); the fp32
multiply and bf16 rounding against torch's bf16 multiply; the gate/up column order; r
against exact rational bounds (r is the fp32 value whose rounding interval contains
1/sqrt(v), checked as m1^2 v < 1 < m2^2 v in fractions); closed forms for rows of
constant magnitude; invariance of y under x -> 2^j x when eps = 0.
"""

from __future__ import annotations

import decimal
import math
from functools import lru_cache

import numpy as np

from .fp8_formats import round_to_bf16
from .quantize import (quant_act_1x128, quant_act_128x1, quant_act_1x128_pow2, quant_act_128x1_pow2)

_CTX = decimal.Context(prec=60, Emin=-10 ** 6, Emax=10 ** 6, traps=[])
_WIDE = decimal.Context(prec=400, Emin=-10 ** 6, Emax=10 ** 6, traps=[decimal.Inexact])


def _bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _round_decimal_to_bf16(v: decimal.Decimal, negative: bool) -> float:
    """Round a 60-digit value to bf16, ties to even, by an exact comparison with the
    midpoint of its two bf16 neighbours. `negative` gives the sign of a value that
    underflowed to zero."""
    if v == 0:
        return -0.0 if negative else 0.0
    a = v.copy_abs()                                 # exact (abs() would round to the default context)
    f = float(a)                                     # correctly rounded to fp64
    lo = float(round_to_bf16(np.float32(f)))         # a bf16 value near a
    # walk to the bf16 pair (lo, hi) with lo <= a < hi, exactly
    def nxt(x, up):
        bits = np.array([x], np.float32).view(np.uint32)[0] >> 16
        bits = bits + 1 if up else bits - 1
        return float(np.array([bits << 16], np.uint32).view(np.float32)[0])
    while decimal.Decimal(lo) > a:
        lo = nxt(lo, False)
    hi = nxt(lo, True)
    while decimal.Decimal(hi) <= a:
        lo, hi = hi, nxt(hi, True)
    if math.isinf(hi):                                         # |silu(g)| <= |g| <= the bf16 maximum
        return -lo if v < 0 else lo
    # bf16 values are short binary fractions (at most ~100 significant decimal digits), so
    # their midpoint is exact in 400 digits; the comparison with a is exact.
    mid = _WIDE.divide(_WIDE.add(decimal.Decimal(lo), decimal.Decimal(hi)), 2)
    if a < mid:
        r = lo
    elif a > mid:
        r = hi
    else:                                                      # a tie (silu of 0 only gives 0 above)
        r = lo if (np.array([lo], np.float32).view(np.uint32)[0] >> 16) % 2 == 0 else hi
    return -r if (v < 0) else r


def silu_exact(g: float) -> decimal.Decimal:
    """silu(g) = g / (1 + exp(-g)) to 60 significant digits."""
    d = decimal.Decimal(g)                           # exact
    if d >= 0:
        return _CTX.divide(d, _CTX.add(1, _CTX.exp(-d)))
    e = _CTX.exp(d)                                  # exp(g) <= 1: no overflow for very negative g
    return _CTX.divide(_CTX.multiply(d, e), _CTX.add(1, e))


@lru_cache(maxsize=1)
def silu_bf16_table() -> np.ndarray:
    """float32 [65536]: entry b is bf16(silu(g)) for the bf16 value g with bit pattern b
    (NaN for the non-finite patterns, which are outside the contract)."""
    out = np.full(65536, np.nan, np.float32)
    g_all = _bf16_bits_to_f64(np.arange(65536))
    for b in range(65536):
        g = g_all[b]
        if not math.isfinite(g):
            continue
        out[b] = _round_decimal_to_bf16(silu_exact(g), negative=(g < 0 or (g == 0 and math.copysign(1, g) < 0)))
    return out


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("inputs must be bf16 values")
    return (bits >> 16).astype(np.int64)


def swiglu_bf16(gu) -> np.ndarray:
    """h[M][F] = bf16(fl32(bf16(silu(gate)) * up)) for GU[M][2F] = [gate | up]."""
    gu = np.asarray(gu, dtype=np.float32)
    M, F2 = gu.shape
    if F2 % 2:
        raise ValueError("GU must have an even number of columns")
    F = F2 // 2
    g, u = gu[:, :F], gu[:, F:]
    s = silu_bf16_table()[_bf16_bits(g)]
    _bf16_bits(u)
    p = (s.astype(np.float32) * u.astype(np.float32)).astype(np.float32)      # fp32 multiply, RNE
    return round_to_bf16(p)


def swiglu_quant_1x128(gu, pow2: bool = False, colwise: bool = False):
    """SwiGLU then 1x128 quantization (+ 128x1 if colwise).
    Returns (q, s) or (q, s, qt, st)."""
    h = swiglu_bf16(gu)
    rows = quant_act_1x128_pow2(h) if pow2 else quant_act_1x128(h)
    if not colwise:
        return rows
    cols = quant_act_128x1_pow2(h) if pow2 else quant_act_128x1(h)
    return rows + cols


def _fp32_neighbours(r64: np.ndarray):
    r32 = r64.astype(np.float32)
    up = np.nextafter(r32, np.float32(np.inf))
    dn = np.nextafter(r32, np.float32(0))
    return r32, dn, up


def rms_rstd(x, eps: float):
    """r = fl32(1 / sqrt(mean(x^2) + eps)) per row, and the rows where the fp64 evaluation
    lies within 2**-38 (relative) of an fp32 rounding midpoint (ambiguous rows).
    Returns (r float32 [M], ambiguous bool [M])."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    eps64 = float(np.float32(eps))
    r64 = np.empty(M, np.float64)
    for m in range(M):
        ss = math.fsum((x[m].astype(np.float64) ** 2).tolist())     # squares are exact in fp64
        r64[m] = 1.0 / math.sqrt(ss / K + eps64)
    r32, dn, up = _fp32_neighbours(r64)
    lo_mid = (r32.astype(np.float64) + dn.astype(np.float64)) / 2
    hi_mid = (r32.astype(np.float64) + up.astype(np.float64)) / 2
    dist = np.minimum(np.abs(r64 - lo_mid), np.abs(hi_mid - r64)) / r64
    return r32, dist < 2.0 ** -38


def rmsnorm_bf16(x, gamma, eps: float):
    """y[M][K] = bf16(fl32(gamma * bf16(fl32(x * r)))). Returns (y, r, ambiguous_rows)."""
    x = np.asarray(x, dtype=np.float32)
    gamma = np.asarray(gamma, dtype=np.float32)
    _bf16_bits(x)
    _bf16_bits(gamma)
    if gamma.shape != (x.shape[1],):
        raise ValueError("gamma must have one entry per column")
    r, amb = rms_rstd(x, eps)
    t = round_to_bf16((x * r[:, None]).astype(np.float32))
    y = round_to_bf16((gamma[None, :] * t).astype(np.float32))
    return y, r, amb


def rmsnorm_quant_1x128(x, gamma, eps: float, pow2: bool = False, colwise: bool = False):
    """RMSNorm then 1x128 quantization (+ 128x1 if colwise).
    Returns (q, s, r, ambiguous_rows) or (q, s, qt, st, r, ambiguous_rows)."""
    y, r, amb = rmsnorm_bf16(x, gamma, eps)
    rows = quant_act_1x128_pow2(y) if pow2 else quant_act_1x128(y)
    if colwise:
        rows = rows + (quant_act_128x1_pow2(y) if pow2 else quant_act_128x1(y))
    return rows + (r, amb)
