"""Number formats: FP8 E4M3, the E8M0 power-of-two scale byte, and bf16 rounding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[AIS] format table: E4M3 is 1 sign bit, 4 exponent bits and 3 mantissa bits;
BF16 is 1/8/7. The pages never state the exponent bias, the NaN encoding, the
largest finite value or the rounding mode. Readings taken here (the plainest
ones consistent with the rest of the pages and with a maximum of 448):

* E4M3 is the "FN" flavour: bias 7, subnormals at exponent field 0, no
  infinities, NaN only at 0x7F / 0xFF, largest finite value 0x7E = 448.
* Encoding rounds to nearest with ties to the even mantissa (the [AIS]
  quantizer equation rounds to a nearby representable value), saturates finite
  magnitudes above 448 to 448, and keeps the sign of zero.
* E8M0 ([SkyRL-FP8] "Deep dive: FP8 quantization with FP32 and power-of-two
  block scales": power-of-two scales carry an exponent only) is a biased
  exponent byte: value 2**(b - 127), 255 is NaN.

Pinned by: torch's ``float8_e4m3fn`` / ``float8_e8m0fnu`` / ``bfloat16`` CPU
conversions, an independent nearest-in-table encoder, and the worked rounding
example on the [AIS] page (tests/test_oracle_formats.py).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_EXP = -6          # exponent of the smallest normal binade (2**-6)
_E4M3_MAN_BITS = 3
_E4M3_BIAS = 7


def decode_e4m3(codes) -> np.ndarray:
    """E4M3 byte -> value (fp64). Exponent field 0 is subnormal: m * 2**-9.

    Otherwise (1 + m/8) * 2**(e - 7). 0x7F and 0xFF decode to NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - _E4M3_BIAS).astype(np.float64)))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def _round_to_grid(a: np.ndarray, man_bits: int, min_exp: int) -> np.ndarray:
    """Round non-negative fp64 values to the binary grid with ``man_bits``
    stored mantissa bits whose smallest normal binade is 2**min_exp (values
    below it are on the subnormal grid of that binade). Ties go to the even
    grid point. Exact for inputs that are fp32 or narrower."""
    _, ex = np.frexp(a)                     # a = f * 2**ex with f in [0.5, 1)
    e = np.maximum(ex - 1, min_exp)         # binade exponent, floored at the subnormal binade
    quantum = np.ldexp(1.0, (e - man_bits).astype(np.int64))
    n = np.rint(a / quantum)                # division by a power of two is exact; rint ties to even
    return n * quantum


def e4m3_round(v) -> np.ndarray:
    """Value of the E4M3 encoding of ``v`` (fp64 out): RNE, saturate to +-448."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encode: non-finite input is outside the contract")
    r = np.minimum(_round_to_grid(np.abs(v), _E4M3_MAN_BITS, _E4M3_MIN_EXP), E4M3_MAX)
    return np.where(np.signbit(v), -r, r)


def encode_e4m3(v) -> np.ndarray:
    """Real values (fp32 or fp64, finite) -> E4M3 bytes (uint8).

    Round to nearest on the E4M3 grid (subnormals included), ties to even,
    then saturate magnitudes above 448 to 448. Negative inputs that round to
    zero give 0x80 (negative zero).
    """
    v = np.asarray(v, dtype=np.float64)
    r = np.abs(e4m3_round(v))
    _, ex = np.frexp(r)
    E = ex - 1                                            # binade of the rounded value
    sub = r < 2.0 ** _E4M3_MIN_EXP
    # subnormal and zero: code = r / 2**-9 (0..7); normal: exponent field E + 7, mantissa r / 2**(E-3) - 8
    man_normal = r / np.ldexp(1.0, (E - _E4M3_MAN_BITS).astype(np.int64)) - 8.0
    code = np.where(sub, r / 2.0 ** -9, (E + _E4M3_BIAS) * 8.0 + man_normal)
    code = code.astype(np.int64)
    code = np.where(np.signbit(v), code | 0x80, code)
    return code.astype(np.uint8)


def decode_e8m0(b) -> np.ndarray:
    """E8M0 scale byte -> 2**(b - 127) in fp64; 255 is NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def round_to_bf16(v) -> np.ndarray:
    """Round fp32 values to bf16 (8 significant bits, fp32's exponent range,
    ties to even) and return them as fp32. Finite inputs only."""
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("bf16 rounding: non-finite input is outside the contract")
    a = np.abs(v).astype(np.float64)
    r = _round_to_grid(a, 7, -126)
    r = np.where(np.signbit(v), -r, r)
    return r.astype(np.float32)      # exact: r has <= 8 significant bits in fp32's range (or is +-inf on overflow)
