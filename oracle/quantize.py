"""Fine-grained FP8 quantizers: 1x128 / 128x1 activation groups, 128x128 weight
blocks, and MXFP8 1x32 groups with a power-of-two (E8M0) scale.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The quantizer is the symmetric one of the [AIS] quantizer equation, with the
integer grid replaced by the E4M3 grid: s = max|X| / qmax over the group, with
qmax = 448 for E4M3, and Q = E4M3(X / s). Granularities:

* activations: one scale per 1x128 group along K ([Jet-RL] "Quantization
  scheme"; [SkyRL-FP8] "Why FP8 matters for RL" on fine-grained block scaling);
* weights: one scale per 128x128 block ([SkyRL-FP8] same section and
  "When independent quantization breaks policy consistency"; [Jet-RL]);
* WGrad operands: 128x1 groups along the token dimension ([Jet-RL]
  "Quantization scheme", backward pass);
* MXFP8: one power-of-two scale per 1x32 group ([SkyRL-FP8] "When independent
  quantization breaks policy consistency" and the "Deep dive" section:
  exponent-only scales, up to 2x coarser); for the backward operands of a dense
  MXFP8 linear layer, 32x1 groups along the token (or output-feature) dimension,
  written transposed.

Readings where the pages are silent:

* s = fl32(amax / 448) is an IEEE fp32 division (round to nearest even), and
  the scaled value is the fp32 quotient fl32(x / s) (a true division, not a
  reciprocal multiply); that fp32 value is then encoded to E4M3.
* A group whose amax is 0 gets s = 1.0 (its codes are +-0).
* Column-wise (128x1) quantization of X[M][K] is row-wise quantization of
  X transposed, from the original bf16 values; outputs are qt[K][M], st[K][M/128].
* MX scale exponent: the smallest integer e with amax <= 448 * 2**e (so the
  scale is rounded up from amax/448 and nothing saturates), clamped to
  [-127, 127]; amax = 0 gives e = 0. The E8M0 byte is e + 127, and
  q = E4M3(x * 2**-e) with the power-of-two scaling exact.

Power-of-two block scales ([SkyRL-FP8] "Deep dive: FP8 quantization with FP32 and
power-of-two block scales": the same blockwise granularity with exponent-only scales).
Reading: the MX exponent rule applied to the 1x128 / 128x1 / 128x128 group, i.e.
s = 2**e with e the smallest integer such that amax <= 448 * 2**e, clamped to
[-127, 127] (0 for an all-zero group), stored as an fp32 value; q = E4M3(x * 2**-e),
an exact scaling, which never saturates.

Pinned by tests/test_oracle_quantize.py: a pure-Python brute force with exact
fractions and a nearest-in-table encoder on small groups, the invariants that
the amax element of every group encodes to +-448 and that a group scaled by
2**j keeps its codes with the scale scaled by 2**j, the half-ulp error bound,
group locality (changing one element changes only its own group), and the MX
invariant 224 < amax * 2**-e <= 448; the MX 32x1 (transposed) layout by a
brute force over columns. The power-of-two block quantizers: the same
brute force with exponent-only scales for all three layouts, 224 < amax / s <= 448,
2**j equivariance, and fl32(amax / 448) <= s < 2 fl32(amax / 448).
"""

from __future__ import annotations

import numpy as np

from .fp8_formats import E4M3_MAX, encode_e4m3

GROUP = 128          # 1x128, 128x1 and 128x128 granularity
MX_GROUP = 32        # MXFP8 1x32 granularity


def _as_f32(x) -> np.ndarray:
    """The quantizers take bf16 tensors, passed as float32 arrays of bf16-exact values."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantizer input must be finite")
    if np.any(x.view(np.uint32) & 0xFFFF):
        raise ValueError("quantizer input must hold bf16 values (float32 with the low 16 bits zero)")
    return x


def _scale_from_amax(amax: np.ndarray) -> np.ndarray:
    """s = fl32(amax / 448); 1.0 where amax == 0."""
    amax = amax.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = amax / np.float32(E4M3_MAX)          # numpy fp32 division: IEEE, round to nearest even
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quant_act_1x128(x):
    """Row-wise 1x128 quantization of X[M][K] (K % 128 == 0).

    Returns (q uint8 [M][K], s float32 [M][K/128]).
    """
    x = _as_f32(x)
    M, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = x.reshape(M, K // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2) if M else np.zeros((0, K // GROUP), np.float32)
    s = _scale_from_amax(amax)
    q = encode_e4m3(g / s[:, :, None])          # fp32 / fp32 -> fp32 quotient
    return q.reshape(M, K), s


def quant_act_128x1(x):
    """Column-wise 128x1 quantization of X[M][K] (M % 128 == 0): groups of 128
    consecutive rows (tokens) in each column, written transposed.

    Returns (qt uint8 [K][M], st float32 [K][M/128]).
    """
    x = _as_f32(x)
    if x.shape[0] % GROUP:
        raise ValueError("M must be a multiple of 128 for 128x1 groups")
    return quant_act_1x128(np.ascontiguousarray(x.T))


def quant_w_128x128(w):
    """128x128 block quantization of W[N][K] (N % 128 == 0, K % 128 == 0).

    Returns (q uint8 [N][K], s float32 [N/128][K/128]).
    """
    w = _as_f32(w)
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("N and K must be multiples of 128")
    b = w.reshape(N // GROUP, GROUP, K // GROUP, GROUP)
    amax = np.max(np.abs(b), axis=(1, 3))
    s = _scale_from_amax(amax)
    q = encode_e4m3(b / s[:, None, :, None])
    return q.reshape(N, K), s


def transpose_payload(q):
    """Byte transpose of an FP8 payload (used for the DGrad weight operand:
    a 128x128 block stays a 128x128 block, so its scale is reused unchanged)."""
    return np.ascontiguousarray(np.asarray(q, dtype=np.uint8).T)


def mx_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2**e, clamped to [-127, 127]; 0 for amax == 0."""
    a = np.asarray(amax, dtype=np.float64)
    f, ex = np.frexp(a)                        # a = f * 2**ex, f in [0.5, 1)
    F = ex - 1                                 # a in [2**F, 2**(F+1))
    e = F - 8                                  # 448 * 2**(F-8) = 1.75 * 2**F
    e = np.where(a <= E4M3_MAX * np.ldexp(1.0, e), e, e + 1)
    e = np.where(a == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int64)


def _pow2_scale(amax):
    """e = mx_exponent(amax) and s = 2**e as fp32 (exact, also at 2**-127)."""
    e = mx_exponent(amax)
    return e, np.ldexp(np.float64(1.0), e).astype(np.float32)


def quant_act_1x128_pow2(x):
    """1x128 quantization of X[M][K] with power-of-two scales.

    Returns (q uint8 [M][K], s float32 [M][K/128], every s a power of two)."""
    x = _as_f32(x)
    M, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = x.reshape(M, K // GROUP, GROUP).astype(np.float64)
    amax = np.max(np.abs(g), axis=2) if M else np.zeros((0, K // GROUP))
    e, s = _pow2_scale(amax)
    q = encode_e4m3(np.ldexp(g, -e[:, :, None]))      # exact power-of-two scaling in fp64
    return q.reshape(M, K), s


def quant_act_128x1_pow2(x):
    """128x1 quantization with power-of-two scales, written transposed: row-wise of X^T.

    Returns (qt uint8 [K][M], st float32 [K][M/128])."""
    x = _as_f32(x)
    if x.shape[0] % GROUP:
        raise ValueError("M must be a multiple of 128 for 128x1 groups")
    return quant_act_1x128_pow2(np.ascontiguousarray(x.T))


def quant_w_128x128_pow2(w):
    """128x128 block quantization of W[N][K] with power-of-two scales.

    Returns (q uint8 [N][K], s float32 [N/128][K/128])."""
    w = _as_f32(w)
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("N and K must be multiples of 128")
    b = w.reshape(N // GROUP, GROUP, K // GROUP, GROUP).astype(np.float64)
    amax = np.max(np.abs(b), axis=(1, 3))
    e, s = _pow2_scale(amax)
    q = encode_e4m3(np.ldexp(b, -e[:, None, :, None]))
    return q.reshape(N, K), s


def quant_mx_1x32(x):
    """MXFP8 quantization of X[R][K] (K % 32 == 0): one E8M0 scale per 1x32 group.

    Returns (q uint8 [R][K], e8m0 uint8 [R][K/32]).
    """
    x = _as_f32(x)
    R, K = x.shape
    if K % MX_GROUP:
        raise ValueError("K must be a multiple of 32")
    g = x.reshape(R, K // MX_GROUP, MX_GROUP).astype(np.float64)
    amax = np.max(np.abs(g), axis=2) if R else np.zeros((0, K // MX_GROUP))
    e = mx_exponent(amax)
    q = encode_e4m3(np.ldexp(g, -e[:, :, None]))     # exact power-of-two scaling in fp64
    return q.reshape(R, K), (e + 127).astype(np.uint8)


def quant_mx_32x1(x):
    """MXFP8 quantization with 32x1 groups along the rows of X[R][K] (R % 32 == 0), written
    transposed: the operand layout of a GEMM that contracts over R (the MXFP8 recipe's
    backward operands, [SkyRL-FP8] "When independent quantization breaks policy
    consistency": 1x32 blocks along the contraction dimension). Element (r, k) is quantized
    with the group of rows 32 * (r // 32) .. +31 of column k.

    Returns (qt uint8 [K][R], e8m0t uint8 [K][R/32])."""
    x = _as_f32(x)
    if x.shape[0] % MX_GROUP:
        raise ValueError("R must be a multiple of 32 for 32x1 groups")
    return quant_mx_1x32(np.ascontiguousarray(x.T))

