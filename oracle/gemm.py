"""Block-scaled FP8 GEMMs, defined as products of the dequantized operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every GEMM here is the plain definition: dequantize each operand (E4M3 value
times the scale of the group or block the element belongs to, exact in fp64),
then multiply in fp64. The result differs from the exact real product only by
fp64 rounding (relative error of order K * 2**-53 of the sum of |terms|), far
below any tolerance used against the GPU.

* forward   Y  = X . W^T     X: 1x128 groups, W: 128x128 blocks
  ([SkyRL-FP8] TL;DR and "Why FP8 matters for RL": FP8 linear-layer GEMMs with
  fine-grained block scaling; [Jet-RL] "Quantization scheme").
* DGrad     dX = dY . W      dY: 1x128 groups, W: 128x128 blocks
* WGrad     dW = dY^T . X    both operands grouped 128x1 along the token dim,
  i.e. the column-wise (transposed) quantized copies
  ([Jet-RL] "Quantization scheme", backward pass: DGrad and WGrad run in FP8,
  WGrad with 1x128 and 128x1 groups).
* MXFP8 dense linear ([SkyRL-FP8]: the MXFP8 recipe for the linear layers; 1x32
  blocks along each GEMM's contraction dimension):
    forward  Y  = X . W^T    X [M][K], W [N][K], 1x32 groups along K;
    DGrad    dX = dY . W     dY [M][N] 1x32 along N; W quantized 32x1 along N,
                             i.e. the transposed copy Wt [K][N] with 1x32 groups;
    WGrad    dW = dY^T . X   both 32x1 along the tokens: dYt [N][M], Xt [K][M].
* grouped   per expert e, rows [off[e], off[e+1]) of the routed activations
  times expert e's weight ([SkyRL-FP8] MoE experts hold most parameters), in either
  recipe: MXFP8 1x32 scales on both operands, or the blockwise recipe (activation
  rows in 1x128 groups, each expert's weight in 128x128 blocks, as for the dense
  forward).

Pinned by tests/test_oracle_gemm.py: an exact-rational (fractions.Fraction)
triple loop on small non-square shapes with per-element scale lookup; the
grouped GEMMs (both recipes) equal the dense GEMM per expert and for a single expert, and
the blockwise one also matches the exact-rational loop; the MXFP8 dense
GEMMs by the same exact-rational loop with E8M0 scales looked up per 32-element block.
"""

from __future__ import annotations

import numpy as np

from .fp8_formats import decode_e4m3, decode_e8m0
from .quantize import GROUP, MX_GROUP


def dequant_1x128(q, s) -> np.ndarray:
    """q[R][K] uint8, s[R][K/128] -> fp64 [R][K]; element (r, k) uses s[r, k // 128]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    return decode_e4m3(q) * np.repeat(s, GROUP, axis=1)


def dequant_128x128(q, s) -> np.ndarray:
    """q[N][K] uint8, s[N/128][K/128] -> fp64 [N][K]; element (n, k) uses s[n // 128, k // 128]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    return decode_e4m3(q) * np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)


def dequant_mx(q, e8m0) -> np.ndarray:
    """q[R][K] uint8, e8m0[R][K/32] -> fp64 [R][K]; element (r, k) uses 2**(e8m0[r, k // 32] - 127)."""
    q = np.asarray(q, dtype=np.uint8)
    return decode_e4m3(q) * np.repeat(decode_e8m0(e8m0), MX_GROUP, axis=1)


def gemm_fwd(xq, sx, wq, sw) -> np.ndarray:
    """Y[M][N] = deq(X) . deq(W)^T  (fp64)."""
    return dequant_1x128(xq, sx) @ dequant_128x128(wq, sw).T


def gemm_dgrad(dyq, sdy, wq, sw) -> np.ndarray:
    """dX[M][K] = deq(dY) . deq(W) with dY[M][N] in 1x128 groups along N and
    W[N][K] in 128x128 blocks (fp64)."""
    return dequant_1x128(dyq, sdy) @ dequant_128x128(wq, sw)


def gemm_wgrad(dyqt, sdyt, xqt, sxt) -> np.ndarray:
    """dW[N][K] = deq(dY)^T . deq(X), from the column-wise copies
    dYt[N][M] (st [N][M/128]) and Xt[K][M] (st [K][M/128]) (fp64)."""
    return dequant_1x128(dyqt, sdyt) @ dequant_1x128(xqt, sxt).T


def gemm_mx_fwd(xq, ex, wq, ew) -> np.ndarray:
    """Y[M][N] = deq(X) . deq(W)^T with 1x32 E8M0 groups along K on both (fp64)."""
    return dequant_mx(xq, ex) @ dequant_mx(wq, ew).T


def gemm_mx_dgrad(dyq, edy, wqt, ewt) -> np.ndarray:
    """dX[M][K] = deq(dY) . deq(W), dY[M][N] with 1x32 groups along N and W given as its
    32x1-quantized transposed copy Wt[K][N] (1x32 groups along N) (fp64)."""
    return dequant_mx(dyq, edy) @ dequant_mx(wqt, ewt).T


def gemm_mx_wgrad(dyqt, edyt, xqt, ext) -> np.ndarray:
    """dW[N][K] = deq(dY)^T . deq(X) from the 32x1 (token-group) copies dYt[N][M] and
    Xt[K][M] (fp64)."""
    return dequant_mx(dyqt, edyt) @ dequant_mx(xqt, ext).T


def _expert_rows(offsets, E, T):
    """Row ranges [lo, hi) of the E experts; offsets must run from 0 to T, non-decreasing."""
    offsets = np.asarray(offsets, dtype=np.int64)
    if offsets.shape != (E + 1,) or offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be non-decreasing from 0 to T with E+1 entries")
    return [(int(offsets[e]), int(offsets[e + 1])) for e in range(E)]


def grouped_gemm_mx(xq, ex, wq, ew, offsets) -> np.ndarray:
    """MXFP8 grouped GEMM.

    xq[T][K], ex[T][K/32]: routed rows, grouped by expert;
    wq[E][N][K], ew[E][N][K/32]: per-expert weights;
    offsets[E+1]: rows of expert e are offsets[e] .. offsets[e+1]-1.
    Returns Y[T][N] (fp64).
    """
    wq = np.asarray(wq)
    E, N, _ = wq.shape
    T = np.asarray(xq).shape[0]
    y = np.zeros((T, N), dtype=np.float64)
    for e, (lo, hi) in enumerate(_expert_rows(offsets, E, T)):
        if hi > lo:
            y[lo:hi] = dequant_mx(xq[lo:hi], ex[lo:hi]) @ dequant_mx(wq[e], ew[e]).T
    return y


def grouped_gemm_block(xq, sx, wq, sw, offsets) -> np.ndarray:
    """Blockwise grouped GEMM.

    xq[T][K], sx[T][K/128]: routed rows in 1x128 groups, grouped by expert;
    wq[E][N][K], sw[E][N/128][K/128]: per-expert weights in 128x128 blocks;
    offsets[E+1]: rows of expert e are offsets[e] .. offsets[e+1]-1.
    Returns Y[T][N] (fp64).
    """
    wq = np.asarray(wq)
    E, N, _ = wq.shape
    T = np.asarray(xq).shape[0]
    y = np.zeros((T, N), dtype=np.float64)
    for e, (lo, hi) in enumerate(_expert_rows(offsets, E, T)):
        if hi > lo:
            y[lo:hi] = dequant_1x128(xq[lo:hi], sx[lo:hi]) @ dequant_128x128(wq[e], sw[e]).T
    return y
