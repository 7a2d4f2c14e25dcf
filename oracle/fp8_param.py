"""fp8_param: FP8 parameter storage requantized from an FP32 master after every optimizer step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[SkyRL-FP8] "Deep dive: FP8 quantization with FP32 and power-of-two block scales": with
fp8_param the optimizer updates the FP32 master copy and the FP8 parameter storage is
recomputed from it after each step, Q(W_t), with fp32 block scales or fp32 scales restricted
to powers of two. The page's ablation (Fig. 12) measures the cumulative FP8 storage
displacement over many RL-sized steps, normalised by the FP32 master displacement (close to
1 for both scale formats), and the cosine between one master update and the FP8 storage
change it causes, against the update size. It quotes per-element updates up to
|dW| = 1.01e-6 and a mean relative update |dW|/|W| of 0.6-0.9e-4 per step.

Readings:
* Q is the 128x128-block weight quantizer applied to the fp32 master directly:
  s = fl32(amax / 448) (or the power-of-two rule of the blockwise recipe), and
  q = E4M3(fl32(w / s)) with an IEEE fp32 division (w has 24 significant bits here; the
  power-of-two case is the exact scaling). Q(W_t) comes with its byte transpose, the DGrad
  operand.
* Tiny blocks. An fp32 amax below about 224 * 2^-149 makes fl32(amax / 448) round to zero;
  such a scale is raised to the smallest positive fp32 value, 2^-149, so the quotient stays
  finite. A block whose amax sits a little above that gets a subnormal scale with only a few
  significant bits, and fl32(w / s) can then exceed 448 (up to 512); the encoder saturates
  it to +-448 like any other value beyond the E4M3 range. bf16 inputs never reach either
  case: their smallest amax gives a scale with at least 7 significant bits.
* Displacement after T steps: ||deq Q(W_T) - deq Q(W_0)|| / ||W_T - W_0||, in the L2 and the
  L1 norm (fp64). Cosine: <dW, deq Q(W + dW) - deq Q(W)> / (||dW|| ||..||).
* Synthetic trajectory (no model or optimizer is available): W_0 ~ N(0, 0.02) fp32 and
  Adam-like steps dW_t = lr * sign(b + z_t), lr = 1e-6, with a fixed per-element bias
  b ~ N(0, 1) and noise z_t drawn from a fixed bank of N(0, 1) matrices used in turn (the
  bank makes the trajectory reproducible on the GPU without sending fresh noise each step).
  Each step is one fp32 addition W_{t+1} = fl32(W_t + dW_t).

Pinned by tests/test_oracle_fp8_param.py: a pure-Python brute force of the fp32-input
quantizer on small blocks (exact fractions, nearest-in-table encoding; both scale formats),
blocks whose amax gives an underflowed or few-bit subnormal scale (same brute force), the
closed form of an update that moves every element by a whole number of quantization
steps (displacement ratio exactly 1, cosine exactly 1), invariance of both metrics under a
common power-of-two scaling, hand-computed sign steps (sign(0) = 0, fp32 sum before the
sign), and the closed form of a trajectory whose every step adds exactly lr.
"""

from __future__ import annotations

import numpy as np

from .fp8_formats import E4M3_MAX, decode_e4m3, encode_e4m3
from .quantize import GROUP, mx_exponent


_F32_MIN_POSITIVE = np.float32(2.0 ** -149)


def _as_f32_finite(w) -> np.ndarray:
    w = np.asarray(w, dtype=np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("fp32 master weights must be finite")
    return w


def quant_w_128x128_f32(w, pow2: bool = False):
    """128x128-block quantization of an fp32 matrix W[N][K] (N, K % 128 == 0).

    Returns (q uint8 [N][K], s float32 [N/128][K/128])."""
    w = _as_f32_finite(w)
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("N and K must be multiples of 128")
    b = w.reshape(N // GROUP, GROUP, K // GROUP, GROUP)
    amax = np.max(np.abs(b), axis=(1, 3)).astype(np.float32)
    if pow2:
        e = mx_exponent(amax)
        s = np.ldexp(np.float64(1.0), e).astype(np.float32)
        v = np.ldexp(b.astype(np.float64), -e[:, None, :, None]).astype(np.float32)   # exact, or the fp32 rounding
    else:
        s = np.where(amax == 0, np.float32(1.0), (amax / np.float32(E4M3_MAX)).astype(np.float32))
        s = np.where(s == 0, _F32_MIN_POSITIVE, s).astype(np.float32)                    # underflowed scale
        v = (b / s[:, None, :, None]).astype(np.float32)                                 # IEEE fp32 division
    return encode_e4m3(v).reshape(N, K), s.astype(np.float32)


def dequant(q, s) -> np.ndarray:
    """deq(Q) in fp64 for a 128x128-block quantized weight."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    return decode_e4m3(q) * np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)


def displacement_ratios(w0, w1, d0, d1):
    """(L2, L1) of ||d1 - d0|| / ||w1 - w0||: FP8 storage displacement over master displacement."""
    dm = np.asarray(w1, np.float64) - np.asarray(w0, np.float64)
    dq = np.asarray(d1, np.float64) - np.asarray(d0, np.float64)
    return float(np.linalg.norm(dq) / np.linalg.norm(dm)), float(np.abs(dq).sum() / np.abs(dm).sum())


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).reshape(-1)
    b = np.asarray(b, np.float64).reshape(-1)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    return 0.0 if na == 0 or nb == 0 else float(a @ b / (na * nb))


def sign_step(bias, z, lr) -> np.ndarray:
    """dW = lr * sign(b + z) in fp32 (sign(0) = 0)."""
    return (np.float32(lr) * np.sign((np.asarray(bias, np.float32) + np.asarray(z, np.float32)).astype(np.float32))
            ).astype(np.float32)


def trajectory(w0, bias, bank, lr, steps, checkpoints, pow2: bool = False):
    """Run the synthetic fp8_param trajectory: W_{t+1} = fl32(W_t + lr sign(b + bank[t % len])),
    requantizing Q(W_t) at each checkpoint t. Returns {t: (W_t, q_t, s_t)} for t in
    checkpoints (t = 0 included)."""
    w = np.array(w0, dtype=np.float32, copy=True)
    out = {0: (w.copy(),) + quant_w_128x128_f32(w, pow2)}
    cps = set(checkpoints)
    for t in range(1, steps + 1):
        w = (w + sign_step(bias, bank[(t - 1) % len(bank)], lr)).astype(np.float32)
        if t in cps:
            out[t] = (w.copy(),) + quant_w_128x128_f32(w, pow2)
    return out
