"""Weight sync: the zero-requantization install, and the naive control path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[SkyRL-FP8] "On-Policy FP8 weight sync" and Fig. 3: the rollout side installs
the trainer's FP8 payload together with its block scales, with no quantizer of
its own, so trainer and rollout weights are bit-identical. The install is
therefore the identity on bytes.

[SkyRL-FP8] "When independent quantization breaks policy consistency" and
Fig. 2: the old bridge dequantizes to BF16, drops the trainer's scales, and the
rollout engine requantizes the BF16 values with its own (per-tensor) recipe.
Reading taken for that control path: dequantize in fp32 (fl32(dec(q) * s)),
round to bf16, then per-tensor quantization s_t = fl32(amax / 448),
q' = E4M3(fl32(w' / s_t)) ([AIS] notes per-tensor dynamic scaling for FP8
rollout). The mismatch is measured as the mean relative error
sum|w_rollout - w_trainer| / sum|w_trainer| over the tensor (the page gives a
number, 0.038 on a 4B model, but no formula; this one is defined at w = 0).

Pinned by tests/test_oracle_weight_sync.py: a block-uniform power-of-two-scale
weight survives the naive path unchanged (closed form), a hand-computed
relative error on a tiny tensor, and a nonzero error on generic weights.
"""

from __future__ import annotations

import numpy as np

from .fp8_formats import E4M3_MAX, decode_e4m3, encode_e4m3, round_to_bf16
from .gemm import dequant_128x128


def install(q, s):
    """Install = verbatim copy of payload and scales (no quantizer)."""
    return np.array(q, dtype=np.uint8, copy=True), np.array(s, copy=True)


def dequant_to_bf16(q, s):
    """First step of the naive path: the 128x128-block weight dequantized in fp32
    (fl32(dec(q) * s)) and rounded to bf16 (float32 array of bf16 values). Elementwise, so
    any split into 128-row blocks gives the same values."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    s_full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)
    w32 = decode_e4m3(q).astype(np.float32) * s_full           # fp32 product, IEEE rounding
    return round_to_bf16(w32)


def per_tensor_scale(amax) -> np.float32:
    """The rollout recipe's per-tensor scale fl32(amax / 448) of the bf16 tensor (1 if all zero)."""
    amax = np.float32(amax)
    return np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))


def requant_per_tensor(wb, s_t):
    """Last step of the naive path: E4M3(fl32(w' / s_t)), elementwise."""
    return encode_e4m3(np.asarray(wb, dtype=np.float32) / np.float32(s_t))


def naive_resync(q, s):
    """Dequantize a 128x128-block weight to bf16 and requantize it per tensor.

    Returns (q' uint8 [N][K], s_t float32 scalar).
    """
    wb = dequant_to_bf16(q, s)
    amax = np.float32(np.max(np.abs(wb))) if wb.size else np.float32(0)
    s_t = per_tensor_scale(amax)
    return requant_per_tensor(wb, s_t), s_t


def mean_relative_error(w_ref, w_other) -> float:
    """sum |w_other - w_ref| / sum |w_ref| in fp64."""
    w_ref = np.asarray(w_ref, dtype=np.float64)
    w_other = np.asarray(w_other, dtype=np.float64)
    den = np.sum(np.abs(w_ref))
    return float(np.sum(np.abs(w_other - w_ref)) / den) if den else 0.0


def weight_value_block(q, s):
    """Dequantized value (fp64) of a 128x128-block weight."""
    return dequant_128x128(q, s)


def weight_value_tensor(q, s_t):
    """Dequantized value (fp64) of a per-tensor-scaled weight."""
    return decode_e4m3(q) * np.float64(np.float32(s_t))
