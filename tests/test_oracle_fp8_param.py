"""Pins of oracle/fp8_param.py: the fp32-input 128x128 quantizer against a pure-Python brute
force (exact fractions, nearest-in-table encoding), and the displacement metrics against
closed forms."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8_param as P
from oracle.fp8_formats import decode_e4m3
from test_oracle_quantize import _brute_mx_exponent, _enc_fraction, _fl32


def _brute_block_f32(vals, pow2):
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fr)
    if pow2:
        e = _brute_mx_exponent(float(amax))
        s = Fraction(2) ** e
        codes = [_enc_fraction(_fl32(v / s), np.signbit(np.float32(v0))) for v, v0 in zip(fr, vals)]
    else:
        s = Fraction(1) if amax == 0 else _fl32(amax / 448)
        if s == 0:
            s = Fraction(1, 2 ** 149)          # a scale that underflowed: the smallest positive fp32
        codes = [_enc_fraction(_fl32(v / s), np.signbit(np.float32(v0))) for v, v0 in zip(fr, vals)]
    return codes, float(s)


@pytest.mark.parametrize("pow2", [False, True])
def test_f32_quantizer_brute_force(pow2):
    rng = np.random.default_rng(50)
    w = (rng.standard_normal((256, 128)) * 0.02).astype(np.float32)     # full 24-bit significands
    w[3, 5] = np.float32(0.3)
    w[130, 7] = np.float32(-1.2345678e-3)
    w[200:256, :] = 0.0
    w[200:256, 0] = np.float32(3e-39)                                   # fp32 subnormal in a tiny block
    q, s = P.quant_w_128x128_f32(w, pow2)
    assert q.shape == (256, 128) and s.shape == (2, 1)
    for bi in range(2):
        blk = w[bi * 128:(bi + 1) * 128, :]
        codes, sc = _brute_block_f32(blk.reshape(-1), pow2)
        assert s[bi, 0] == np.float32(sc)
        assert list(q[bi * 128:(bi + 1) * 128].reshape(-1)) == codes


def test_f32_quantizer_tiny_blocks():
    """Blocks whose amax lies deep in the fp32 subnormal range: fl32(amax / 448) is zero (the
    scale becomes 2^-149) or a subnormal with one or two significant bits (quotients above
    448 saturate). The brute force applies the same reading with exact fractions; the
    hand-computed cases fix it independently of the brute force."""
    tiny = [2.0 ** -140, 2.0 ** -148, 2.0 ** -149, 300 * 2.0 ** -149, 223 * 2.0 ** -149, 225 * 2.0 ** -149]
    w = np.zeros((128, 128 * len(tiny)), np.float32)
    for b, a in enumerate(tiny):
        w[0, 128 * b] = np.float32(a)
        w[5, 128 * b + 3] = -np.float32(a)
        w[9, 128 * b + 7] = np.float32(a) * np.float32(0.5) if a >= 2.0 ** -148 else 0.0
    for pow2 in (False, True):
        q, s = P.quant_w_128x128_f32(w, pow2)
        for b in range(len(tiny)):
            blk = w[:, 128 * b:128 * (b + 1)]
            codes, sc = _brute_block_f32(blk.reshape(-1), pow2)
            assert s[0, b] == np.float32(sc), (b, pow2)
            assert list(q[:, 128 * b:128 * (b + 1)].reshape(-1)) == codes, (b, pow2)
        assert not np.any((q & 0x7F) == 0x7F)                    # never a NaN code
    q, s = P.quant_w_128x128_f32(w)
    two149 = np.float32(2.0 ** -149)
    # 2^-140 / 448 = 1.14 * 2^-149 rounds to 2^-149: the quotient 512 saturates to 448, the
    # half-size element's 256 is exact (0x78)
    assert s[0, 0] == two149 and q[0, 0] == 0x7E and q[5, 3] == 0xFE and q[9, 7] == 0x78
    # 2^-148 / 448 and 2^-149 / 448 round to zero: s = 2^-149, quotients 2 and 1
    assert s[0, 1] == two149 and q[0, 128] == 0x40 and q[9, 135] == 0x38     # E4M3(2) = 0x40, E4M3(1) = 0x38
    assert s[0, 2] == two149 and q[0, 256] == 0x38 and q[5, 259] == 0xB8
    # 300 * 2^-149 / 448 = 0.67 * 2^-149 rounds to 2^-149 (quotient 300 -> 288 = 0x79); 223 * 2^-149
    # gives 0.498 * 2^-149 -> 0 -> 2^-149 (quotient 223 -> 224 = 0x76); 225 * 2^-149 gives 0.502 * 2^-149
    # -> 2^-149 (quotient 225 -> 224)
    assert s[0, 3] == two149 and q[0, 384] == 0x79
    assert s[0, 4] == two149 and q[0, 512] == 0x76
    assert s[0, 5] == two149 and q[0, 640] == 0x76


def test_sign_step_hand_values():
    """dW = fl32(lr) * sign(fl32(b + z)): the sign of the fp32 sum, 0 where the sum is zero."""
    bias = np.array([1.0, -1.0, 0.0, 0.5, -0.25, 1.0, 1.0, -0.0, 3.0], np.float32)
    z = np.array([0.0, 0.0, 0.0, -0.5, 0.25, -1.0 + 2.0 ** -23, -1.0 + 2.0 ** -30, 0.0, -2.5], np.float32)
    # sums: 1, -1, 0, 0, 0, 2^-23 (exact), 0 (z rounds to -1 in fp32), -0, 0.5
    lr = np.float32(1e-6)
    expect = np.array([lr, -lr, 0, 0, 0, lr, 0, 0, lr], np.float32)
    d = P.sign_step(bias, z, 1e-6)
    assert d.dtype == np.float32 and np.array_equal(d, expect)
    assert float(d[0]) == float(np.float32(1e-6)) and float(np.float32(1e-6)) != 1e-6     # lr is the fp32 value
    d2 = P.sign_step(bias[:2], z[:2], 2.0 ** -20)
    assert d2.tolist() == [2.0 ** -20, -(2.0 ** -20)]


def test_trajectory_closed_form():
    """With a bias that dominates the noise every step adds exactly +lr (or -lr): W_0 and lr
    powers of two keep every fp32 sum exact, so W_T = W_0 + T * lr * sign(b) in closed form,
    and the checkpoints carry the quantization of exactly that matrix."""
    rng = np.random.default_rng(53)
    w0 = np.full((128, 128), 0.5, np.float32)
    w0[:, ::2] = -0.25
    bias = np.where(rng.standard_normal(w0.shape) > 0, np.float32(4.0), np.float32(-4.0)).astype(np.float32)
    bank = [np.clip(rng.standard_normal(w0.shape), -1, 1).astype(np.float32) for _ in range(3)]
    lr = 2.0 ** -12
    out = P.trajectory(w0, bias, bank, lr, 7, [3, 7])
    for t in (0, 3, 7):
        expect = (w0.astype(np.float64) + t * lr * np.sign(bias)).astype(np.float32)
        assert np.array_equal(out[t][0], expect), t
        q, s = P.quant_w_128x128_f32(expect)
        assert np.array_equal(out[t][1], q) and np.array_equal(out[t][2], s)


def test_f32_quantizer_rejects_bad_input():
    with pytest.raises(ValueError):
        P.quant_w_128x128_f32(np.full((128, 128), np.inf, np.float32))
    with pytest.raises(ValueError):
        P.quant_w_128x128_f32(np.zeros((100, 128), np.float32))


def test_displacement_closed_form():
    """A block whose values are exact E4M3 codes times a power-of-two scale, moved by whole
    code steps that keep the block amax: Q is exact at both ends, so the storage displacement
    equals the master displacement (ratios 1, cosine 1)."""
    codes = np.arange(0x20, 0x60, dtype=np.uint8)                  # positive codes, values 2^-3 .. 2^1.875
    grid = decode_e4m3(codes)
    w0 = np.zeros((128, 128), np.float32)
    w0[0, :64] = grid[:64] * 2.0 ** -8
    w0[1, 0] = 448.0 * 2.0 ** -8                                   # fixes amax = 448 * 2^-8 -> s = 2^-8
    w1 = w0.copy()
    w1[0, 1:63] = grid[2:64] * 2.0 ** -8                           # every value up by one code step
    for pow2 in (False, True):
        q0, s0 = P.quant_w_128x128_f32(w0, pow2)
        q1, s1 = P.quant_w_128x128_f32(w1, pow2)
        d0, d1 = P.dequant(q0, s0), P.dequant(q1, s1)
        assert np.array_equal(d0, w0) and np.array_equal(d1, w1)
        l2, l1 = P.displacement_ratios(w0, w1, d0, d1)
        assert l2 == 1.0 and l1 == 1.0
        assert abs(P.cosine(w1 - w0, d1 - d0) - 1.0) < 1e-15


def test_metrics_scale_invariance_and_zero_update():
    rng = np.random.default_rng(51)
    w0 = (rng.standard_normal((128, 256)) * 0.02).astype(np.float32)
    w1 = (w0 + np.float32(1e-3) * np.sign(rng.standard_normal(w0.shape)).astype(np.float32)).astype(np.float32)
    d0 = P.dequant(*P.quant_w_128x128_f32(w0))
    d1 = P.dequant(*P.quant_w_128x128_f32(w1))
    base = P.displacement_ratios(w0, w1, d0, d1)
    sc = np.float32(2.0 ** 5)
    e0 = P.dequant(*P.quant_w_128x128_f32(w0 * sc))
    e1 = P.dequant(*P.quant_w_128x128_f32(w1 * sc))
    assert P.displacement_ratios(w0 * sc, w1 * sc, e0, e1) == pytest.approx(base, rel=1e-12)
    assert P.cosine(w1 - w0, np.zeros_like(d1)) == 0.0


def test_trajectory_is_stepwise_requantization():
    rng = np.random.default_rng(52)
    w0 = (rng.standard_normal((128, 128)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(w0.shape).astype(np.float32)
    bank = [rng.standard_normal(w0.shape).astype(np.float32) for _ in range(3)]
    out = P.trajectory(w0, bias, bank, 1e-6, 5, [2, 5])
    w = w0.copy()
    for t in range(5):
        w = (w + P.sign_step(bias, bank[t % 3], 1e-6)).astype(np.float32)
        if t + 1 in (2, 5):
            assert np.array_equal(out[t + 1][0], w)
            q, s = P.quant_w_128x128_f32(w)
            assert np.array_equal(out[t + 1][1], q) and np.array_equal(out[t + 1][2], s)
