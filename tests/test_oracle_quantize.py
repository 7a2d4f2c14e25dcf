"""Pins for the oracle's quantizers: a pure-Python brute force (exact fractions,
nearest-in-table encoding) on small inputs, and invariants fixed by the method:
amax element -> +-448, power-of-two scale equivariance, the half-ulp error bound,
group locality per recipe, and the MX scale rule's range invariant."""

import bisect
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quantize as Q
from oracle.fp8_formats import decode_e4m3
from workloads import bf16_round

# positive finite E4M3 values from torch's decoder (a library routine, not the oracle)
_TABLE = torch.from_numpy(np.arange(0, 0x7F, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
_TABLE_FR = [Fraction(float(t)) for t in _TABLE]


def _enc_fraction(v: Fraction, negative: bool) -> int:
    """Nearest entry of the (ascending) positive E4M3 table, ties to the even code."""
    a = min(abs(v), Fraction(448))
    hi = bisect.bisect_left(_TABLE_FR, a)
    if hi < len(_TABLE_FR) and _TABLE_FR[hi] == a:
        c = hi
    else:
        lo = hi - 1
        dlo, dhi = a - _TABLE_FR[lo], _TABLE_FR[hi] - a
        c = lo if dlo < dhi else hi if dhi < dlo else (lo if lo % 2 == 0 else hi)
    return c | (0x80 if negative else 0)


def _fl32(fr: Fraction) -> Fraction:
    """Round an exact rational to fp32 (via fp64 first: innocuous for a quotient of
    two fp32 numbers, since 53 >= 2*24 + 2)."""
    return Fraction(float(np.float32(float(fr))))


def _brute_group(vals):
    """One group, by hand: amax, s = fl32(amax/448), q = enc(fl32(x/s))."""
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fr)
    s = Fraction(1) if amax == 0 else _fl32(amax / 448)
    codes = [_enc_fraction(_fl32(v / s), np.signbit(np.float32(float(v0)))) for v, v0 in zip(fr, vals)]
    return codes, float(s)


def _sample(shape, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    return bf16_round(rng.standard_normal(shape).astype(np.float32) * np.float32(sigma))


def test_1x128_brute_force():
    x = _sample((3, 384), 10)
    x[1, 5] = 300.0                      # an outlier in one group
    x[2, 128:256] = 0.0                  # an all-zero group
    x[2, 130] = -0.0
    q, s = Q.quant_act_1x128(x)
    assert q.shape == (3, 384) and s.shape == (3, 3) and q.dtype == np.uint8 and s.dtype == np.float32
    for r in range(3):
        for g in range(3):
            codes, sc = _brute_group(x[r, g * 128:(g + 1) * 128])
            assert list(q[r, g * 128:(g + 1) * 128]) == codes
            assert s[r, g] == np.float32(sc)
    assert s[2, 1] == 1.0 and q[2, 130] == 0x80


def test_128x128_brute_force():
    w = _sample((256, 256), 11, 0.02)
    w[3, 200] = 1.5
    q, s = Q.quant_w_128x128(w)
    assert s.shape == (2, 2)
    for bi in range(2):
        for bj in range(2):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            codes, sc = _brute_group(blk.reshape(-1))
            assert s[bi, bj] == np.float32(sc)
            assert list(q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128].reshape(-1)) == codes


def test_128x1_brute_force_and_layout():
    x = _sample((256, 128), 12)
    qt, st = Q.quant_act_128x1(x)
    assert qt.shape == (128, 256) and st.shape == (128, 2)
    for k in (0, 77, 127):
        for mb in range(2):
            codes, sc = _brute_group(x[mb * 128:(mb + 1) * 128, k])
            assert list(qt[k, mb * 128:(mb + 1) * 128]) == codes and st[k, mb] == np.float32(sc)


def _brute_mx_exponent(amax: float) -> int:
    if amax == 0:
        return 0
    e = -200
    while not (Fraction(amax) <= 448 * Fraction(2) ** e):
        e += 1
    return max(-127, min(127, e))


def test_mx_brute_force():
    x = _sample((4, 96), 13)
    x[0, 0:32] = 0
    x[1, 40] = 448.0 * 4                   # amax exactly 448 * 2**2 -> e = 2
    x[2, 70] = 1800.0                      # next bf16 above 448 * 2**2 -> e = 3
    q, e8 = Q.quant_mx_1x32(x)
    assert e8.shape == (4, 3)
    for r in range(4):
        for g in range(3):
            vals = x[r, g * 32:(g + 1) * 32]
            e = _brute_mx_exponent(float(np.max(np.abs(vals))))
            assert int(e8[r, g]) == e + 127
            for i, v in enumerate(vals):
                c = _enc_fraction(Fraction(float(v)) / Fraction(2) ** e, np.signbit(v))
                assert q[r, g * 32 + i] == c
    assert e8[1, 1] == 127 + 2 and e8[2, 2] == 127 + 3 and e8[0, 0] == 127


@pytest.mark.parametrize("fn,shape,groups", [
    ("act", (256, 512), lambda i, j: (i, j // 128)),
    ("w", (256, 512), lambda i, j: (i // 128, j // 128)),
    ("col", (256, 512), lambda i, j: (j, i // 128)),
    ("mx", (256, 512), lambda i, j: (i, j // 32)),
])
def test_group_locality(fn, shape, groups):
    """Changing one element changes only the scale of its own group and only codes
    inside that group: catches grouping along the wrong axis or a wrong block size."""
    run = {"act": Q.quant_act_1x128, "w": Q.quant_w_128x128, "col": Q.quant_act_128x1, "mx": Q.quant_mx_1x32}[fn]
    x = _sample(shape, 14)
    q0, s0 = run(x)
    i, j = 131, 300
    x2 = x.copy()
    x2[i, j] = 1000.0
    q1, s1 = run(x2)
    diff_s = np.argwhere(s0 != s1)
    assert [tuple(d) for d in diff_s] == [groups(i, j)]
    changed = np.argwhere(q0 != q1)
    if fn == "col":
        changed = changed[:, ::-1]               # qt is [K][M]
    assert len(changed) > 1
    assert all(groups(a, b) == groups(i, j) for a, b in changed)


@pytest.mark.parametrize("fn", ["act", "w", "col"])
def test_amax_element_encodes_to_448(fn):
    run = {"act": Q.quant_act_1x128, "w": Q.quant_w_128x128, "col": Q.quant_act_128x1}[fn]
    x = _sample((256, 256), 15, 0.3)
    q, s = run(x)
    xs = x.T if fn == "col" else x
    bs = (128, 128) if fn == "w" else (1, 128)
    R, C = xs.shape
    for r0 in range(0, R, bs[0]):
        for c0 in range(0, C, bs[1]):
            blk = xs[r0:r0 + bs[0], c0:c0 + bs[1]]
            qb = q[r0:r0 + bs[0], c0:c0 + bs[1]]
            at = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert qb[at] == (0xFE if blk[at] < 0 else 0x7E)
            assert np.all((qb & 0x7F) <= 0x7E)


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 30])
def test_power_of_two_equivariance(j):
    x = _sample((4, 512), 16)
    q0, s0 = Q.quant_act_1x128(x)
    q1, s1 = Q.quant_act_1x128(x * np.float32(2.0 ** j))
    assert np.array_equal(q0, q1) and np.array_equal(s1, s0 * np.float32(2.0 ** j))
    w = _sample((256, 256), 17, 0.02)
    q0, s0 = Q.quant_w_128x128(w)
    q1, s1 = Q.quant_w_128x128(w * np.float32(2.0 ** j))
    assert np.array_equal(q0, q1) and np.array_equal(s1, s0 * np.float32(2.0 ** j))
    q0, e0 = Q.quant_mx_1x32(x)
    q1, e1 = Q.quant_mx_1x32(x * np.float32(2.0 ** j))
    assert np.array_equal(q0, q1) and np.array_equal(e1.astype(int), e0.astype(int) + j)


def _ulp_e4m3(a):
    a = np.maximum(np.abs(a), 2.0 ** -6)
    return np.ldexp(1.0, np.frexp(a)[1] - 1 - 3)


def test_half_ulp_error_bound():
    x = _sample((64, 1024), 18)
    q, s = Q.quant_act_1x128(x)
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    y = x.astype(np.float64) / sf
    err = np.abs(decode_e4m3(q) * sf - x)
    # fp32 quotient adds at most 2**-24 relative before the E4M3 rounding
    bound = (0.5 * _ulp_e4m3(y) + np.abs(y) * 2.0 ** -23) * sf
    assert np.all(err <= bound)


def test_mx_range_invariant_and_no_saturation():
    x = _sample((128, 1024), 19, 3.0)
    x[5, :32] *= np.float32(2.0 ** 40)
    x[6, :32] *= np.float32(2.0 ** -40)
    q, e8 = Q.quant_mx_1x32(x)
    e = e8.astype(np.int64) - 127
    amax = np.max(np.abs(x.reshape(128, 32, 32)), axis=2).astype(np.float64)
    r = amax * np.ldexp(1.0, -e)
    assert np.all((r > 224) & (r <= 448))
    scaled = x.reshape(128, 32, 32).astype(np.float64) * np.ldexp(1.0, -e)[:, :, None]
    assert np.all(np.abs(scaled) <= 448)
    dq = decode_e4m3(q).reshape(128, 32, 32)
    assert np.all(np.abs(dq - scaled) <= 0.5 * _ulp_e4m3(scaled) + 0)


def test_shape_checks():
    with pytest.raises(ValueError):
        Q.quant_act_1x128(np.zeros((2, 100), np.float32))
    with pytest.raises(ValueError):
        Q.quant_act_128x1(np.zeros((100, 128), np.float32))
    with pytest.raises(ValueError):
        Q.quant_w_128x128(np.zeros((128, 100), np.float32))
    with pytest.raises(ValueError):
        Q.quant_mx_1x32(np.zeros((2, 40), np.float32))
    q, s = Q.quant_act_1x128(np.zeros((0, 256), np.float32))
    assert q.shape == (0, 256) and s.shape == (0, 2)


# ------------------------------------------------------------------------------------------
# power-of-two block scales (1x128 / 128x1 / 128x128 groups with exponent-only scales)
# ------------------------------------------------------------------------------------------

def _brute_pow2_group(vals):
    """One group by hand: e = smallest integer with amax <= 448 * 2**e (clamped to
    [-127, 127], 0 for an all-zero group), q = nearest-even E4M3 of x * 2**-e (exact)."""
    amax = max(abs(float(v)) for v in vals)
    e = _brute_mx_exponent(amax)
    codes = [_enc_fraction(Fraction(float(v)) / Fraction(2) ** e, bool(np.signbit(v))) for v in vals]
    return codes, e


def test_pow2_1x128_brute_force():
    x = _sample((4, 384), 20)
    x[0, 0:128] = 0.0                         # all-zero group -> e = 0
    x[1, 130] = 448.0 * 2.0 ** -3             # amax exactly 448 * 2**-3 -> e = -3
    x[2, 300] = 1792.0 + 8.0                  # just above 448 * 2**2 -> e = 3
    x[3, 5] = 9.2e-41                         # a subnormal among normal values
    x = bf16_round(x)                         # (the planted values above are bf16-exact)
    q, s = Q.quant_act_1x128_pow2(x)
    assert q.shape == (4, 384) and s.shape == (4, 3) and s.dtype == np.float32
    for r in range(4):
        for g in range(3):
            vals = x[r, g * 128:(g + 1) * 128]
            codes, e = _brute_pow2_group(vals)
            assert list(q[r, g * 128:(g + 1) * 128]) == codes
            assert Fraction(float(s[r, g])) == Fraction(2) ** e
    assert s[0, 0] == 1.0 and s[1, 1] == np.float32(2.0 ** -3)


def test_pow2_128x128_and_128x1_brute_force():
    w = _sample((256, 256), 21, 0.02)
    w[7, 140] = -0.75
    q, s = Q.quant_w_128x128_pow2(w)
    assert s.shape == (2, 2)
    for bi in range(2):
        for bj in range(2):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128].reshape(-1)
            codes, e = _brute_pow2_group(blk)
            assert Fraction(float(s[bi, bj])) == Fraction(2) ** e
            assert list(q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128].reshape(-1)) == codes
    x = _sample((256, 128), 22)
    qt, st = Q.quant_act_128x1_pow2(x)
    assert qt.shape == (128, 256) and st.shape == (128, 2)
    for k in (0, 63, 127):
        for mb in range(2):
            codes, e = _brute_pow2_group(x[mb * 128:(mb + 1) * 128, k])
            assert list(qt[k, mb * 128:(mb + 1) * 128]) == codes
            assert Fraction(float(st[k, mb])) == Fraction(2) ** e


@pytest.mark.parametrize("fn", ["act", "w"])
def test_pow2_range_invariant_and_fp32_bracket(fn):
    """Every nonzero group in range: 224 < amax / s <= 448 (the amax element's code lies in
    (224, 448], nothing saturates), and the FP32 recipe's scale s32 = fl32(amax / 448)
    satisfies s32 <= s < 2 * s32."""
    x = _sample((256, 512), 23, 3.0)
    x[:, 7] *= np.float32(200.0)
    x = bf16_round(x)
    if fn == "act":
        q, s = Q.quant_act_1x128_pow2(x)
        _, s32 = Q.quant_act_1x128(x)
        amax = np.max(np.abs(x.reshape(256, 4, 128)), axis=2)
    else:
        q, s = Q.quant_w_128x128_pow2(x)
        _, s32 = Q.quant_w_128x128(x)
        amax = np.max(np.abs(x.reshape(2, 128, 4, 128)), axis=(1, 3))
    ratio = amax.astype(np.float64) / s.astype(np.float64)
    assert np.all(ratio > 224) and np.all(ratio <= 448)
    assert np.all(s32 <= s) and np.all(s < 2 * s32.astype(np.float64))
    assert not np.any((q & 0x7F) == 0x7F)                     # no NaN codes


@pytest.mark.parametrize("j", [-20, -1, 1, 9])
def test_pow2_equivariance(j):
    x = _sample((128, 256), 24)
    q1, s1 = Q.quant_act_1x128_pow2(x)
    q2, s2 = Q.quant_act_1x128_pow2(bf16_round(x * np.float32(2.0 ** j)))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0 ** j)


def test_mx_32x1_brute_force_and_layout():
    x = _sample((96, 64), 14)
    x[0:32, 3] = 0.0                        # an all-zero column group
    x[40, 7] = 448.0 * 8                    # amax exactly 448 * 2**3
    x[70, 9] = -1e-39                       # a subnormal bf16 value (after rounding)
    x = bf16_round(x)
    qt, et = Q.quant_mx_32x1(x)
    assert qt.shape == (64, 96) and et.shape == (64, 3)
    for k in (0, 3, 7, 9, 63):
        for rg in range(3):
            vals = x[rg * 32:(rg + 1) * 32, k]
            e = _brute_mx_exponent(float(np.max(np.abs(vals))))
            assert int(et[k, rg]) == e + 127
            for i, v in enumerate(vals):
                assert qt[k, rg * 32 + i] == _enc_fraction(Fraction(float(v)) / Fraction(2) ** e, np.signbit(v))
    assert et[3, 0] == 127 and et[7, 1] == 127 + 3
    with pytest.raises(ValueError):
        Q.quant_mx_32x1(x[:40])


def test_transpose_payload_layout():
    """qt[j][i] == q[i][j] for every index of a non-square payload of distinct bytes; the
    result is a new C-contiguous uint8 array (the DGrad operand is read row by row)."""
    q = (np.arange(3 * 80, dtype=np.int64) % 251).astype(np.uint8).reshape(3, 80)
    qt = Q.transpose_payload(q)
    assert qt.shape == (80, 3) and qt.dtype == np.uint8 and qt.flags["C_CONTIGUOUS"]
    for i in range(3):
        for j in range(80):
            assert qt[j, i] == (i * 80 + j) % 251
    assert qt.ctypes.data != q.ctypes.data
    # 128x128 blocks map onto 128x128 blocks: block (bi, bj) of q is block (bj, bi) of qt
    w = (np.arange(256 * 384, dtype=np.int64) % 253).astype(np.uint8).reshape(256, 384)
    wt = Q.transpose_payload(w)
    for bi in range(2):
        for bj in range(3):
            blk = w[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)]
            assert np.array_equal(wt[128 * bj:128 * (bj + 1), 128 * bi:128 * (bi + 1)], blk.T)
