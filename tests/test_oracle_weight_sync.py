"""Pins for the oracle's weight-sync functions: install is the identity on
bytes; the naive dequantize -> bf16 -> per-tensor requantize path is exact in a
closed-form special case and lossy otherwise; the relative-error definition on
a hand-computed tensor."""

import numpy as np

from oracle import quantize as Q
from oracle.fp8_formats import decode_e4m3
from oracle import weight_sync as S
from workloads import bf16_round, normal_bf16


def test_install_is_verbatim():
    w = normal_bf16((256, 384), 0.02, 100, 0)
    q, s = Q.quant_w_128x128(w)
    q2, s2 = S.install(q, s)
    assert q2 is not q and np.array_equal(q2, q) and np.array_equal(s2.view(np.uint32), s.view(np.uint32))


def test_naive_path_exact_when_all_blocks_share_a_power_of_two_scale():
    """If every block's amax is 448 * 2**-6 the block scale is 2**-6 everywhere,
    each dequantized value (4 significant bits times a power of two) is exact in
    bf16, and the per-tensor requantization reproduces the same codes and scale."""
    rng = np.random.default_rng(101)
    codes = rng.integers(0, 0x7E, size=(256, 256), dtype=np.uint8) | (rng.integers(0, 2, (256, 256), dtype=np.uint8) << 7)
    codes[::128, ::128] = 0x7E                           # one +448 code per block
    w = (decode_e4m3(codes) * 2.0 ** -6).astype(np.float32)
    q, s = Q.quant_w_128x128(w)
    assert np.all(s == np.float32(2.0 ** -6)) and np.array_equal(q, codes)
    q2, s_t = S.naive_resync(q, s)
    assert s_t == np.float32(2.0 ** -6) and np.array_equal(q2, q)
    assert S.mean_relative_error(S.weight_value_block(q, s), S.weight_value_tensor(q2, s_t)) == 0.0


def test_naive_path_is_lossy_on_generic_weights():
    w = normal_bf16((512, 512), 0.02, 100, 1)
    q, s = Q.quant_w_128x128(w)
    q2, s_t = S.naive_resync(q, s)
    err = S.mean_relative_error(S.weight_value_block(q, s), S.weight_value_tensor(q2, s_t))
    assert 0.005 < err < 0.2
    assert not np.array_equal(q2, q)


def test_relative_error_definition_by_hand():
    ref = np.array([1.0, -2.0, 0.0, 4.0])
    other = np.array([1.5, -2.0, 0.25, 3.0])
    # (0.5 + 0 + 0.25 + 1) / (1 + 2 + 0 + 4) = 1.75 / 7
    assert S.mean_relative_error(ref, other) == 0.25
    assert S.mean_relative_error(np.zeros(3), np.ones(3)) == 0.0


def _brute_naive(q, s):
    """Exact-rational naive path: (codes, s_t) and the codes that skipping the bf16 step gives."""
    from fractions import Fraction

    from test_oracle_producers import _bf16r, _f32r
    from test_oracle_quantize import _enc_fraction

    dec = [Fraction(float(v)) for v in decode_e4m3(np.arange(0x7F, dtype=np.uint8))]
    n, k = q.shape
    v32 = {}
    for i in range(n):
        for j in range(k):
            c = int(q[i, j])
            v = dec[c & 0x7F] * Fraction(float(s[i // 128, j // 128]))
            v32[i, j] = _f32r(-v if c & 0x80 else v)
    wp = {ij: _bf16r(v) for ij, v in v32.items()}
    st = _f32r(max(abs(v) for v in wp.values()) / 448)
    codes = np.zeros((n, k), np.int64)
    skip = np.zeros((n, k), np.int64)
    for (i, j), v in wp.items():
        neg = bool(q[i, j] & 0x80)
        codes[i, j] = _enc_fraction(_f32r(v / st), neg)
        skip[i, j] = _enc_fraction(_f32r(v32[i, j] / st), neg)
    return codes, st, skip


def test_naive_resync_brute_force():
    """The naive path recomputed element by element in exact rationals: w' = bf16(fl32(dec(q) s)),
    s_t = fl32(amax(w') / 448), q' = E4M3(fl32(w' / s_t)), on generic quantized weights and on
    a constructed pair of blocks: block 0 holds the tensor amax (code 448, s = 1, so s_t = 1),
    block 1 has s = 1.0625 + 2^-12, so code 1.0 dequantizes to 1.06274 in fp32 (above the
    1.0 / 1.125 midpoint: E4M3 1.125) but to exactly the midpoint 1.0625 in bf16 (ties to even:
    E4M3 1.0). Skipping the bf16 step therefore changes that code."""
    from fractions import Fraction

    w = normal_bf16((128, 384), 0.02, 100, 2)
    q, s = Q.quant_w_128x128(w)
    q2, s_t = S.naive_resync(q, s)
    codes, st, _ = _brute_naive(q, s)
    assert Fraction(float(s_t)) == st and np.array_equal(q2.astype(np.int64), codes)

    rng = np.random.default_rng(104)
    qc = rng.integers(0, 0x41, size=(128, 256), dtype=np.uint8) | (rng.integers(0, 2, (128, 256), dtype=np.uint8) << 7)
    qc[0, 0] = 0x7E
    qc[3, 130] = 0x38                                           # +1.0 in block 1
    qc[4, 131] = 0xB8                                           # -1.0 in block 1
    sc = np.array([[1.0, 1.0625 + 2.0 ** -12]], np.float32)
    q2, s_t = S.naive_resync(qc, sc)
    codes, st, skip = _brute_naive(qc, sc)
    assert s_t == np.float32(1.0) and st == 1
    assert np.array_equal(q2.astype(np.int64), codes)
    assert q2[3, 130] == 0x38 and q2[4, 131] == 0xB8            # bf16 midpoint -> even code 1.0
    assert skip[3, 130] == 0x39 and skip[4, 131] == 0xB9        # without the bf16 step: 1.125


def test_naive_path_by_row_blocks_equals_whole_tensor():
    """Split into 128-row blocks with the tensor scale taken from the maximum of the blocks'
    maxima, the naive path gives the whole tensor's bytes and scale, and its error sums add
    up to the whole tensor's mean relative error (how the benchmark evaluates it in
    parallel)."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((512, 256)) * 0.02).astype(np.float32)
    w[300, 7] = 0.9                                     # the tensor maximum sits in one block only
    q, s = Q.quant_w_128x128(bf16_round(w))
    q2, s_t = S.naive_resync(q, s)
    parts = [S.dequant_to_bf16(q[r:r + 128], s[r // 128:r // 128 + 1]) for r in range(0, 512, 128)]
    s_t_b = S.per_tensor_scale(max(np.max(np.abs(p)) for p in parts))
    assert s_t_b == s_t
    q2_b = np.concatenate([S.requant_per_tensor(p, s_t_b) for p in parts])
    assert np.array_equal(q2_b, q2)
    a = S.weight_value_block(q, s)
    b = S.weight_value_tensor(q2, s_t)
    num = sum(float(np.sum(np.abs(S.weight_value_tensor(q2_b[r:r + 128], s_t_b)
                                  - S.weight_value_block(q[r:r + 128], s[r // 128:r // 128 + 1]))))
              for r in range(0, 512, 128))
    assert abs(num / float(np.sum(np.abs(a))) - S.mean_relative_error(a, b)) < 1e-12
