"""Pins for the oracle's weight-sync functions: install is the identity on
bytes; the naive dequantize -> bf16 -> per-tensor requantize path is exact in a
closed-form special case and lossy otherwise; the relative-error definition on
a hand-computed tensor."""

import numpy as np

from oracle import quantize as Q
from oracle.fp8_formats import decode_e4m3
from oracle import weight_sync as S
from workloads import normal_bf16


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
