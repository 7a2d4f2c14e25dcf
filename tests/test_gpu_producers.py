"""GPU parity of the fused producers (SwiGLU -> FP8, RMSNorm -> FP8) and their bf16 forms
against the oracle: bf16 values, r, FP8 bytes and scales bit for bit. bf16(silu(g)) is
checked for every finite bf16 input. RMSNorm rows whose exact r lies within 2^-38 of an
fp32 rounding midpoint (reported by the oracle) would be excused from the bitwise
comparison; the seeded inputs here have none."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import producers as P
from oracle import quantize as OQ
import workloads as W
from gpu_util import assert_bytes_equal, bf16_dev, host

pytestmark = pytest.mark.gpu


def _gu(M, F_, seed, sigma=2.0):
    rng = np.random.default_rng(seed)
    gu = (rng.standard_normal((M, 2 * F_)).astype(np.float32) * np.float32(sigma))
    # gates across the regimes of silu: very negative, tiny (bf16 ties of g/2), large, zeros
    g = gu[:, :F_]
    g[0, :64] = -np.float32(90.0) - np.arange(64, dtype=np.float32)
    g[0, 64:128] = np.ldexp(np.float32(1.0), -np.arange(100, 164)).astype(np.float32) * 3
    if M > 1:
        g[1, :64] = -g[0, 64:128]
        g[1, 64:128] = np.float32(50.0) + np.arange(64, dtype=np.float32)
        g[1, 128 % F_] = 0.0
        g[1, 129 % F_] = -0.0
    return W.bf16_round(gu)


def test_silu_every_bf16_input():
    """h = bf16(silu(g) * 1) = bf16(silu(g)) for all 65280 finite bf16 g, bit for bit."""
    bits = np.arange(65536, dtype=np.uint32)
    g = (bits << 16).view(np.float32).copy()
    g[~np.isfinite(g)] = 0.0
    gate = g.reshape(128, 512)
    gu = np.concatenate([gate, np.ones_like(gate)], axis=1)
    h = host(F.fp8_swiglu_bf16(bf16_dev(gu)))
    ref = P.swiglu_bf16(gu)
    bad = np.flatnonzero(h.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"{bad.size} mismatches, first gates {g.reshape(-1)[bad[:5]]}"


@pytest.mark.parametrize("M,F_", [(256, 512), (37, 384), (1, 128), (130, 1280)])
def test_swiglu_bf16(M, F_):
    gu = _gu(M, F_, 100 + M)
    h = F.fp8_swiglu_bf16(bf16_dev(gu))
    assert_bytes_equal(h, P.swiglu_bf16(gu), "h")          # bf16 values compared as fp32 bit patterns


@pytest.mark.parametrize("M,F_,cols,pow2", [(256, 512, False, False), (37, 384, False, True), (128, 1280, True, False),
                                           (384, 256, True, True), (1000, 128, False, False)])
def test_swiglu_quant(M, F_, cols, pow2):
    gu = _gu(M, F_, 200 + M + F_)
    gud = bf16_dev(gu)
    q, s, qt, st = F.fp8_swiglu_quant_1x128(gud, colwise=cols, pow2_scales=pow2)
    ref = P.swiglu_quant_1x128(gu, pow2=pow2, colwise=cols)
    assert_bytes_equal(q, ref[0], "q")
    assert_bytes_equal(s, ref[1], "s")
    if cols:
        assert_bytes_equal(qt, ref[2], "qt")
        assert_bytes_equal(st, ref[3], "st")
        q2, s2, _, _ = F.fp8_swiglu_quant_1x128(gud, pow2_scales=pow2)        # rows-only kernel agrees
        torch.cuda.synchronize()
        assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    # fused == unfused (bf16 h through the plain quantizer)
    h = F.fp8_swiglu_bf16(gud)
    quant = F.fp8_quant_act_1x128_pow2 if pow2 else F.fp8_quant_act_1x128
    uq, us, _, _ = quant(h)
    torch.cuda.synchronize()
    assert torch.equal(q, uq) and torch.equal(s.view(torch.int32), us.view(torch.int32))


def _x_gamma(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[0] *= np.float32(2.0 ** -70)                               # tiny row
    if M > 1:
        x[1] *= np.float32(2.0 ** 60)                            # huge row
    if M > 2:
        x[2, ::5] = 0.0
    if M > 3:
        x[3, :] = 0.0                                            # all-zero row: r = 1/sqrt(eps)
    if M > 4:
        x[4, 7] = np.float32(3.0e4)                              # one dominant entry
    gamma = (np.float32(1.0) + rng.standard_normal(K).astype(np.float32) * np.float32(0.1))
    return W.bf16_round(x), W.bf16_round(gamma)


def _assert_rstd(rstd, r, amb):
    assert amb.sum() == 0, "seeded inputs should have no ambiguous rows"
    assert_bytes_equal(rstd, r, "rstd")


@pytest.mark.parametrize("M,K", [(256, 4096), (37, 1152), (3, 8192), (2, 65536), (130, 20480), (5, 128)])
def test_rmsnorm_bf16(M, K):
    x, gamma = _x_gamma(M, K, 300 + M)
    y, rstd = F.fp8_rmsnorm_bf16(bf16_dev(x), bf16_dev(gamma), 1e-6)
    ry, r, amb = P.rmsnorm_bf16(x, gamma, 1e-6)
    _assert_rstd(rstd, r, amb)
    assert_bytes_equal(y, ry, "y")


@pytest.mark.parametrize("M,K,cols,pow2", [(256, 4096, False, False), (37, 1152, False, True), (128, 512, True, False),
                                           (256, 384, True, True), (6, 16384, False, False), (2, 40960, False, False)])
def test_rmsnorm_quant(M, K, cols, pow2):
    x, gamma = _x_gamma(M, K, 400 + M + K)
    xd, gd = bf16_dev(x), bf16_dev(gamma)
    q, s, qt, st, rstd = F.fp8_rmsnorm_quant_1x128(xd, gd, 1e-6, colwise=cols, pow2_scales=pow2)
    ref = P.rmsnorm_quant_1x128(x, gamma, 1e-6, pow2=pow2, colwise=cols)
    _assert_rstd(rstd, ref[-2], ref[-1])
    assert_bytes_equal(q, ref[0], "q")
    assert_bytes_equal(s, ref[1], "s")
    if cols:
        assert_bytes_equal(qt, ref[2], "qt")
        assert_bytes_equal(st, ref[3], "st")
    # fused == unfused, and the two kernels' r agree
    y, r2 = F.fp8_rmsnorm_bf16(xd, gd, 1e-6)
    quant = F.fp8_quant_act_1x128_pow2 if pow2 else F.fp8_quant_act_1x128
    uq, us, _, _ = quant(y)
    torch.cuda.synchronize()
    assert torch.equal(q, uq) and torch.equal(s.view(torch.int32), us.view(torch.int32))
    assert torch.equal(rstd.view(torch.int32), r2.view(torch.int32))


def test_producers_empty_inputs():
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s, _, _ = F.fp8_swiglu_quant_1x128(e)
    assert q.shape == (0, 128) and s.shape == (0, 1)
    g = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    q, s, _, _, r = F.fp8_rmsnorm_quant_1x128(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), g)
    assert q.shape == (0, 128) and r.shape == (0,)
