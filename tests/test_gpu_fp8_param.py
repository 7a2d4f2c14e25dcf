"""GPU parity of the fp8_param requantization (128x128 blocks quantized from an fp32 master,
with the byte transpose) against the oracle, bit for bit, and the synthetic displacement
check: a 5000-step trajectory of RL-sized updates requantized on the GPU reproduces the
oracle's codes exactly, and the FP8 storage displacement tracks the FP32 master
displacement (ratio near 1) for both scale formats, while single RL-sized steps have a low
update/storage-change cosine that rises with the update size."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import fp8_param as P
from oracle import quantize as OQ
from gpu_util import assert_bytes_equal, dev, host

pytestmark = pytest.mark.gpu


def _f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def _master(N, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[:128, :128] = 0.0                                     # an all-zero block
    w[5, 130 % K] = np.float32(0.731)                       # a block outlier
    w[200 % N, 7] = np.float32(1.0e30)                      # a huge value
    w[131 % N, 250 % K] = np.float32(2.0e-40)               # an fp32 subnormal
    return w


@pytest.mark.parametrize("N,K,pow2", [(256, 512, False), (256, 512, True), (128, 128, False), (384, 1024, True),
                                      (1024, 256, False)])
def test_fp8_param_requant_parity(N, K, pow2):
    w = _master(N, K, 30000 + N + K)
    q, s, qt = F.fp8_quant_w_128x128_f32(_f32_dev(w), transpose=True, pow2_scales=pow2)
    rq, rs = P.quant_w_128x128_f32(w, pow2)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(s, rs, "s")
    assert_bytes_equal(qt, OQ.transpose_payload(rq), "qt")


def test_fp8_param_tiny_blocks():
    """Blocks whose only nonzero values are fp32 subnormals: a scale that rounds to zero
    (raised to 2^-149) and one with a single significant bit whose quotient (512) saturates
    to 448; never a NaN code."""
    tiny = [2.0 ** -140, 2.0 ** -148, 2.0 ** -149, 300 * 2.0 ** -149, 223 * 2.0 ** -149, 3e-39]
    w = np.zeros((256, 128 * len(tiny)), np.float32)
    for b, a in enumerate(tiny):
        w[0, 128 * b] = np.float32(a)
        w[131, 128 * b + 5] = -np.float32(a)
        w[200, 128 * b + 9] = np.float32(a) * np.float32(0.5)
    for pow2 in (False, True):
        q, s, qt = F.fp8_quant_w_128x128_f32(_f32_dev(w), transpose=True, pow2_scales=pow2)
        rq, rs = P.quant_w_128x128_f32(w, pow2)
        assert_bytes_equal(q, rq, "q")
        assert_bytes_equal(s, rs, "s")
        assert_bytes_equal(qt, OQ.transpose_payload(rq), "qt")
        assert not np.any((host(q) & 0x7F) == 0x7F)
        if not pow2:
            assert host(s)[0, 0] == np.float32(2.0 ** -149) and host(q)[0, 0] == 0x7E


def test_fp8_param_bf16_values_match_bf16_quantizer():
    """On bf16-representable masters the fp32-input quantizer gives the bf16 quantizer's bytes."""
    rng = np.random.default_rng(30100)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w = (w.view(np.uint32) & 0xFFFF0000).view(np.float32)
    for pow2 in (False, True):
        q, s, _ = F.fp8_quant_w_128x128_f32(_f32_dev(w), pow2_scales=pow2)
        bq = F.fp8_quant_w_128x128_pow2 if pow2 else F.fp8_quant_w_128x128
        q2, s2, _ = bq(torch.from_numpy(w).to(torch.bfloat16).to(dev()))
        torch.cuda.synchronize()
        assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))


def _deq_gpu(q, s):
    return P.dequant(host(q), host(s))


@pytest.mark.parametrize("pow2", [False, True])
def test_fig12_displacement_trajectory(pow2):
    N = K = 256
    rng = np.random.default_rng(31000)
    w0 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = rng.standard_normal((N, K)).astype(np.float32)
    bank = [rng.standard_normal((N, K)).astype(np.float32) for _ in range(4)]
    lr, steps, cps = 1e-6, 5000, (1000, 5000)
    ref = P.trajectory(w0, bias, bank, lr, steps, cps, pow2)
    wd = _f32_dev(w0)
    bd = _f32_dev(bias)
    zd = [_f32_dev(z) for z in bank]
    q0, s0, _ = F.fp8_quant_w_128x128_f32(wd, pow2_scales=pow2)
    assert_bytes_equal(q0, ref[0][1], "q at step 0")
    d0 = _deq_gpu(q0, s0)
    for t in range(1, steps + 1):
        wd = wd + torch.sign(bd + zd[(t - 1) % 4]) * lr              # fp32: the oracle's step exactly
        if t in cps:
            q, s, _ = F.fp8_quant_w_128x128_f32(wd, pow2_scales=pow2)
            assert_bytes_equal(wd, ref[t][0], f"master at step {t}")
            assert_bytes_equal(q, ref[t][1], f"q at step {t}")
            assert_bytes_equal(s, ref[t][2], f"s at step {t}")
    l2, l1 = P.displacement_ratios(w0, host(wd), d0, _deq_gpu(q, s))
    rel_update = lr / float(np.mean(np.abs(w0)))
    assert 0.5e-4 < rel_update < 1.0e-4                      # the pages' 0.6-0.9e-4 per step
    assert 0.95 < l2 < 1.10 and 0.90 < l1 < 1.10, (l2, l1)


def test_fig12_cosine_rises_with_update_size():
    rng = np.random.default_rng(32000)
    w = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    b = rng.standard_normal(w.shape).astype(np.float32)
    wd = _f32_dev(w)
    for pow2 in (False, True):
        d0 = _deq_gpu(*F.fp8_quant_w_128x128_f32(wd, pow2_scales=pow2)[:2])
        cos = []
        for mag in (1e-7, 1e-6, 1e-5, 1e-4, 1e-3, 1e-2):
            dw = P.sign_step(b, np.zeros_like(b), mag)
            w1 = (w + dw).astype(np.float32)
            q1, s1, _ = F.fp8_quant_w_128x128_f32(_f32_dev(w1), pow2_scales=pow2)
            rq, rs = P.quant_w_128x128_f32(w1, pow2)
            assert_bytes_equal(q1, rq, f"q, update {mag}")
            cos.append(P.cosine(w1.astype(np.float64) - w, _deq_gpu(q1, s1) - d0))
        assert all(a < b for a, b in zip(cos, cos[1:])), cos
        assert cos[1] < 0.1 and cos[-1] > 0.99, cos
