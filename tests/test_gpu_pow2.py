"""GPU parity of the power-of-two block-scale entry points (the _pow2 quantizers and
GEMMs) against the oracle: bytes and scales bit for bit, GEMMs within the GEMM
tolerance, on seeded inputs with the quantizer's edge cases and scale exponents that span
the whole E8M0 range, the subnormal fp32 scale 2^-127 included."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import gemm as OG
from oracle import quantize as OQ
import workloads as W
from gpu_util import assert_bf16_consistent, assert_bytes_equal, assert_gemm_close, bf16_dev, f32_dev, host, u8_dev
from test_gpu_parity import _rand, _special_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(256, 512), (37, 384), (1, 128), (1000, 256)])
def test_pow2_quant_act_rows(M, K):
    x = _rand((M, K), 11000 + M)
    x[: min(M, 8)] = _special_rows(K, M)[: min(M, 8)]
    q, s, _, _ = F.fp8_quant_act_1x128_pow2(bf16_dev(x))
    rq, rs = OQ.quant_act_1x128_pow2(x)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(s, rs, "s")


@pytest.mark.parametrize("M,K,rows", [(256, 384, True), (384, 256, False), (128, 128, True), (512, 640, True)])
def test_pow2_quant_act_rows_and_columns(M, K, rows):
    x = _rand((M, K), 12000 + M + K)
    x[:8] = _special_rows(K, 17)
    x[:, 3] = 0.0
    x[200 % M, 5] = 1e30
    x[130 % M, 7] = 448.0 * 2.0 ** -20                 # amax exactly 448 * 2^e
    x = W.bf16_round(x)
    q, s, qt, st = F.fp8_quant_act_1x128_pow2(bf16_dev(x), rowwise=rows, colwise=True)
    rqt, rst = OQ.quant_act_128x1_pow2(x)
    assert_bytes_equal(qt, rqt, "qt")
    assert_bytes_equal(st, rst, "st")
    if rows:
        rq, rs = OQ.quant_act_1x128_pow2(x)
        assert_bytes_equal(q, rq, "q")
        assert_bytes_equal(s, rs, "s")
    else:
        assert q is None and s is None


@pytest.mark.parametrize("N,K", [(512, 512), (384, 256), (128, 1024)])
def test_pow2_quant_w_128x128(N, K):
    w = _rand((N, K), 13000 + N, 0.02).copy()
    w[:128, :128] = 0.0
    w[130 % N, 300 % K] = -3.0e38
    w[200 % N, 5] = 1e-39
    w = W.bf16_round(w)
    q, s, qt = F.fp8_quant_w_128x128_pow2(bf16_dev(w), transpose=True)
    rq, rs = OQ.quant_w_128x128_pow2(w)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(s, rs, "s")
    assert_bytes_equal(qt, OQ.transpose_payload(rq), "qt")


@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (300, 384, 640), (1, 128, 128), (17, 256, 384),
                                   (4096, 4096, 256), (777, 1280, 1152), (64, 8320, 256)])
def test_pow2_fwd(M, N, K):
    x = _rand((M, K), 14000 + M)
    w = _rand((N, K), 14001 + M, 0.02)
    xq, sx, _, _ = F.fp8_quant_act_1x128_pow2(bf16_dev(x))
    wq, sw, _ = F.fp8_quant_w_128x128_pow2(bf16_dev(w))
    y32 = F.fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    y16 = F.fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    rxq, rsx = OQ.quant_act_1x128_pow2(x)
    rwq, rsw = OQ.quant_w_128x128_pow2(w)
    ref = OG.gemm_fwd(rxq, rsx, rwq, rsw)
    assert_gemm_close(host(y32), ref, "pow2 fwd f32")
    assert_bf16_consistent(y16, y32, ref, "pow2 fwd bf16")


def test_pow2_fwd_full_exponent_range():
    """Scale exponents over the whole E8M0 range: ex[m][kb] = r[m] + g[kb] and
    ew[nb][kb] = c[nb] - g[kb] with g spanning [-120, 120], so single scales reach 2^-127
    (an fp32 subnormal, exponent field 0) and 2^127 while each product of scales is
    2^(r[m] + c[nb]). Dividing both results by that power of two (exact) leaves outputs of
    ordinary size, compared under the usual tolerance; a misread exponent changes one K
    block's weight by a power of two. The payloads are the E4M3 codes of Gaussian rows."""
    rng = np.random.default_rng(14500)
    M, N, K = 256, 512, 1024
    xq = OQ.quant_act_1x128(_rand((M, K), 14501))[0]
    wq = OQ.quant_act_1x128(_rand((N, K), 14502))[0]
    g = np.array([-120, -90, -50, -10, 10, 50, 90, 120])
    r = rng.integers(-7, 8, M)
    r[:2] = (-7, 7)
    c = np.array([-7, 7, 0, 3])
    ex, ew = r[:, None] + g[None, :], c[:, None] - g[None, :]
    assert ex.min() == -127 and ex.max() == 127 and ew.min() == -127 and ew.max() == 127
    sx = np.ldexp(np.float32(1.0), ex).astype(np.float32)
    sw = np.ldexp(np.float32(1.0), ew).astype(np.float32)
    assert (sx[0, 0].view(np.uint32) >> 23) == 0 and (sw[0, 7].view(np.uint32) >> 23) == 0
    y = host(F.fp8_gemm_blockscaled_pow2_fwd(u8_dev(xq), f32_dev(sx), u8_dev(wq), f32_dev(sw), out_dtype=torch.float32))
    ref = OG.gemm_fwd(xq, sx, wq, sw)
    norm = np.ldexp(1.0, -(r[:, None] + np.repeat(c, 128)[None, :]))
    assert_gemm_close(y * norm, ref * norm, "pow2 exponent range")


@pytest.mark.parametrize("M,N,K", [(256, 512, 384), (130, 256, 640), (1, 128, 128), (200, 256, 8320)])
def test_pow2_dgrad(M, N, K):
    dy = _rand((M, N), 15000 + M, 1e-3)
    w = _rand((N, K), 15001 + M, 0.02)
    dyq, sdy, _, _ = F.fp8_quant_act_1x128_pow2(bf16_dev(dy))
    wq, sw, wqt = F.fp8_quant_w_128x128_pow2(bf16_dev(w), transpose=True)
    dx32 = F.fp8_gemm_blockscaled_pow2_dgrad(dyq, sdy, wqt, sw, out_dtype=torch.float32)
    dx16 = F.fp8_gemm_blockscaled_pow2_dgrad(dyq, sdy, wqt, sw, out_dtype=torch.bfloat16)
    rdyq, rsdy = OQ.quant_act_1x128_pow2(dy)
    rwq, rsw = OQ.quant_w_128x128_pow2(w)
    ref = OG.gemm_dgrad(rdyq, rsdy, rwq, rsw)
    assert_gemm_close(host(dx32), ref, "pow2 dgrad f32")
    assert_bf16_consistent(dx16, dx32, ref, "pow2 dgrad bf16")


@pytest.mark.parametrize("M,N,K", [(256, 384, 256), (512, 128, 640), (128, 1024, 128), (1024, 2048, 1024)])
def test_pow2_wgrad(M, N, K):
    dy = _rand((M, N), 16000 + M, 1e-3)
    x = _rand((M, K), 16001 + M)
    _, _, dyqt, sdyt = F.fp8_quant_act_1x128_pow2(bf16_dev(dy), rowwise=False, colwise=True)
    _, _, xqt, sxt = F.fp8_quant_act_1x128_pow2(bf16_dev(x), rowwise=False, colwise=True)
    dw = F.fp8_gemm_blockscaled_pow2_wgrad(dyqt, sdyt, xqt, sxt)
    rdyqt, rsdyt = OQ.quant_act_128x1_pow2(dy)
    rxqt, rsxt = OQ.quant_act_128x1_pow2(x)
    ref = OG.gemm_wgrad(rdyqt, rsdyt, rxqt, rsxt)
    assert_gemm_close(host(dw), ref, "pow2 wgrad")
    base = torch.full_like(dw, 0.5)
    acc = F.fp8_gemm_blockscaled_pow2_wgrad(dyqt, sdyt, xqt, sxt, dw=base.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(acc, dw + 0.5)


def test_pow2_scales_through_the_fp32_scale_gemm():
    """Power-of-two scales are also valid fp32 scales: the general GEMM on the same
    operands agrees with the pow2 GEMM within the tolerance of each against the oracle."""
    M, N, K = 512, 768, 1024
    x = _rand((M, K), 17000)
    w = _rand((N, K), 17001, 0.02)
    xq, sx, _, _ = F.fp8_quant_act_1x128_pow2(bf16_dev(x))
    wq, sw, _ = F.fp8_quant_w_128x128_pow2(bf16_dev(w))
    a = F.fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    b = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    rxq, rsx = OQ.quant_act_1x128_pow2(x)
    rwq, rsw = OQ.quant_w_128x128_pow2(w)
    ref = OG.gemm_fwd(rxq, rsx, rwq, rsw)
    assert_gemm_close(host(a), ref, "pow2 path")
    assert_gemm_close(host(b), ref, "fp32-scale path")
