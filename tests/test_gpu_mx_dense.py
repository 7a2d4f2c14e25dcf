"""GPU parity of the MXFP8 dense linear layer against the oracle: the 1x32 / 32x1 (transposed)
quantizer bit for bit, and the forward, DGrad and WGrad GEMMs within the GEMM tolerance
(bf16 outputs also equal to the RNE rounding of the same kernel's fp32 output)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import gemm as OG
from oracle import quantize as OQ
import workloads as W
from gpu_util import assert_bf16_consistent, assert_bytes_equal, assert_gemm_close, bf16_dev, host
from test_gpu_parity import _rand, _special_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("R,K,rows,cols", [(256, 512, True, True), (128, 128, False, True), (384, 256, True, True),
                                           (37, 96, True, False), (1024, 384, True, True)])
def test_mx_quant_rows_and_columns(R, K, rows, cols):
    x = _rand((R, K), 20000 + R + K)
    if K >= 128:
        x[:8] = _special_rows(K, 21)[:, :K]
        x[:, 3] = 0.0                                          # an all-zero column
        x[40 % R, 7] = 448.0 * 8                               # exactly at an exponent boundary
        x = W.bf16_round(x)
    q, e, qt, et = F.mxfp8_quant_act_1x32(bf16_dev(x), rowwise=rows, colwise=cols)
    if rows:
        rq, re = OQ.quant_mx_1x32(x)
        assert_bytes_equal(q, rq, "q")
        assert_bytes_equal(e, re, "e8m0")
    if cols:
        rqt, ret = OQ.quant_mx_32x1(x)
        assert_bytes_equal(qt, rqt, "qt")
        assert_bytes_equal(et, ret, "e8m0t")
        if rows:                                               # the tile kernel's rows equal the 1x32 kernel's
            q2, e2 = F.mxfp8_quant_1x32(bf16_dev(x))
            torch.cuda.synchronize()
            assert torch.equal(q, q2) and torch.equal(e, e2)


@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (300, 384, 640), (1, 128, 128), (17, 256, 384),
                                   (4096, 4096, 256), (777, 1280, 1152)])
def test_mx_fwd(M, N, K):
    x = _rand((M, K), 21000 + M)
    w = _rand((N, K), 21001 + M, 0.02)
    xq, ex, _, _ = F.mxfp8_quant_act_1x32(bf16_dev(x))
    wq, ew, _, _ = F.mxfp8_quant_act_1x32(bf16_dev(w))
    y32 = F.fp8_gemm_mxfp8_fwd(xq, ex, wq, ew, out_dtype=torch.float32)
    y16 = F.fp8_gemm_mxfp8_fwd(xq, ex, wq, ew, out_dtype=torch.bfloat16)
    rxq, rex = OQ.quant_mx_1x32(x)
    rwq, rew = OQ.quant_mx_1x32(w)
    ref = OG.gemm_mx_fwd(rxq, rex, rwq, rew)
    assert_gemm_close(host(y32), ref, "mx fwd f32")
    assert_bf16_consistent(y16, y32, ref, "mx fwd bf16")


@pytest.mark.parametrize("M,N,K", [(256, 512, 384), (130, 256, 640), (1, 128, 128), (200, 256, 8320)])
def test_mx_dgrad(M, N, K):
    dy = _rand((M, N), 22000 + M, 1e-3)
    w = _rand((N, K), 22001 + M, 0.02)
    dyq, edy, _, _ = F.mxfp8_quant_act_1x32(bf16_dev(dy))
    _, _, wqt, ewt = F.mxfp8_quant_act_1x32(bf16_dev(w), rowwise=False, colwise=True)
    dx32 = F.fp8_gemm_mxfp8_dgrad(dyq, edy, wqt, ewt, out_dtype=torch.float32)
    dx16 = F.fp8_gemm_mxfp8_dgrad(dyq, edy, wqt, ewt, out_dtype=torch.bfloat16)
    rdyq, redy = OQ.quant_mx_1x32(dy)
    rwqt, rewt = OQ.quant_mx_32x1(w)
    ref = OG.gemm_mx_dgrad(rdyq, redy, rwqt, rewt)
    assert_gemm_close(host(dx32), ref, "mx dgrad f32")
    assert_bf16_consistent(dx16, dx32, ref, "mx dgrad bf16")


@pytest.mark.parametrize("M,N,K", [(256, 384, 256), (512, 128, 640), (128, 1024, 128), (1024, 2048, 1024)])
def test_mx_wgrad(M, N, K):
    dy = _rand((M, N), 23000 + M, 1e-3)
    x = _rand((M, K), 23001 + M)
    _, _, dyqt, edyt = F.mxfp8_quant_act_1x32(bf16_dev(dy), rowwise=False, colwise=True)
    _, _, xqt, ext = F.mxfp8_quant_act_1x32(bf16_dev(x), rowwise=False, colwise=True)
    dw = F.fp8_gemm_mxfp8_wgrad(dyqt, edyt, xqt, ext)
    rdyqt, redyt = OQ.quant_mx_32x1(dy)
    rxqt, rext = OQ.quant_mx_32x1(x)
    ref = OG.gemm_mx_wgrad(rdyqt, redyt, rxqt, rext)
    assert_gemm_close(host(dw), ref, "mx wgrad")
    base = torch.full_like(dw, 0.5)
    acc = F.fp8_gemm_mxfp8_wgrad(dyqt, edyt, xqt, ext, dw=base.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(acc, dw + 0.5)


def test_mx_fwd_matches_grouped_single_expert():
    """The dense MXFP8 forward and the grouped MXFP8 GEMM with one expert compute the same
    product; both are compared with the oracle."""
    M, N, K = 512, 256, 512
    x = _rand((M, K), 24000)
    w = _rand((N, K), 24001, 0.02)
    xq, ex, _, _ = F.mxfp8_quant_act_1x32(bf16_dev(x))
    wq, ew, _, _ = F.mxfp8_quant_act_1x32(bf16_dev(w))
    y = F.fp8_gemm_mxfp8_fwd(xq, ex, wq, ew, out_dtype=torch.float32)
    off = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    yg = F.fp8_grouped_gemm(xq, ex, wq.unsqueeze(0), ew.unsqueeze(0), off, out_dtype=torch.float32)
    ref = OG.gemm_mx_fwd(*OQ.quant_mx_1x32(x), *OQ.quant_mx_1x32(w))
    assert_gemm_close(host(y), ref, "dense mx")
    assert_gemm_close(host(yg), ref, "grouped mx")
