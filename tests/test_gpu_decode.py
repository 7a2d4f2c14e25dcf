"""GPU tests of the decode-shaped forward path: the bf16-input form (the activations
quantized 1x128 inside the call), the decode weight layout written by the install, and
the bit identity of trainer and rollout outputs across both layouts ([SkyRL-FP8]
"On-Policy FP8 weight sync": installed weights reproduce the trainer's outputs exactly;
"Performance analysis": decode is bound by the weight stream)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
import workloads as W
from oracle import gemm as OG
from oracle import quantize as OQ
from gpu_util import assert_bytes_equal, assert_gemm_close, bf16_dev, dev, host

pytestmark = pytest.mark.gpu


def decode_layout_reference(q: np.ndarray) -> np.ndarray:
    """The decode layout as the header defines it, written with numpy reshapes: for 16-row
    group f and K block kb, lane i = 16 g + r (r = i % 16, g = i // 16) holds bytes
    kb*128 + 16 g .. +15 (first kilobyte) and kb*128 + 64 + 16 g .. +15 (second) of row 16 f + r."""
    N, K = q.shape
    t = q.reshape(N // 16, 16, K // 128, 2, 4, 16)          # [f][r][kb][half][g][byte]
    return np.ascontiguousarray(t.transpose(0, 2, 3, 4, 1, 5)).reshape(N, K)


def _weights(N, K, seed):
    w = W.normal_bf16((N, K), 0.02, 77, seed)
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w))
    return w, wq, sw


def _install_decode(wq, sw):
    dq, ds = torch.empty_like(wq), torch.empty_like(sw)
    F.fp8_weight_install(wq, sw, dq, ds, layout=F.LAYOUT_DECODE)
    return dq, ds


@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (2048, 1024)])
def test_decode_layout_install_bytes(N, K):
    _, wq, sw = _weights(N, K, N + K)
    dq, ds = _install_decode(wq, sw)
    assert_bytes_equal(dq, decode_layout_reference(host(wq)), "decode-layout payload")
    assert_bytes_equal(ds, host(sw), "scales (verbatim)")
    # same-layout installs stay verbatim copies
    dq2, ds2 = torch.empty_like(dq), torch.empty_like(ds)
    F.fp8_weight_install(dq, ds, dq2, ds2, layout=F.LAYOUT_DECODE, src_layout=F.LAYOUT_DECODE)
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq) and torch.equal(ds2.view(torch.int32), ds.view(torch.int32))


@pytest.mark.parametrize("M", [1, 17, 64, 130, 256])
@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (2048, 1024)])
def test_decode_layout_forward_matches_rows(M, N, K):
    """Trainer (row-major payload) and rollout (decode layout) outputs are bit-identical for
    both forms of X and both output types, and within tolerance of the oracle."""
    x = W.normal_bf16((M, K), 1.0, 78, M * 7 + N)
    w, wq, sw = _weights(N, K, M + 3 * N + K)
    dq, ds = _install_decode(wq, sw)
    xt = bf16_dev(x)
    xq, sx = F.fp8_quant_act_1x128(xt)[:2]
    for dt in (torch.float32, torch.bfloat16):
        y_rows = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=dt)
        y_dec = F.fp8_gemm_blockscaled_fwd_decode_layout(xq, sx, dq, ds, N=N, K=K, out_dtype=dt)
        y_rows_f = F.fp8_gemm_blockscaled_fwd(wq=wq, sw=sw, x_bf16=xt, out_dtype=dt)
        y_dec_f = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=xt, N=N, K=K, out_dtype=dt)
        torch.cuda.synchronize()
        iv = torch.int32 if dt == torch.float32 else torch.int16
        for other, name in ((y_dec, "decode layout"), (y_rows_f, "bf16 X"), (y_dec_f, "bf16 X, decode layout")):
            assert torch.equal(other.view(iv), y_rows.view(iv)), f"{name} differs from the row-major forward"
        if dt == torch.float32:
            rxq, rsx = OQ.quant_act_1x128(x)
            rwq, rsw = OQ.quant_w_128x128(w)
            assert_gemm_close(host(y_rows), OG.gemm_fwd(rxq, rsx, rwq, rsw), f"decode fwd M={M} N={N} K={K}")


def test_bf16_form_workspace_copy_and_repeat():
    """The bf16-input call accepts a workspace with any contents, its K-block-major copy of X
    holds exactly the 1x128 quantizer's bytes and scales, and repeated calls on one workspace
    agree bit for bit."""
    M, N, K = 200, 1024, 1536
    x = W.normal_bf16((M, K), 1.0, 79, 1)
    _, wq, sw = _weights(N, K, 5)
    ws = F.fwd_workspace(M, K, dev())
    ws.fill_(0xFF)
    xt = bf16_dev(x)
    ys = [F.fp8_gemm_blockscaled_fwd(wq=wq, sw=sw, x_bf16=xt, out_dtype=torch.float32, workspace=ws)
          for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int32), ys[0].view(torch.int32))
    rq, rs = OQ.quant_act_1x128(x)
    nkb = K // 128
    qpad = (M * K + 255) // 256 * 256
    wsq = host(ws[:M * K]).reshape(nkb, M, 128)
    wss = host(ws[qpad:qpad + M * nkb * 4]).view(np.float32).reshape(nkb, M)
    assert np.array_equal(wsq, rq.reshape(M, nkb, 128).transpose(1, 0, 2))
    assert np.array_equal(wss.view(np.uint32), np.ascontiguousarray(rs.T).view(np.uint32))


def test_decode_many_workgroups_per_cu():
    """A wide weight gives more workgroups than CUs, so several share a CU: outputs of both
    layouts agree bit for bit and match the oracle on sampled columns."""
    M, N, K = 256, 32768, 256
    x = W.normal_bf16((M, K), 1.0, 80, 2)
    w, wq, sw = _weights(N, K, 6)
    dq, ds = _install_decode(wq, sw)
    xt = bf16_dev(x)
    y_rows = F.fp8_gemm_blockscaled_fwd(wq=wq, sw=sw, x_bf16=xt, out_dtype=torch.bfloat16)
    y_dec = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=xt, N=N, K=K, out_dtype=torch.bfloat16)
    y32 = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=xt, N=N, K=K, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_rows.view(torch.int16), y_dec.view(torch.int16))
    assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y_dec.view(torch.int16))
    cols = np.random.default_rng(3).choice(N // 128, 6, replace=False)
    wcols = np.concatenate([np.arange(c * 128, (c + 1) * 128) for c in sorted(cols)])
    rxq, rsx = OQ.quant_act_1x128(x)
    rwq, rsw = OQ.quant_w_128x128(w[wcols])
    assert_gemm_close(host(y32)[:, wcols], OG.gemm_fwd(rxq, rsx, rwq, rsw), "decode, many workgroups")


@pytest.mark.parametrize("K", [256, 512, 640, 768, 1280])
def test_decode_every_k_block(K):
    """X nonzero in one K block at a time: every K block of the weight stream (before, at and
    past the prefetch distance, over several passes of the K loop) enters the product once,
    identically for both weight layouts, and the result matches the oracle. Regression for
    weight loads that took a stale descriptor (a load reading its base SGPRs too soon after
    the VALU instruction that wrote them)."""
    M, N = 1, 384
    nkb = K // 128
    w = W.normal_bf16((N, K), 0.02, 81, K)
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w))
    dq, ds = _install_decode(wq, sw)
    rwq, rsw = OQ.quant_w_128x128(w)
    for j in range(nkb):
        x = np.zeros((M, K), np.float32)
        x[:, j * 128:(j + 1) * 128] = W.normal_bf16((M, 128), 1.0, 82, K * 16 + j)
        xt = bf16_dev(x)
        xq, sx = F.fp8_quant_act_1x128(xt)[:2]
        y_rows = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
        y_dec = F.fp8_gemm_blockscaled_fwd_decode_layout(xq, sx, dq, ds, N=N, K=K, out_dtype=torch.float32)
        y_dec_f = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=xt, N=N, K=K,
                                                           out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y_dec.view(torch.int32), y_rows.view(torch.int32)), f"K block {j}: layouts differ"
        assert torch.equal(y_dec_f.view(torch.int32), y_rows.view(torch.int32)), f"K block {j}: bf16-X form differs"
        rxq, rsx = OQ.quant_act_1x128(host(xt))
        assert_gemm_close(host(y_rows), OG.gemm_fwd(rxq, rsx, rwq, rsw), f"K={K} block {j}")


# Shapes that make the launch choose each configuration of the decode kernel (weight
# fragments per wave 1, 2 and 3; row part 64), with one to three row parts (the last one
# ragged) and grids of one to a few hundred workgroups. (1, 49280), (130, 24576) and
# (200, 36864) give the grids with a workgroup per CU for two row parts per workgroup, which
# take the form that stages decode-layout weights in LDS (the last two with a ragged second
# row part). (65, 24576) and (256, 12288) give three-fragment grids of exactly one workgroup per
# CU, which take the staged form with one row part; one-fragment grids of at most 256
# workgroups take it too.
_CONFIG_SHAPES = [(1, 128), (1, 16512), (1, 32896), (1, 49280), (65, 8320), (65, 16512), (65, 32896),
                  (65, 24576), (129, 11008), (129, 16512), (130, 24576), (200, 36864), (256, 12288)]


@pytest.mark.parametrize("M,N", _CONFIG_SHAPES)
@pytest.mark.parametrize("K", [256, 640])
def test_decode_every_config(M, N, K):
    """Each configuration: row-major and decode-layout weights and both forms of X give the
    same bits, and sampled 128-column blocks match the oracle."""
    _check_layouts_and_oracle(M, N, K)


@pytest.mark.parametrize("M,N", [(1, 384), (130, 4096)])
@pytest.mark.parametrize("K", [8192, 8320])
def test_decode_long_k(M, N, K):
    """K = 8192 (64 K blocks) is the longest K range whose scales the decode kernel loads into
    LDS before its K loop; K = 8320 (65) takes the kernel that copies the scales per K block.
    Both weight layouts and both forms of X agree bit for bit and match the oracle."""
    _check_layouts_and_oracle(M, N, K)


def _check_layouts_and_oracle(M, N, K):
    x = W.normal_bf16((M, K), 1.0, 83, M * 3 + N + K)
    w = W.normal_bf16((N, K), 0.02, 84, N + K)
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w))
    dq, ds = _install_decode(wq, sw)
    xt = bf16_dev(x)
    xq, sx = F.fp8_quant_act_1x128(xt)[:2]
    y_rows = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    y_dec = F.fp8_gemm_blockscaled_fwd_decode_layout(xq, sx, dq, ds, N=N, K=K, out_dtype=torch.float32)
    y_dec_b = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=xt, N=N, K=K, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_dec.view(torch.int32), y_rows.view(torch.int32)), "decode layout differs"
    assert torch.equal(y_dec_b.view(torch.int16), y_rows.to(torch.bfloat16).view(torch.int16)), "bf16 form differs"
    blocks = np.random.default_rng(N).choice(N // 128, min(4, N // 128), replace=False)
    cols = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in sorted(blocks)])
    rxq, rsx = OQ.quant_act_1x128(x)
    rwq, rsw = OQ.quant_w_128x128(w[cols])
    assert_gemm_close(host(y_rows)[:, cols], OG.gemm_fwd(rxq, rsx, rwq, rsw), f"M={M} N={N} K={K}")
