"""HIP graph capture of library calls: the bench times its steps as graph replays, so every
kind of call its workloads make (blockwise, power-of-two and MXFP8 quantizers and GEMMs,
the few-row and grouped GEMMs, producers, install, FP32-master requantization) is captured
here, replayed several times with eager work and synchronizations in between, and every
replay is compared with the eager result. The
kernels are deterministic (fixed reduction order, no atomics), so the comparison is bitwise.
The calls launch kernels only (no memset, copy, allocation or synchronization)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from gpu_util import bf16_dev, dev
from test_gpu_parity import _rand
import workloads as W

pytestmark = pytest.mark.gpu


def _replays_match(run, outs, reps=3):
    """run() enqueues the calls writing into `outs`; compare graph replays with eager."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for r in range(reps):
        for o in outs:
            o.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {r}, output {i} differs from eager"


def test_graph_decode_call():
    """bf16 activations quantized inside the call (workspace) + the few-row GEMM."""
    M, N, K = 256, 4096, 1024
    x = bf16_dev(_rand((M, K), 11000))
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(_rand((N, K), 11001, 0.02)))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    ws = F.fwd_workspace(M, K, dev())
    _replays_match(lambda: F.fp8_gemm_blockscaled_fwd(wq=wq, sw=sw, x_bf16=x, y=y, workspace=ws), [y])


def test_graph_dense_forward_and_backward():
    """Row + column quantization, the large-tile forward, DGrad and WGrad (fp32 out)."""
    M, N, K = 512, 768, 512
    x = bf16_dev(_rand((M, K), 11100))
    dy = bf16_dev(_rand((M, N), 11101))
    w = bf16_dev(_rand((N, K), 11102, 0.02))
    u8, f32 = torch.uint8, torch.float32
    xq, sx = torch.empty((M, K), dtype=u8, device=dev()), torch.empty((M, K // 128), dtype=f32, device=dev())
    xqt, sxt = torch.empty((K, M), dtype=u8, device=dev()), torch.empty((K, M // 128), dtype=f32, device=dev())
    dq, sd = torch.empty((M, N), dtype=u8, device=dev()), torch.empty((M, N // 128), dtype=f32, device=dev())
    dqt, sdt = torch.empty((N, M), dtype=u8, device=dev()), torch.empty((N, M // 128), dtype=f32, device=dev())
    wq, sw = torch.empty((N, K), dtype=u8, device=dev()), torch.empty((N // 128, K // 128), dtype=f32, device=dev())
    wqt = torch.empty((K, N), dtype=u8, device=dev())
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev())
    dw = torch.empty((N, K), dtype=f32, device=dev())

    def run():
        F.fp8_quant_act_1x128(x, xq, sx, xqt, sxt, colwise=True)
        F.fp8_quant_w_128x128(w, wq, sw, wqt, transpose=True)
        F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, y=y)
        F.fp8_quant_act_1x128(dy, dq, sd, dqt, sdt, colwise=True)
        F.fp8_gemm_blockscaled_dgrad(dq, sd, wqt, sw, dx=dx)
        F.fp8_gemm_blockscaled_wgrad(dqt, sdt, xqt, sxt, dw=dw)
    _replays_match(run, [xq, sx, xqt, sxt, wq, sw, wqt, y, dq, sd, dqt, sdt, dx, dw])


def test_graph_grouped_moe():
    """MXFP8 quantization + the grouped GEMM (offsets read on the device)."""
    perm, offsets = W.zipf_topk_routing(128, 8, 2, 1.1, np.random.default_rng(11200))
    E, N, K = 8, 256, 512
    x = bf16_dev(_rand((128, K), 11201)[perm])
    wq, sw = F.mxfp8_quant_1x32(bf16_dev(_rand((E, N, K), 11202, 0.02)))
    off = torch.from_numpy(offsets).to(dev())
    T = x.shape[0]
    xq = torch.empty((T, K), dtype=torch.uint8, device=dev())
    sx = torch.empty((T, K // 32), dtype=torch.uint8, device=dev())
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev())

    def run():
        F.mxfp8_quant_1x32(x, q=xq, e8m0=sx)
        F.fp8_grouped_gemm(xq, sx, wq, sw, off, y=y)
    _replays_match(run, [xq, sx, y])


def test_graph_pow2_layer():
    """Power-of-two scales: quantizers (rows + columns, weight with transpose) and the three GEMMs."""
    M, N, K = 256, 512, 384
    x = bf16_dev(_rand((M, K), 11300))
    dy = bf16_dev(_rand((M, N), 11301))
    w = bf16_dev(_rand((N, K), 11302, 0.02))
    xq, sx, xqt, sxt = F.fp8_quant_act_1x128_pow2(x, colwise=True)
    dq, sd, dqt, sdt = F.fp8_quant_act_1x128_pow2(dy, colwise=True)
    wq, sw, wqt = F.fp8_quant_w_128x128_pow2(w, transpose=True)
    y = F.fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw)
    dx = F.fp8_gemm_blockscaled_pow2_dgrad(dq, sd, wqt, sw)
    dw = F.fp8_gemm_blockscaled_pow2_wgrad(dqt, sdt, xqt, sxt)

    def run():
        F.fp8_quant_act_1x128_pow2(x, xq, sx, xqt, sxt, colwise=True)
        F.fp8_quant_act_1x128_pow2(dy, dq, sd, dqt, sdt, colwise=True)
        F.fp8_quant_w_128x128_pow2(w, wq, sw, wqt, transpose=True)
        F.fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw, y=y)
        F.fp8_gemm_blockscaled_pow2_dgrad(dq, sd, wqt, sw, dx=dx)
        F.fp8_gemm_blockscaled_pow2_wgrad(dqt, sdt, xqt, sxt, dw=dw)
    _replays_match(run, [xq, sx, xqt, sxt, dq, sd, dqt, sdt, wq, sw, wqt, y, dx, dw])


def test_graph_mxfp8_dense_layer():
    """MXFP8 dense linear: 1x32 rows + 32x1 columns, forward, DGrad and WGrad."""
    M, N, K = 256, 512, 384
    x = bf16_dev(_rand((M, K), 11400))
    dy = bf16_dev(_rand((M, N), 11401))
    w = bf16_dev(_rand((N, K), 11402, 0.02))
    wt = bf16_dev(np.ascontiguousarray(_rand((N, K), 11402, 0.02).T))
    xq, ex, xqt, ext = F.mxfp8_quant_act_1x32(x, colwise=True)
    dq, ed, dqt, edt = F.mxfp8_quant_act_1x32(dy, colwise=True)
    wq, ew = F.mxfp8_quant_1x32(w)
    wtq, ewt = F.mxfp8_quant_1x32(wt)
    y = F.fp8_gemm_mxfp8_fwd(xq, ex, wq, ew)
    dx = F.fp8_gemm_mxfp8_dgrad(dq, ed, wtq, ewt)
    dw = F.fp8_gemm_mxfp8_wgrad(dqt, edt, xqt, ext)

    def run():
        F.mxfp8_quant_act_1x32(x, xq, ex, xqt, ext, colwise=True)
        F.mxfp8_quant_act_1x32(dy, dq, ed, dqt, edt, colwise=True)
        F.mxfp8_quant_1x32(w, q=wq, e8m0=ew)
        F.fp8_gemm_mxfp8_fwd(xq, ex, wq, ew, y=y)
        F.fp8_gemm_mxfp8_dgrad(dq, ed, wtq, ewt, dx=dx)
        F.fp8_gemm_mxfp8_wgrad(dqt, edt, xqt, ext, dw=dw)
    _replays_match(run, [xq, ex, xqt, ext, dq, ed, dqt, edt, wq, ew, y, dx, dw])


def test_graph_blockwise_grouped_producers_install_requant():
    """Blockwise grouped GEMM, the fused producers, the weight install and the FP32-master
    requantization, captured together."""
    perm, offsets = W.zipf_topk_routing(128, 8, 2, 1.1, np.random.default_rng(11500))
    E, N, K = 8, 256, 512
    x = bf16_dev(_rand((128, K), 11501)[perm])
    wg, swg, _ = F.fp8_quant_w_128x128(bf16_dev(_rand((E * N, K), 11502, 0.02)))
    wg, swg = wg.view(E, N, K), swg.view(E, N // 128, K // 128)
    off = torch.from_numpy(offsets).to(dev())
    xq, sx, _, _ = F.fp8_quant_act_1x128(x)
    yg = F.fp8_grouped_gemm(xq, sx, wg, swg, off, recipe=F.RECIPE_BLOCK128)
    gu = bf16_dev(_rand((256, 2 * 384), 11503))
    hq, hs, hqt, hst = F.fp8_swiglu_quant_1x128(gu, colwise=True)
    xr = bf16_dev(_rand((256, 512), 11504))
    gamma = bf16_dev(1.0 + _rand((512,), 11505, 0.1))
    rq, rs, rqt, rst, rr = F.fp8_rmsnorm_quant_1x128(xr, gamma, 1e-6, colwise=True)
    dq, ds = torch.empty_like(wg), torch.empty_like(swg)
    master = torch.from_numpy(np.random.default_rng(11506).standard_normal((512, 384)).astype(np.float32) * 0.02).to(dev())
    mq, ms, mqt = F.fp8_quant_w_128x128_f32(master, transpose=True)

    def run():
        F.fp8_quant_act_1x128(x, xq, sx)
        F.fp8_grouped_gemm(xq, sx, wg, swg, off, recipe=F.RECIPE_BLOCK128, y=yg)
        F.fp8_swiglu_quant_1x128(gu, hq, hs, hqt, hst, colwise=True)
        F.fp8_rmsnorm_quant_1x128(xr, gamma, 1e-6, rq, rs, rqt, rst, rr, colwise=True)
        F.fp8_weight_install(wg, swg, dq, ds)
        F.fp8_quant_w_128x128_f32(master, mq, ms, mqt, transpose=True)
    _replays_match(run, [xq, sx, yg, hq, hs, hqt, hst, rq, rs, rqt, rst, rr, dq, ds, mq, ms, mqt])
