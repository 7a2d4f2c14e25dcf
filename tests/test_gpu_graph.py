"""HIP graph capture of library calls: the bench times its steps as graph replays, so the
calls it makes are captured here, replayed several times with eager work and
synchronizations in between, and every replay is compared with the eager result. The
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
    ws = torch.empty(F.fp8rl_fwd_workspace_bytes(M, K), dtype=torch.uint8, device=dev())
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
