"""GPU test of the allocation-free forward (fp8_gemm_blockscaled_fwd_decode_layout_noalloc):
through the C ABI it gives the same bits as the workspace form on two calls in a row, the
second smaller, and rejects a size beyond its built-in scratch on the host."""

import ctypes

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
import workloads as W
from gpu_util import bf16_dev, dev

pytestmark = pytest.mark.gpu


def _weights(N, K, seed):
    w = W.normal_bf16((N, K), 0.02, 85, seed)
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w))
    dq, ds = torch.empty_like(wq), torch.empty_like(sw)
    F.fp8_weight_install(wq, sw, dq, ds, layout=F.LAYOUT_DECODE)
    return dq, ds


def test_noalloc_matches_workspace_form_twice():
    # second call smaller: the scratch keeps the first call's bytes past the second's extent
    for M, N, K, dt in [(256, 4096, 4096, torch.bfloat16), (17, 1024, 640, torch.float32)]:
        x = bf16_dev(W.normal_bf16((M, K), 1.0, 86, M + K))
        dq, ds = _weights(N, K, N + K)
        ws = F.fwd_workspace(M, K, dev())
        y_ref = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=x, N=N, K=K, out_dtype=dt, workspace=ws)
        y = torch.empty((M, N), dtype=dt, device=dev())
        F.fp8_gemm_blockscaled_fwd_decode_layout_noalloc(wq=dq, sw=ds, x_bf16=x, N=N, K=K, out_dtype=dt, y=y)
        torch.cuda.synchronize()
        iv = torch.int32 if dt == torch.float32 else torch.int16
        assert torch.equal(y.view(iv), y_ref.view(iv)), f"M={M} N={N} K={K}"


def test_noalloc_quantized_form_and_oversize():
    lib = F.load_library()
    M, N, K = 9, 256, 384
    x = bf16_dev(W.normal_bf16((M, K), 1.0, 87, 1))
    dq, ds = _weights(N, K, 2)
    xq, sx = F.fp8_quant_act_1x128(x)[:2]
    y_ref = F.fp8_gemm_blockscaled_fwd_decode_layout(xq, sx, dq, ds, N=N, K=K)
    y = F.fp8_gemm_blockscaled_fwd_decode_layout_noalloc(xq, sx, dq, ds, N=N, K=K)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    # M * K beyond the scratch: rejected on the host before any launch (the pointers are
    # valid 16-byte-aligned buffers; no kernel runs)
    big_m = F.NOALLOC_SCRATCH_BYTES // K + 1
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.fp8_gemm_blockscaled_fwd_decode_layout_noalloc(None, None, P(x), P(dq), P(ds), big_m, N, K, P(y), 0,
                                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 7, F.status_name(st) if hasattr(F, "status_name") else st
    assert F.load_library().fp8rl_fwd_workspace_bytes(big_m, K) > F.NOALLOC_SCRATCH_BYTES
