"""Guard regions: every output of the quantizers, the GEMMs (ragged, few-row, grouped),
the decode-layout forward and its workspace, the install and the fused producers is a view
into a larger buffer whose 256 bytes before and after hold seeded random bytes; after the
call those bytes must be unchanged (no kernel writes outside its outputs), and the outputs
themselves must match the unguarded call."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
import workloads as W
from gpu_util import bf16_dev, dev

pytestmark = pytest.mark.gpu

PAD = 256


class Guarded:
    """Buffers whose views are the call's outputs, framed by random guard bytes."""

    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)
        self.bufs = []

    def __call__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        pattern = torch.from_numpy(self.rng.integers(0, 256, PAD + n + PAD, dtype=np.uint8))
        buf = pattern.to(dev())
        self.bufs.append((buf, pattern, n))
        return buf[PAD:PAD + n].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        for i, (buf, pattern, n) in enumerate(self.bufs):
            h = buf.cpu()
            assert torch.equal(h[:PAD], pattern[:PAD]), f"{what}: output {i} wrote before its start"
            assert torch.equal(h[PAD + n:], pattern[PAD + n:]), f"{what}: output {i} wrote past its end"


def _same(a, b, what):
    torch.cuda.synchronize()
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


@pytest.mark.parametrize("M,K", [(1, 128), (300, 384), (256, 640)])
def test_quantizers_guarded(M, K):
    g = Guarded(M + K)
    x = bf16_dev(W.normal_bf16((M, K), 1.0, 94, M + K))
    colwise = M % 128 == 0
    outs = (g((M, K), torch.uint8), g((M, K // 128), torch.float32),
            g((K, M), torch.uint8) if colwise else None, g((K, M // 128), torch.float32) if colwise else None)
    F.fp8_quant_act_1x128(x, *outs, rowwise=True, colwise=colwise)
    ref = F.fp8_quant_act_1x128(x, rowwise=True, colwise=colwise)
    for a, b in zip(outs, ref):
        if a is not None:
            _same(a, b, "act 1x128")
    mq, me = g((M, K), torch.uint8), g((M, K // 32), torch.uint8)
    F.mxfp8_quant_1x32(x, q=mq, e8m0=me)
    rq, re = F.mxfp8_quant_1x32(x)
    _same(mq, rq, "mx q")
    _same(me, re, "mx e8m0")
    if M % 128 == 0:
        wq, ws, wqt = g((M, K), torch.uint8), g((M // 128, K // 128), torch.float32), g((K, M), torch.uint8)
        F.fp8_quant_w_128x128(x, q=wq, s=ws, qt=wqt, transpose=True)
        for a, b in zip((wq, ws, wqt), F.fp8_quant_w_128x128(x, transpose=True)):
            _same(a, b, "w 128x128")
    g.check(f"quantizers M={M} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (17, 384, 640), (300, 384, 640), (520, 1024, 256), (130, 24576, 256), (65, 24576, 256)])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_gemms_guarded(M, N, K, dt):
    g = Guarded(M * 7 + N + K)
    x = bf16_dev(W.normal_bf16((M, K), 1.0, 95, M + K))
    w = bf16_dev(W.normal_bf16((N, K), 0.02, 95, N + K))
    xq, sx = F.fp8_quant_act_1x128(x)[:2]
    wq, sw, wqt = F.fp8_quant_w_128x128(w, transpose=True)
    y = g((M, N), dt)
    F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=dt, y=y)
    _same(y, F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=dt), "fwd")
    # bf16 X with a guarded workspace, both weight layouts
    ws = g((F.load_library().fp8rl_fwd_workspace_bytes(M, K),), torch.uint8)
    y2 = g((M, N), dt)
    F.fp8_gemm_blockscaled_fwd(wq=wq, sw=sw, x_bf16=x, out_dtype=dt, y=y2, workspace=ws)
    dq, ds = g((N, K), torch.uint8), g((N // 128, K // 128), torch.float32)
    F.fp8_weight_install(wq, sw, dq, ds, layout=F.LAYOUT_DECODE)
    y3 = g((M, N), dt)
    F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=x, N=N, K=K, out_dtype=dt, y=y3, workspace=ws)
    _same(y2, y, "bf16-X fwd")
    ref3 = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=dq, sw=ds, x_bf16=x, N=N, K=K, out_dtype=dt)
    _same(y3, ref3, "decode-layout fwd")
    if M <= 256:                      # the same bits as the row-major forward (header promise)
        _same(y3, y, "decode layout vs row-major")
    # DGrad: dY [M][N] against W -> dX [M][K]
    dyq, sdy = F.fp8_quant_act_1x128(bf16_dev(W.normal_bf16((M, N), 1.0, 96, M + N)))[:2]
    dx = g((M, K), dt)
    F.fp8_gemm_blockscaled_dgrad(dyq, sdy, wqt, sw, out_dtype=dt, dx=dx)
    _same(dx, F.fp8_gemm_blockscaled_dgrad(dyq, sdy, wqt, sw, out_dtype=dt), "dgrad")
    g.check(f"GEMMs M={M} N={N} K={K} {dt}")


def test_wgrad_and_install_guarded():
    g = Guarded(7)
    M, N, K = 384, 256, 384
    x = bf16_dev(W.normal_bf16((M, K), 1.0, 97, 1))
    dy = bf16_dev(W.normal_bf16((M, N), 1.0, 97, 2))
    _, _, xqt, sxt = F.fp8_quant_act_1x128(x, rowwise=False, colwise=True)
    _, _, dyqt, sdyt = F.fp8_quant_act_1x128(dy, rowwise=False, colwise=True)
    dw = g((N, K), torch.float32)
    dw.zero_()
    F.fp8_gemm_blockscaled_wgrad(dyqt, sdyt, xqt, sxt, dw=dw, accumulate=True)
    _same(dw, F.fp8_gemm_blockscaled_wgrad(dyqt, sdyt, xqt, sxt), "wgrad accumulate onto zero")
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(W.normal_bf16((N, K), 0.02, 97, 3)))
    iq, is_ = g((N, K), torch.uint8), g((N // 128, K // 128), torch.float32)
    F.fp8_weight_install(wq, sw, iq, is_)
    _same(iq, wq, "install payload")
    _same(is_, sw, "install scales")
    g.check("wgrad + install")


@pytest.mark.parametrize("recipe", ["mx", "block"])
def test_grouped_guarded(recipe):
    g = Guarded(11)
    counts = [0, 37, 200, 1, 90, 0, 128]
    E, N, K = len(counts), 256, 256
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    x = bf16_dev(W.normal_bf16((T, K), 1.0, 98, 1))
    w = bf16_dev(W.normal_bf16((E * N, K), 0.02, 98, 2))
    offd = torch.from_numpy(off).to(dev())
    if recipe == "mx":
        xq, sx = F.mxfp8_quant_1x32(x)
        wq, sw = F.mxfp8_quant_1x32(w)
        wq, sw, rc = wq.view(E, N, K), sw.view(E, N, K // 32), F.RECIPE_MXFP8
    else:
        xq, sx = F.fp8_quant_act_1x128(x)[:2]
        wq, sw, _ = F.fp8_quant_w_128x128(w)
        wq, sw, rc = wq.view(E, N, K), sw.view(E, N // 128, K // 128), F.RECIPE_BLOCK128
    for dt in (torch.bfloat16, torch.float32):
        y = g((T, N), dt)
        F.fp8_grouped_gemm(xq, sx, wq, sw, offd, recipe=rc, out_dtype=dt, y=y)
        _same(y, F.fp8_grouped_gemm(xq, sx, wq, sw, offd, recipe=rc, out_dtype=dt), f"grouped {recipe} {dt}")
    g.check(f"grouped {recipe}")


def test_producers_guarded():
    g = Guarded(13)
    M, Fh, K = 256, 384, 512
    gu = bf16_dev(W.normal_bf16((M, 2 * Fh), 1.0, 99, 1))
    outs = (g((M, Fh), torch.uint8), g((M, Fh // 128), torch.float32), g((Fh, M), torch.uint8),
            g((Fh, M // 128), torch.float32))
    F.fp8_swiglu_quant_1x128(gu, *outs, rowwise=True, colwise=True)
    for a, b in zip(outs, F.fp8_swiglu_quant_1x128(gu, rowwise=True, colwise=True)):
        _same(a, b, "swiglu quant")
    x = bf16_dev(W.normal_bf16((M, K), 1.0, 99, 2))
    gamma = bf16_dev(W.bf16_round(np.float32(1.0) + W.normal_bf16((K,), 0.1, 99, 3)))
    outs = (g((M, K), torch.uint8), g((M, K // 128), torch.float32), g((K, M), torch.uint8),
            g((K, M // 128), torch.float32), g((M,), torch.float32))
    F.fp8_rmsnorm_quant_1x128(x, gamma, 1e-6, *outs, rowwise=True, colwise=True)
    for a, b in zip(outs, F.fp8_rmsnorm_quant_1x128(x, gamma, 1e-6, rowwise=True, colwise=True)):
        _same(a, b, "rmsnorm quant")
    g.check("producers")


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("M,K", [(2560, 4096), (4096, 3200), (8320, 1024)])
def test_tile_quantizer_many_tiles(M, K, pow2):
    """Row + column quantization with several 128x128 tiles per CU (tile counts that do not
    divide evenly over the CUs, column-block counts with and without a factor 8, i.e. both
    tile orders): guarded outputs, rows equal to the row-only quantizer's, columns equal to
    the row-only quantizer's on the transposed matrix."""
    g = Guarded(M * 3 + K)
    x = bf16_dev(W.normal_bf16((M, K), 1.0, 93, M + K))
    outs = (g((M, K), torch.uint8), g((M, K // 128), torch.float32), g((K, M), torch.uint8),
            g((K, M // 128), torch.float32))
    quant = F.fp8_quant_act_1x128_pow2 if pow2 else F.fp8_quant_act_1x128
    quant(x, *outs, rowwise=True, colwise=True)
    rq, rs = quant(x, rowwise=True, colwise=False)[:2]
    tq, ts = quant(x.t().contiguous(), rowwise=True, colwise=False)[:2]
    _same(outs[0], rq, "rows q")
    _same(outs[1], rs, "rows s")
    _same(outs[2], tq, "columns qt")
    _same(outs[3], ts, "columns st")
    g.check(f"streaming tile quantizer M={M} K={K} pow2={pow2}")
