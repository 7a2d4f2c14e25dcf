"""GPU parity of the GEMMs in their 256x256-tile configuration, the one the full-size
workloads run, with ragged edges: M = 4000 and N = 4224 give 16 x 17 tiles whose last row
and column of tiles are partial (3968 rows for the blockscaled WGrad, whose rows are whole
128-row weight blocks), and the reduction of 3072 = 24 K blocks takes the row
scales through the LDS ring (8 K blocks per load for 1x128 scales; 4 for row scales on both
operands) over several chunks, so both ring buffers are filled, read and refilled.
Every scale format and GEMM kind runs: fp32 and power-of-two 1x128 / 128x128 scales
(forward, DGrad, WGrad) and MXFP8 (forward, DGrad, WGrad). Operands are quantized by the
oracle from seeded Gaussian data; the oracle recomputes sampled output rows (among them
the rows of the partial last tile) against every column. Tolerance: max error <= 2e-3 x
RMS of the reference rows; bf16 outputs equal the RNE rounding of the fp32 outputs."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import gemm as OG
from oracle import quantize as OQ
from gpu_util import assert_gemm_close, dev, f32_dev, host, u8_dev
from test_gpu_parity import _rand

pytestmark = pytest.mark.gpu

M, N, R = 4000, 4224, 3072            # output rows, output columns, reduction length
ROWS = np.array([0, 1, 255, 256, 1023, 2047, 2500, 3071, 3583, 3840, 3841, 3900, 3998, 3999])
NW = 3968                             # blockscaled WGrad: dW rows are whole 128-row weight blocks
ROWS_W = np.array([0, 255, 256, 2047, 3071, 3583, 3840, 3841, 3900, 3967])


def _e8m0_dev(e):
    return torch.from_numpy(np.ascontiguousarray(e, dtype=np.uint8)).to(dev())


@pytest.fixture(scope="module")
def data():
    a = _rand((M, R), 40000)                   # A rows: X, dY or the column-wise dY copy
    b = _rand((N, R), 40001, 0.02)             # B rows: W or the column-wise X copy
    wd = _rand((R, N), 40002, 0.02)            # the DGrad weight W[R][N] (output has N columns)
    return a, b, wd


def _check(y32, y16, ref, what):
    got = host(y32[torch.from_numpy(ROWS).to(dev())])
    assert_gemm_close(got, ref, what)
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), f"{what}: bf16 != RNE(f32)"


@pytest.mark.parametrize("pow2", [False, True])
def test_bigtile_blockscaled_forward(data, pow2):
    a, b, _ = data
    qa = OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128
    qw = OQ.quant_w_128x128_pow2 if pow2 else OQ.quant_w_128x128
    fwd = F.fp8_gemm_blockscaled_pow2_fwd if pow2 else F.fp8_gemm_blockscaled_fwd
    aq, sa = qa(a)
    bq, sb = qw(b)
    args = (u8_dev(aq), f32_dev(sa), u8_dev(bq), f32_dev(sb))
    y32 = fwd(*args, out_dtype=torch.float32)
    y16 = fwd(*args, out_dtype=torch.bfloat16)
    _check(y32, y16, OG.gemm_fwd(aq[ROWS], sa[ROWS], bq, sb), f"fwd pow2={pow2}")


def test_bigtile_deterministic(data):
    """Two launches of the ring-path kernel on the ragged big-tile shape give the same bits
    (fixed K order, no atomics)."""
    a, b, _ = data
    aq, sa = OQ.quant_act_1x128(a)
    bq, sb = OQ.quant_w_128x128(b)
    args = (u8_dev(aq), f32_dev(sa), u8_dev(bq), f32_dev(sb))
    y1 = F.fp8_gemm_blockscaled_fwd(*args, out_dtype=torch.float32)
    y2 = F.fp8_gemm_blockscaled_fwd(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("pow2", [False, True])
def test_bigtile_blockscaled_dgrad(data, pow2):
    a, _, wd = data
    qa = OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128
    qw = OQ.quant_w_128x128_pow2 if pow2 else OQ.quant_w_128x128
    dgrad = F.fp8_gemm_blockscaled_pow2_dgrad if pow2 else F.fp8_gemm_blockscaled_dgrad
    aq, sa = qa(a)
    wq, sw = qw(wd)                                             # W[R][N], 128x128 blocks
    args = (u8_dev(aq), f32_dev(sa), u8_dev(OQ.transpose_payload(wq)), f32_dev(sw))
    y32 = dgrad(*args, out_dtype=torch.float32)
    y16 = dgrad(*args, out_dtype=torch.bfloat16)
    _check(y32, y16, OG.gemm_dgrad(aq[ROWS], sa[ROWS], wq, sw), f"dgrad pow2={pow2}")


@pytest.mark.parametrize("pow2", [False, True])
def test_bigtile_blockscaled_wgrad(data, pow2):
    a, b, _ = data
    qa = OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128
    wgrad = F.fp8_gemm_blockscaled_pow2_wgrad if pow2 else F.fp8_gemm_blockscaled_wgrad
    aq, sa = qa(a[:NW])                                         # dY^T rows, 128-token groups
    bq, sb = qa(b)                                              # X^T rows, 128-token groups
    dw = wgrad(u8_dev(aq), f32_dev(sa), u8_dev(bq), f32_dev(sb))
    ref = OG.gemm_wgrad(aq[ROWS_W], sa[ROWS_W], bq, sb)
    rows = torch.from_numpy(ROWS_W).to(dev())
    assert_gemm_close(host(dw[rows]), ref, f"wgrad pow2={pow2}")
    # accumulate mode adds onto what the output holds
    dw2 = wgrad(u8_dev(aq), f32_dev(sa), u8_dev(bq), f32_dev(sb), dw=dw.clone(), accumulate=True)
    assert_gemm_close(host(dw2[rows]), 2.0 * ref, f"wgrad accumulate pow2={pow2}")


def test_bigtile_mxfp8(data):
    a, b, wd = data
    aq, ea = OQ.quant_mx_1x32(a)
    bq, eb = OQ.quant_mx_1x32(b)
    A = (u8_dev(aq), _e8m0_dev(ea))
    y32 = F.fp8_gemm_mxfp8_fwd(*A, u8_dev(bq), _e8m0_dev(eb), out_dtype=torch.float32)
    y16 = F.fp8_gemm_mxfp8_fwd(*A, u8_dev(bq), _e8m0_dev(eb), out_dtype=torch.bfloat16)
    _check(y32, y16, OG.gemm_mx_fwd(aq[ROWS], ea[ROWS], bq, eb), "mx fwd")
    wqt, ewt = OQ.quant_mx_32x1(wd)                             # W[R][N] -> Wt[N][R], 32-row groups
    x32 = F.fp8_gemm_mxfp8_dgrad(*A, u8_dev(wqt), _e8m0_dev(ewt), out_dtype=torch.float32)
    x16 = F.fp8_gemm_mxfp8_dgrad(*A, u8_dev(wqt), _e8m0_dev(ewt), out_dtype=torch.bfloat16)
    _check(x32, x16, OG.gemm_mx_dgrad(aq[ROWS], ea[ROWS], wqt, ewt), "mx dgrad")
    dw = F.fp8_gemm_mxfp8_wgrad(*A, u8_dev(bq), _e8m0_dev(eb))
    assert_gemm_close(host(dw[torch.from_numpy(ROWS).to(dev())]), OG.gemm_mx_wgrad(aq[ROWS], ea[ROWS], bq, eb),
                      "mx wgrad")


def _codes_dev(shape, gen):
    """Random E4M3 codes on the GPU, NaN codes (0x7F, 0xFF) replaced by 0x7E / 0xFE."""
    c = torch.randint(0, 256, shape, dtype=torch.int32, device=dev(), generator=gen)
    c = torch.where((c & 0x7F) == 0x7F, c - 1, c)
    return c.to(torch.uint8)


@pytest.mark.parametrize("nkb", [1024, 1032])
def test_bigtile_longest_reduction(nkb):
    """Forward GEMM 4096 x 4096 with K = 128 nkb: 1024 K blocks fill the per-tile table of B's
    block scales (its maximum), 1032 take the per-K-block scale loads instead. Operands are
    random E4M3 codes and scales made on the GPU; the oracle recomputes sampled rows against
    two whole 128-row weight blocks."""
    M = N = 4096
    K = 128 * nkb
    gen = torch.Generator(device=dev())
    gen.manual_seed(12000 + nkb)
    xq = _codes_dev((M, K), gen)
    wq = _codes_dev((N, K), gen)
    sx = torch.rand((M, nkb), device=dev(), generator=gen) * 2.0 ** -12 + 2.0 ** -14
    sw = torch.rand((N // 128, nkb), device=dev(), generator=gen) * 2.0 ** -12 + 2.0 ** -14
    y = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    rows = torch.tensor([0, 1, 255, 256, 2047, 4095], device=dev())
    blocks = [0, 31]
    wrows = torch.cat([torch.arange(b * 128, (b + 1) * 128, device=dev()) for b in blocks])
    ref = OG.gemm_fwd(host(xq[rows]), host(sx[rows]), host(wq[wrows]), host(sw[torch.tensor(blocks, device=dev())]))
    got = host(y[rows][:, wrows])
    assert_gemm_close(got, ref, f"fwd K blocks {nkb}")
