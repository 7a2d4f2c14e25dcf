"""GPU parity tests (element by element) of every libfp8rl entry point against the CPU
oracle, on seeded inputs that span several tiles, ragged tails and the edge cases of
the method (all-zero groups, signed zeros, subnormal and maximal bf16 values, exact
powers of two at the MX scale boundaries, empty experts). Inputs come from
``workloads``; expected values come only from ``oracle``."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import gemm as OG
from oracle import quantize as OQ
from oracle import weight_sync as OS
from oracle.fp8_formats import decode_e4m3
import workloads as W
from gpu_util import (assert_bf16_consistent, assert_bytes_equal, assert_gemm_close, bf16_dev, dev, f32_dev, host,
                      u8_dev)

pytestmark = pytest.mark.gpu


def _special_rows(K, seed):
    """Rows exercising the quantizer's edge cases, K % 128 == 0."""
    rng = np.random.default_rng(seed)
    rows = []
    z = np.zeros(K, np.float32)
    rows.append(z.copy())                                        # all-zero groups
    r = z.copy(); r[::3] = -0.0; rows.append(r)                   # signed zeros only
    r = (rng.standard_normal(K) * 1e-39).astype(np.float32); rows.append(r)   # bf16 subnormals
    r = np.full(K, 3.3895314e38, np.float32); r[1::2] *= -1; rows.append(r)   # bf16 max magnitude
    r = rng.standard_normal(K).astype(np.float32); r[5] = 9.2e-41; rows.append(r * np.float32(2.0 ** 100))
    r = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -120); rows.append(r)  # tiny scales
    r = rng.standard_normal(K).astype(np.float32); r[::7] = 448.0; r[1::7] = -448.0 * 4; rows.append(r)
    r = (rng.integers(-448, 449, K)).astype(np.float32); rows.append(r)      # integers up to 448
    return W.bf16_round(np.stack(rows))


def _rand(shape, seed, sigma=1.0):
    return W.bf16_round(np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(sigma))


# ------------------------------------------------------------------------------------- quantizers

@pytest.mark.parametrize("M,K", [(256, 512), (37, 384), (1, 128), (1000, 256)])
def test_quant_act_rows(M, K):
    x = _rand((M, K), 1000 + M)
    x[: min(M, 8)] = _special_rows(K, M)[: min(M, 8)]
    q, s, _, _ = F.fp8_quant_act_1x128(bf16_dev(x))
    rq, rs = OQ.quant_act_1x128(x)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(s, rs, "s")


def test_quant_act_rows_tiny_workload():
    x = W.tiny_forward()["x"]
    q, s, _, _ = F.fp8_quant_act_1x128(bf16_dev(x))
    rq, rs = OQ.quant_act_1x128(x)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(s, rs, "s")


@pytest.mark.parametrize("M,K,rows", [(256, 384, True), (384, 256, False), (128, 128, True), (512, 640, True)])
def test_quant_act_rows_and_columns(M, K, rows):
    x = _rand((M, K), 2000 + M + K)
    x[:8] = _special_rows(K, 7)
    x[:, 3] = 0.0                                      # an all-zero column group
    x[200 % M, 5] = 1e30
    x = W.bf16_round(x)
    q, s, qt, st = F.fp8_quant_act_1x128(bf16_dev(x), rowwise=rows, colwise=True)
    rqt, rst = OQ.quant_act_128x1(x)
    assert_bytes_equal(qt, rqt, "qt")
    assert_bytes_equal(st, rst, "st")
    if rows:
        rq, rs = OQ.quant_act_1x128(x)
        assert_bytes_equal(q, rq, "q")
        assert_bytes_equal(s, rs, "s")
    else:
        assert q is None and s is None


def _mixed_regimes(M, K, seed):
    """N(0,1) rows scaled so that groups of one wave take different arithmetic: rows times
    2^-124 (amax near 2^-122: a subnormal fp32 scale, the fp64 form), rows times 2^118 (the
    reciprocal's low part subnormal), the rest unscaled; one column block holds N(0,1) times
    2^-125 in every row, so that its 128x1 groups have subnormal scales too."""
    x = _rand((M, K), seed)
    r = np.arange(M)
    x[r % 7 == 3] *= np.float32(2.0 ** -124)
    x[r % 11 == 5] *= np.float32(2.0 ** 118)
    x[:, 128:256] = _rand((M, 128), seed + 1) * np.float32(2.0 ** -125)
    return W.bf16_round(x)


@pytest.mark.parametrize("pow2", [False, True])
def test_quant_act_mixed_scale_regimes(pow2):
    """Groups of one wave with tiny, ordinary and huge amax side by side, in the row
    kernel, the row + column tile kernel and the column-only form."""
    x = _mixed_regimes(384, 640, 2500)
    assert np.isfinite(x).all()
    quant = F.fp8_quant_act_1x128_pow2 if pow2 else F.fp8_quant_act_1x128
    rows_ref = OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128
    cols_ref = OQ.quant_act_128x1_pow2 if pow2 else OQ.quant_act_128x1
    rq, rs = rows_ref(x)
    rqt, rst = cols_ref(x)
    q, s, _, _ = quant(bf16_dev(x))
    assert_bytes_equal(q, rq, "rows q")
    assert_bytes_equal(s, rs, "rows s")
    q, s, qt, st = quant(bf16_dev(x), rowwise=True, colwise=True)
    assert_bytes_equal(q, rq, "tile q")
    assert_bytes_equal(s, rs, "tile s")
    assert_bytes_equal(qt, rqt, "tile qt")
    assert_bytes_equal(st, rst, "tile st")


def test_mxfp8_quant_mixed_scale_regimes():
    x = _mixed_regimes(200, 512, 2600)
    q, e = F.mxfp8_quant_1x32(bf16_dev(x))
    rq, re = OQ.quant_mx_1x32(x)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(e, re, "e8m0")


@pytest.mark.parametrize("N,K", [(512, 512), (384, 256), (128, 1024)])
def test_quant_w_128x128(N, K):
    w = W.tiny_forward()["w"] if (N, K) == (512, 512) else _rand((N, K), 3000 + N, 0.02)
    w = w.copy()
    w[:128, :128] = 0.0                                # an all-zero block
    w[130 % N, 300 % K] = -3.0e38
    w[200 % N, 5] = 1e-39
    w = W.bf16_round(w)
    q, s, qt = F.fp8_quant_w_128x128(bf16_dev(w), transpose=True)
    rq, rs = OQ.quant_w_128x128(w)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(s, rs, "s")
    assert_bytes_equal(qt, OQ.transpose_payload(rq), "qt")


@pytest.mark.parametrize("R,K", [(100, 256), (7, 32), (64, 2048)])
def test_mxfp8_quant(R, K):
    x = _rand((R, K), 4000 + R)
    if K >= 128:
        x[:8] = _special_rows(K, 9)[:, :K]
        x[9 % R, 0] = 448.0 * 4                        # exactly at a scale boundary
        x[10 % R, 32] = 1800.0                         # the next bf16 above it
    q, e = F.mxfp8_quant_1x32(bf16_dev(x))
    rq, re = OQ.quant_mx_1x32(x)
    assert_bytes_equal(q, rq, "q")
    assert_bytes_equal(e, re, "e8m0")


# ------------------------------------------------------------------------------------- GEMMs

def _quantized_pair(M, N, K, seed, w_sigma=0.02):
    x = _rand((M, K), seed)
    w = _rand((N, K), seed + 1, w_sigma)
    return x, w


@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (300, 384, 640), (1, 128, 128), (17, 256, 384),
                                   (4096, 4096, 256), (777, 1280, 1152)])
def test_fwd(M, N, K):
    x, w = _quantized_pair(M, N, K, 5000 + M)
    xq, sx, _, _ = F.fp8_quant_act_1x128(bf16_dev(x))
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w))
    y32 = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    y16 = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    rxq, rsx = OQ.quant_act_1x128(x)
    rwq, rsw = OQ.quant_w_128x128(w)
    ref = OG.gemm_fwd(rxq, rsx, rwq, rsw)
    assert_gemm_close(host(y32), ref, "fwd f32")
    assert_bf16_consistent(y16, y32, ref, "fwd bf16")


def test_fwd_tiny_workload_and_determinism():
    d = W.tiny_forward()
    xq, sx, _, _ = F.fp8_quant_act_1x128(bf16_dev(d["x"]))
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(d["w"]))
    y1 = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    y2 = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    rxq, rsx = OQ.quant_act_1x128(d["x"])
    rwq, rsw = OQ.quant_w_128x128(d["w"])
    assert_gemm_close(host(y1), OG.gemm_fwd(rxq, rsx, rwq, rsw), "tiny fwd")


def test_fwd_decodes_every_e4m3_code():
    """Y = X . W^T with W one-hot (code 1.0 on the diagonal) and unit scales returns the
    decoded value of every code of X: checks the MFMA's E4M3 decode of all 256 codes
    (NaN codes excluded from the product, checked apart)."""
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    finite = (codes & 0x7F) != 0x7F
    xq = np.where(finite, codes, 0).astype(np.uint8)
    wq = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(wq, 0x38)
    y = F.fp8_gemm_blockscaled_fwd(u8_dev(xq), f32_dev(np.ones((2, 1))), u8_dev(wq), f32_dev(np.ones((1, 1))),
                                   out_dtype=torch.float32)
    got = host(y)
    ref = decode_e4m3(xq)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(got[~finite] == 0)


@pytest.mark.parametrize("M,N,K", [(256, 8320, 256), (100, 4224, 384), (256, 12416, 128), (64, 16640, 256),
                                   (33, 24704, 128), (200, 4224, 512), (130, 8320, 1024), (1, 12416, 2048),
                                   (130, 32768, 128), (90, 12288, 128), (256, 24576, 128), (40, 49152, 128),
                                   (60, 65536, 128)])
def test_fwd_few_rows(M, N, K):
    """M <= 256 runs the few-row kernel: each workgroup takes a part of MR = 64, 128 or 256
    rows and a run of F 16-row weight fragments. These shapes select (MR, F) = (256, 1),
    (256, 3), (256, 8), (128, 3), (128, 6), (128, 8), (128, 12), (64, 4), (64, 6), (64, 8),
    (64, 12) and (64, 16); row parts end inside M (M = 33, 90, 100, 130, 200), N = 8320 and
    16640 leave a last run with fewer fragments, and runs straddle 128-row scale blocks."""
    x, w = _quantized_pair(M, N, K, 5500 + M)
    xq, sx, _, _ = F.fp8_quant_act_1x128(bf16_dev(x))
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w))
    y32 = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    y16 = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    rxq, rsx = OQ.quant_act_1x128(x)
    rwq, rsw = OQ.quant_w_128x128(w)
    ref = OG.gemm_fwd(rxq, rsx, rwq, rsw)
    assert_gemm_close(host(y32), ref, "few-row fwd f32")
    assert_bf16_consistent(y16, y32, ref, "few-row fwd bf16")


@pytest.mark.parametrize("M,N,K", [(256, 4096, 512), (200, 1024, 384)])
def test_fwd_bf16_input_matches_two_step(M, N, K):
    x, w = _quantized_pair(M, N, K, 6000 + M)
    xd = bf16_dev(x)
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w))
    xq, sx, _, _ = F.fp8_quant_act_1x128(xd)
    two = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    fused = F.fp8_gemm_blockscaled_fwd(wq=wq, sw=sw, x_bf16=xd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(two, fused)
    rxq, rsx = OQ.quant_act_1x128(x)
    rwq, rsw = OQ.quant_w_128x128(w)
    assert_gemm_close(host(fused), OG.gemm_fwd(rxq, rsx, rwq, rsw), "fused fwd")


@pytest.mark.parametrize("M,N,K", [(256, 512, 384), (130, 256, 640), (1, 128, 128), (200, 256, 8320)])
def test_dgrad(M, N, K):
    dy = _rand((M, N), 7000 + M, 1e-3)
    w = _rand((N, K), 7001 + M, 0.02)
    dyq, sdy, _, _ = F.fp8_quant_act_1x128(bf16_dev(dy))
    wq, sw, wqt = F.fp8_quant_w_128x128(bf16_dev(w), transpose=True)
    dx32 = F.fp8_gemm_blockscaled_dgrad(dyq, sdy, wqt, sw, out_dtype=torch.float32)
    dx16 = F.fp8_gemm_blockscaled_dgrad(dyq, sdy, wqt, sw, out_dtype=torch.bfloat16)
    rdyq, rsdy = OQ.quant_act_1x128(dy)
    rwq, rsw = OQ.quant_w_128x128(w)
    ref = OG.gemm_dgrad(rdyq, rsdy, rwq, rsw)
    assert_gemm_close(host(dx32), ref, "dgrad f32")
    assert_bf16_consistent(dx16, dx32, ref, "dgrad bf16")


@pytest.mark.parametrize("M,N,K", [(256, 384, 256), (512, 128, 640), (128, 1024, 128)])
def test_wgrad(M, N, K):
    dy = _rand((M, N), 8000 + M, 1e-3)
    x = _rand((M, K), 8001 + M)
    _, _, dyqt, sdyt = F.fp8_quant_act_1x128(bf16_dev(dy), rowwise=False, colwise=True)
    _, _, xqt, sxt = F.fp8_quant_act_1x128(bf16_dev(x), rowwise=False, colwise=True)
    dw = F.fp8_gemm_blockscaled_wgrad(dyqt, sdyt, xqt, sxt)
    rdyqt, rsdyt = OQ.quant_act_128x1(dy)
    rxqt, rsxt = OQ.quant_act_128x1(x)
    ref = OG.gemm_wgrad(rdyqt, rsdyt, rxqt, rsxt)
    assert_gemm_close(host(dw), ref, "wgrad")
    base = torch.full_like(dw, 0.5)
    acc = F.fp8_gemm_blockscaled_wgrad(dyqt, sdyt, xqt, sxt, dw=base.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(acc, dw + 0.5)            # one fp32 add of the same product


def _routing(T_tokens, E, topk, seed):
    perm, offsets = W.zipf_topk_routing(T_tokens, E, topk, 1.1, np.random.default_rng(seed))
    return perm, offsets


@pytest.mark.parametrize("T_tokens,E,topk,N,K", [(200, 8, 2, 256, 256), (64, 16, 4, 128, 384), (300, 1, 1, 64, 128),
                                                 (256, 8, 4, 384, 1024)])
def test_grouped_mx(T_tokens, E, topk, N, K):
    perm, offsets = _routing(T_tokens, E, topk, 9000 + E)
    x = _rand((T_tokens, K), 9001 + E)[perm]
    w = _rand((E, N, K), 9002 + E, 0.02)
    xq, sx = F.mxfp8_quant_1x32(bf16_dev(x))
    wq, sw = F.mxfp8_quant_1x32(bf16_dev(w))
    off = torch.from_numpy(offsets).to(dev())
    y32 = F.fp8_grouped_gemm(xq, sx, wq, sw, off, out_dtype=torch.float32)
    y16 = F.fp8_grouped_gemm(xq, sx, wq, sw, off, out_dtype=torch.bfloat16)
    rxq, rsx = OQ.quant_mx_1x32(x)
    rwq, rsw = OQ.quant_mx_1x32(w.reshape(E * N, K))
    ref = OG.grouped_gemm_mx(rxq, rsx, rwq.reshape(E, N, K), rsw.reshape(E, N, K // 32), offsets)
    assert_gemm_close(host(y32), ref, "grouped f32")
    assert_bf16_consistent(y16, y32, ref, "grouped bf16")


def test_grouped_mx_empty_experts_and_malformed_offsets():
    E, N, K = 6, 128, 256
    x = _rand((100, K), 9100)
    w = _rand((E, N, K), 9101, 0.02)
    xq, sx = F.mxfp8_quant_1x32(bf16_dev(x))
    wq, sw = F.mxfp8_quant_1x32(bf16_dev(w))
    rxq, rsx = OQ.quant_mx_1x32(x)
    rwq, rsw = OQ.quant_mx_1x32(w.reshape(E * N, K))
    rwq, rsw = rwq.reshape(E, N, K), rsw.reshape(E, N, K // 32)
    good = np.array([0, 0, 40, 40, 41, 100, 100], np.int32)          # empty experts 0, 2, 5
    y = F.fp8_grouped_gemm(xq, sx, wq, sw, torch.from_numpy(good).to(dev()), out_dtype=torch.float32)
    assert_gemm_close(host(y), OG.grouped_gemm_mx(rxq, rsx, rwq, rsw, good), "grouped empty experts")
    # offsets outside [0, T] and a decreasing step: clamped, never out of bounds. After
    # clamping: expert 1 owns rows [0, 60), expert 3 rows [60, 100), the others are empty
    # (the last step 5000 -> -3 clamps to 100 -> 0, an empty expert).
    bad = np.array([-50, 0, 60, 60, 5000, 5000, -3], np.int32)
    y = F.fp8_grouped_gemm(xq, sx, wq, sw, torch.from_numpy(bad).to(dev()), out_dtype=torch.float32)
    got = host(y)
    ref1 = OG.dequant_mx(rxq[:60], rsx[:60]) @ OG.dequant_mx(rwq[1], rsw[1]).T
    ref3 = OG.dequant_mx(rxq[60:], rsx[60:]) @ OG.dequant_mx(rwq[3], rsw[3]).T
    assert_gemm_close(got[:60], ref1, "grouped clamped expert 1")
    assert_gemm_close(got[60:], ref3, "grouped clamped expert 3")


@pytest.mark.parametrize("T_tokens,E,topk,N,K", [(200, 8, 2, 256, 256), (64, 16, 4, 128, 384), (300, 1, 1, 128, 2048),
                                                 (256, 8, 4, 384, 1024), (500, 4, 2, 640, 3072)])
def test_grouped_block(T_tokens, E, topk, N, K):
    """Blockwise grouped GEMM: 1x128 row scales (through the LDS ring when K / 128 is a
    multiple of 8: K = 1024, 2048, 3072; per K block otherwise) and each expert's 128x128
    block scales, on Zipf-routed ragged experts. Operands are the oracle's quantization."""
    perm, offsets = _routing(T_tokens, E, topk, 9200 + E)
    x = _rand((T_tokens, K), 9201 + E)[perm]
    w = _rand((E, N, K), 9202 + E, 0.02)
    rxq, rsx = OQ.quant_act_1x128(x)
    rwq, rsw = OQ.quant_w_128x128(w.reshape(E * N, K))
    rwq, rsw = rwq.reshape(E, N, K), rsw.reshape(E, N // 128, K // 128)
    args = (u8_dev(rxq), f32_dev(rsx), u8_dev(rwq), f32_dev(rsw), torch.from_numpy(offsets).to(dev()))
    y32 = F.fp8_grouped_gemm(*args, recipe=F.RECIPE_BLOCK128, out_dtype=torch.float32)
    y16 = F.fp8_grouped_gemm(*args, recipe=F.RECIPE_BLOCK128, out_dtype=torch.bfloat16)
    ref = OG.grouped_gemm_block(rxq, rsx, rwq, rsw, offsets)
    assert_gemm_close(host(y32), ref, "grouped block f32")
    assert_bf16_consistent(y16, y32, ref, "grouped block bf16")


@pytest.mark.parametrize("E,recipe", [(150, "mx"), (150, "block"), (129, "mx")])
def test_grouped_many_experts(E, recipe):
    """More experts than one 64-lane step of the tile search (three steps for E = 129 and
    150), many of them empty, rows ragged: every routed row must land on its own expert."""
    T_tokens, topk, N, K = 300, 2, 128, 256
    perm, offsets = _routing(T_tokens, E, topk, 9400 + E)
    assert np.sum(np.diff(offsets) == 0) > 0 and offsets[-1] == T_tokens * topk
    x = _rand((T_tokens, K), 9401 + E)[perm]
    w = _rand((E, N, K), 9402 + E, 0.02)
    off = torch.from_numpy(offsets).to(dev())
    if recipe == "mx":
        rxq, rsx = OQ.quant_mx_1x32(x)
        rwq, rsw = OQ.quant_mx_1x32(w.reshape(E * N, K))
        rwq, rsw = rwq.reshape(E, N, K), rsw.reshape(E, N, K // 32)
        args = (u8_dev(rxq), u8_dev(rsx), u8_dev(rwq), u8_dev(rsw), off)
        y = F.fp8_grouped_gemm(*args, recipe=F.RECIPE_MXFP8, out_dtype=torch.float32)
        ref = OG.grouped_gemm_mx(rxq, rsx, rwq, rsw, offsets)
    else:
        rxq, rsx = OQ.quant_act_1x128(x)
        rwq, rsw = OQ.quant_w_128x128(w.reshape(E * N, K))
        rwq, rsw = rwq.reshape(E, N, K), rsw.reshape(E, N // 128, K // 128)
        args = (u8_dev(rxq), f32_dev(rsx), u8_dev(rwq), f32_dev(rsw), off)
        y = F.fp8_grouped_gemm(*args, recipe=F.RECIPE_BLOCK128, out_dtype=torch.float32)
        ref = OG.grouped_gemm_block(rxq, rsx, rwq, rsw, offsets)
    assert_gemm_close(host(y), ref, f"grouped E={E} {recipe}")


def test_grouped_block_empty_experts_and_gpu_quantizers():
    """Empty experts, and operands from the library's own quantizers (whose bytes and scales
    equal the oracle's): the weight stack [E][N][K] quantized as one [E*N][K] matrix gives
    each expert's 128x128 blocks."""
    E, N, K = 6, 256, 1024
    x = _rand((100, K), 9300)
    w = _rand((E, N, K), 9301, 0.02)
    xq, sx, _, _ = F.fp8_quant_act_1x128(bf16_dev(x))
    wq, sw, _ = F.fp8_quant_w_128x128(bf16_dev(w.reshape(E * N, K)))
    good = np.array([0, 0, 40, 40, 41, 100, 100], np.int32)          # empty experts 0, 2, 5
    y = F.fp8_grouped_gemm(xq, sx, wq.view(E, N, K), sw.view(E, N // 128, K // 128), torch.from_numpy(good).to(dev()),
                           recipe=F.RECIPE_BLOCK128, out_dtype=torch.float32)
    rxq, rsx = OQ.quant_act_1x128(x)
    rwq, rsw = OQ.quant_w_128x128(w.reshape(E * N, K))
    ref = OG.grouped_gemm_block(rxq, rsx, rwq.reshape(E, N, K), rsw.reshape(E, N // 128, K // 128), good)
    assert_gemm_close(host(y), ref, "grouped block empty experts")


# ------------------------------------------------------------------------------------- weight sync

def test_install_bit_identity_and_naive_control():
    d = W.tiny_forward()
    xd, wd = bf16_dev(d["x"]), bf16_dev(d["w"])
    # trainer side
    wq, sw, _ = F.fp8_quant_w_128x128(wd)
    xq, sx, _, _ = F.fp8_quant_act_1x128(xd)
    y_train = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    # rollout side: install payload + scales into its own buffers, no quantizer
    dq = torch.empty_like(wq)
    ds = torch.empty_like(sw)
    F.fp8_weight_install(wq, sw, dq, ds)
    y_roll = F.fp8_gemm_blockscaled_fwd(xq, sx, dq, ds, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dq, wq) and torch.equal(ds.view(torch.int32), sw.view(torch.int32))
    assert torch.equal(y_train.view(torch.int16), y_roll.view(torch.int16))
    rwq, rsw = OQ.quant_w_128x128(d["w"])
    assert OS.mean_relative_error(OS.weight_value_block(rwq, rsw),
                                  OS.weight_value_block(host(dq), host(ds))) == 0.0
    # naive path (oracle: dequantize -> bf16 -> per-tensor requantize), run through the GPU GEMM
    nq, ns = OS.naive_resync(rwq, rsw)
    rel = OS.mean_relative_error(OS.weight_value_block(rwq, rsw), OS.weight_value_tensor(nq, ns))
    assert rel > 0.0
    ns_grid = np.full(rsw.shape, ns, np.float32)
    y_naive = F.fp8_gemm_blockscaled_fwd(xq, sx, u8_dev(nq), f32_dev(ns_grid), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert not torch.equal(y_naive.view(torch.int16), y_train.view(torch.int16))


def test_install_mx_and_multi_block():
    w = _rand((3 * 64, 256), 9200, 0.02)
    q, e = F.mxfp8_quant_1x32(bf16_dev(w))
    dq, de = torch.empty_like(q), torch.empty_like(e)
    F.fp8_weight_install(q, e, dq, de, recipe=F.RECIPE_MXFP8)
    torch.cuda.synchronize()
    assert torch.equal(dq, q) and torch.equal(de, e)
    big = _rand((1024, 2048), 9201, 0.02)
    q, s, _ = F.fp8_quant_w_128x128(bf16_dev(big))
    dq, ds = torch.empty_like(q), torch.empty_like(s)
    F.fp8_weight_install(q, s, dq, ds)
    torch.cuda.synchronize()
    assert torch.equal(dq, q) and torch.equal(ds, s)
