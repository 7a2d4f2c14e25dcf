"""GPU parity at the workloads' full sizes, in the launch configurations the benchmark
times. The GPU runs every call on the whole tensors; the oracle recomputes sampled
outputs on its own (quantization is group-local, so sampled rows, columns and 128x128
blocks need only their own inputs). Quantized bytes and scales: bit-exact. GEMMs: max
error <= 2e-3 x RMS of the sampled reference outputs (bf16 outputs also within half a
bf16 ulp)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import gemm as OG
from oracle import quantize as OQ
from oracle import weight_sync as OS
import workloads as W
from gpu_util import assert_bytes_equal, assert_gemm_close, dev, host

pytestmark = pytest.mark.gpu


def _sample(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=k, replace=False))


def _rows_of(t: torch.Tensor, idx):
    return t[torch.from_numpy(idx).to(t.device)]


@pytest.fixture(scope="module")
def dense():
    d = W.dense_forward(with_down=True)
    return d, {k: W.to_bf16_tensor(v).to(dev()) for k, v in d.items()}


def _check_linear(x, w, xq, sx, wq, sw, y16, rows, blocks, what):
    """Quantized bytes of sampled X rows / W blocks, and Y on rows x (those W blocks)."""
    rxq, rsx = OQ.quant_act_1x128(x[rows])
    assert_bytes_equal(_rows_of(xq, rows), rxq, f"{what} xq rows")
    assert_bytes_equal(_rows_of(sx, rows), rsx, f"{what} sx rows")
    wrows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    rwq, rsw = OQ.quant_w_128x128(w[wrows])
    assert_bytes_equal(_rows_of(wq, wrows), rwq, f"{what} wq blocks")
    assert_bytes_equal(_rows_of(sw, np.array(blocks)), rsw, f"{what} sw blocks")
    ref = OG.gemm_fwd(rxq, rsx, rwq, rsw)
    got16 = host(_rows_of(y16, rows))[:, wrows]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(got16.astype(np.float64)))[1] - 9)
    assert np.all(np.abs(got16 - ref) <= 2e-3 * rms + half_ulp), f"{what}: bf16 output outside tolerance"
    return ref, wrows


def test_dense_forward_full_size(dense):
    d, t = dense
    xq, sx, xqt, sxt = F.fp8_quant_act_1x128(t["x"], rowwise=True, colwise=True)
    wq, sw, _ = F.fp8_quant_w_128x128(t["w_gu"])
    y = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    y32 = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    M, K = d["x"].shape
    rows = _sample(M, 24, 1)
    blocks = sorted(_sample(d["w_gu"].shape[0] // 128, 3, 2).tolist())
    ref, wrows = _check_linear(d["x"], d["w_gu"], xq, sx, wq, sw, y, rows, blocks, "gate/up")
    assert_gemm_close(host(_rows_of(y32, rows))[:, wrows], ref, "gate/up f32")
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    # column-wise copy of X (the WGrad operand): sampled columns over all tokens
    cols = _sample(K, 12, 3)
    rqt, rst = OQ.quant_act_1x128(np.ascontiguousarray(d["x"][:, cols].T))
    assert_bytes_equal(_rows_of(xqt, cols), rqt, "xqt columns")
    assert_bytes_equal(_rows_of(sxt, cols), rst, "sxt columns")


def test_dense_forward_pow2_full_size(dense):
    """The gate/up layer with power-of-two block scales (the scaled MFMA applies them): the
    pow2 quantizers' bytes and scales on sampled rows and weight blocks, and Y on those rows
    against every column of the sampled weight blocks."""
    d, t = dense
    xq, sx, _, _ = F.fp8_quant_act_1x128_pow2(t["x"])
    wq, sw, _ = F.fp8_quant_w_128x128_pow2(t["w_gu"])
    y32 = F.fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    y16 = F.fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    rows = _sample(d["x"].shape[0], 16, 11)
    blocks = sorted(_sample(d["w_gu"].shape[0] // 128, 3, 12).tolist())
    rxq, rsx = OQ.quant_act_1x128_pow2(d["x"][rows])
    assert_bytes_equal(_rows_of(xq, rows), rxq, "pow2 xq rows")
    assert_bytes_equal(_rows_of(sx, rows), rsx, "pow2 sx rows")
    wrows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    rwq, rsw = OQ.quant_w_128x128_pow2(d["w_gu"][wrows])
    assert_bytes_equal(_rows_of(wq, wrows), rwq, "pow2 wq blocks")
    assert_bytes_equal(_rows_of(sw, np.array(blocks)), rsw, "pow2 sw blocks")
    ref = OG.gemm_fwd(rxq, rsx, rwq, rsw)
    assert_gemm_close(host(_rows_of(y32, rows))[:, wrows], ref, "pow2 gate/up f32")
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


def test_dense_down_projection_full_size(dense):
    d, t = dense
    x2q, sx2, _, _ = F.fp8_quant_act_1x128(t["x2"])
    wq, sw, _ = F.fp8_quant_w_128x128(t["w_dn"])
    y = F.fp8_gemm_blockscaled_fwd(x2q, sx2, wq, sw, out_dtype=torch.bfloat16)
    rows = _sample(d["x2"].shape[0], 16, 4)
    blocks = sorted(_sample(d["w_dn"].shape[0] // 128, 3, 5).tolist())
    _check_linear(d["x2"], d["w_dn"], x2q, sx2, wq, sw, y, rows, blocks, "down")


def test_dense_backward_full_size(dense):
    d, t = dense
    dy_np = W.dense_backward()["dy"]
    dy = W.to_bf16_tensor(dy_np).to(dev())
    M, N = dy_np.shape
    K = d["x"].shape[1]
    dyq, sdy, dyqt, sdyt = F.fp8_quant_act_1x128(dy, rowwise=True, colwise=True)
    _, _, xqt, sxt = F.fp8_quant_act_1x128(t["x"], rowwise=False, colwise=True)
    wq, sw, wqt = F.fp8_quant_w_128x128(t["w_gu"], transpose=True)
    dx = F.fp8_gemm_blockscaled_dgrad(dyq, sdy, wqt, sw, out_dtype=torch.bfloat16)
    dw = F.fp8_gemm_blockscaled_wgrad(dyqt, sdyt, xqt, sxt)
    # DGrad: sampled dX rows x sampled 128-column blocks of K; needs W[:, block] for all N
    rows = _sample(M, 12, 6)
    kblocks = sorted(_sample(K // 128, 2, 7).tolist())
    kcols = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in kblocks])
    rdyq, rsdy = OQ.quant_act_1x128(dy_np[rows])
    assert_bytes_equal(_rows_of(dyq, rows), rdyq, "dyq rows")
    wsub = np.ascontiguousarray(d["w_gu"][:, kcols])
    rwq, rsw = OQ.quant_w_128x128(wsub)
    ref = OG.gemm_dgrad(rdyq, rsdy, rwq, rsw)
    got = host(_rows_of(dx, rows))[:, kcols]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(got.astype(np.float64)))[1] - 9)
    assert np.all(np.abs(got - ref) <= 2e-3 * rms + half_ulp), "dgrad outside tolerance"
    assert_bytes_equal(_rows_of(wqt, kcols), OQ.transpose_payload(rwq), "wqt columns")
    # WGrad: dW[n, k] for sampled n and k: column-wise groups of dY and X over all tokens
    ns, ks = _sample(N, 10, 8), _sample(K, 10, 9)
    rdyqt, rsdyt = OQ.quant_act_1x128(np.ascontiguousarray(dy_np[:, ns].T))
    rxqt, rsxt = OQ.quant_act_1x128(np.ascontiguousarray(d["x"][:, ks].T))
    assert_bytes_equal(_rows_of(dyqt, ns), rdyqt, "dyqt columns")
    ref = OG.gemm_wgrad(rdyqt, rsdyt, rxqt, rsxt)
    assert_gemm_close(host(_rows_of(dw, ns))[:, ks], ref, "wgrad")


def test_dense_backward_pow2_full_size(dense):
    """The backward_pow2 workload: power-of-two 1x128 / 128x1 / 128x128 scales, DGrad and
    WGrad with the scales applied by the MFMA, on sampled outputs."""
    d, t = dense
    dy_np = W.dense_backward()["dy"]
    dy = W.to_bf16_tensor(dy_np).to(dev())
    M, N = dy_np.shape
    K = d["x"].shape[1]
    dyq, sdy, dyqt, sdyt = F.fp8_quant_act_1x128_pow2(dy, rowwise=True, colwise=True)
    _, _, xqt, sxt = F.fp8_quant_act_1x128_pow2(t["x"], rowwise=False, colwise=True)
    wq, sw, wqt = F.fp8_quant_w_128x128_pow2(t["w_gu"], transpose=True)
    dx = F.fp8_gemm_blockscaled_pow2_dgrad(dyq, sdy, wqt, sw, out_dtype=torch.float32)
    dw = F.fp8_gemm_blockscaled_pow2_wgrad(dyqt, sdyt, xqt, sxt)
    rows = _sample(M, 12, 16)
    kblocks = sorted(_sample(K // 128, 2, 17).tolist())
    kcols = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in kblocks])
    rdyq, rsdy = OQ.quant_act_1x128_pow2(dy_np[rows])
    assert_bytes_equal(_rows_of(dyq, rows), rdyq, "pow2 dyq rows")
    assert_bytes_equal(_rows_of(sdy, rows), rsdy, "pow2 sdy rows")
    rwq, rsw = OQ.quant_w_128x128_pow2(np.ascontiguousarray(d["w_gu"][:, kcols]))
    assert_gemm_close(host(_rows_of(dx, rows))[:, kcols], OG.gemm_dgrad(rdyq, rsdy, rwq, rsw), "pow2 dgrad")
    ns, ks = _sample(N, 10, 18), _sample(K, 10, 19)
    rdyqt, rsdyt = OQ.quant_act_1x128_pow2(np.ascontiguousarray(dy_np[:, ns].T))
    rxqt, rsxt = OQ.quant_act_1x128_pow2(np.ascontiguousarray(d["x"][:, ks].T))
    assert_bytes_equal(_rows_of(dyqt, ns), rdyqt, "pow2 dyqt columns")
    assert_bytes_equal(_rows_of(sdyt, ns), rsdyt, "pow2 sdyt columns")
    assert_gemm_close(host(_rows_of(dw, ns))[:, ks], OG.gemm_wgrad(rdyqt, rsdyt, rxqt, rsxt), "pow2 wgrad")


def test_decode_full_size_install_and_naive_control():
    d = W.decode_rollout()
    x = W.to_bf16_tensor(d["x"]).to(dev())
    M, K = d["x"].shape
    rxq, rsx = OQ.quant_act_1x128(d["x"])
    for i, n in enumerate(W.DECODE_N):
        w = d[f"w{n}"]
        wq, sw, _ = F.fp8_quant_w_128x128(W.to_bf16_tensor(w).to(dev()))
        iq, is_ = torch.empty_like(wq), torch.empty_like(sw)
        F.fp8_weight_install(wq, sw, iq, is_)
        y_roll = F.fp8_gemm_blockscaled_fwd(wq=iq, sw=is_, x_bf16=x, out_dtype=torch.bfloat16)
        xq, sx, _, _ = F.fp8_quant_act_1x128(x)
        y_train = F.fp8_gemm_blockscaled_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(iq, wq) and torch.equal(is_.view(torch.int32), sw.view(torch.int32))
        assert torch.equal(y_roll.view(torch.int16), y_train.view(torch.int16))
        blocks = sorted(_sample(n // 128, 3, 10 + i).tolist())
        wrows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
        rwq, rsw = OQ.quant_w_128x128(w[wrows])
        assert_bytes_equal(_rows_of(iq, wrows), rwq, f"installed wq N={n}")
        ref = OG.gemm_fwd(rxq, rsx, rwq, rsw)
        got = host(y_roll)[:, wrows]
        rms = float(np.sqrt(np.mean(ref ** 2)))
        half_ulp = np.ldexp(1.0, np.frexp(np.abs(got.astype(np.float64)))[1] - 9)
        assert np.all(np.abs(got - ref) <= 2e-3 * rms + half_ulp), f"decode N={n} outside tolerance"
        # installed vs trainer weights: mean relative error exactly 0; the naive
        # dequantize -> bf16 -> per-tensor requantize path is not (oracle, sampled blocks)
        assert OS.mean_relative_error(OS.weight_value_block(rwq, rsw),
                                      OS.weight_value_block(host(_rows_of(iq, wrows)), host(_rows_of(is_, np.array(blocks))))) == 0.0
        if n == W.DECODE_N[0]:
            fq, fs = OQ.quant_w_128x128(w)
            nq, ns = OS.naive_resync(fq, fs)
            assert OS.mean_relative_error(OS.weight_value_block(fq, fs), OS.weight_value_tensor(nq, ns)) > 0.0


def test_moe_mxfp8_full_size():
    d = W.moe_mxfp8()
    off = d["offsets"]
    xp = W.to_bf16_tensor(d["x_perm"]).to(dev())
    hh = W.to_bf16_tensor(d["h"]).to(dev())
    xq, sx = F.mxfp8_quant_1x32(xp)
    hq, sh = F.mxfp8_quant_1x32(hh)
    wq_gu, sw_gu = F.mxfp8_quant_1x32(W.to_bf16_tensor(d["w_gu"]).to(dev()))
    wq_dn, sw_dn = F.mxfp8_quant_1x32(W.to_bf16_tensor(d["w_dn"]).to(dev()))
    offd = torch.from_numpy(off).to(dev())
    y_gu = F.fp8_grouped_gemm(xq, sx, wq_gu, sw_gu, offd, out_dtype=torch.bfloat16)
    y_dn = F.fp8_grouped_gemm(hq, sh, wq_dn, sw_dn, offd, out_dtype=torch.float32)
    counts = np.diff(off)
    experts = sorted(set([int(np.argmax(counts)), int(np.argmin(counts))] + _sample(len(counts), 4, 11).tolist()))
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.array([lo, lo + 1, (lo + hi) // 2, hi - 2, hi - 1]).clip(lo, hi - 1))
        for name, xin, q, s, wfull, wq, sw, y, f32 in (
                ("gate/up", d["x_perm"], xq, sx, d["w_gu"], wq_gu, sw_gu, y_gu, False),
                ("down", d["h"], hq, sh, d["w_dn"], wq_dn, sw_dn, y_dn, True)):
            rq, rs = OQ.quant_mx_1x32(xin[rows])
            assert_bytes_equal(_rows_of(q, rows), rq, f"{name} xq rows expert {e}")
            assert_bytes_equal(_rows_of(s, rows), rs, f"{name} e8m0 rows expert {e}")
            rwq, rws = OQ.quant_mx_1x32(wfull[e])
            assert_bytes_equal(wq[e], rwq, f"{name} wq expert {e}")
            ref = OG.dequant_mx(rq, rs) @ OG.dequant_mx(rwq, rws).T
            got = host(_rows_of(y, rows))
            rms = float(np.sqrt(np.mean(ref ** 2)))
            if f32:
                assert_gemm_close(got, ref, f"{name} expert {e}", rms=rms)
            else:
                half_ulp = np.ldexp(1.0, np.frexp(np.abs(got.astype(np.float64)))[1] - 9)
                assert np.all(np.abs(got - ref) <= 2e-3 * rms + half_ulp), f"{name} expert {e} outside tolerance"


def test_moe_block128_full_size():
    """The same MoE layer in the blockwise recipe (bench workload moe_block128): 1x128 row
    groups of the routed rows, each expert's weights in 128x128 blocks (the [E][N][K] stack
    quantized as one [E*N][K] matrix, as the benchmark does)."""
    d = W.moe_mxfp8()
    off = d["offsets"]
    E, N, K = d["w_gu"].shape
    _, N2, K2 = d["w_dn"].shape
    xq, sx, _, _ = F.fp8_quant_act_1x128(W.to_bf16_tensor(d["x_perm"]).to(dev()))
    hq, sh, _, _ = F.fp8_quant_act_1x128(W.to_bf16_tensor(d["h"]).to(dev()))
    wq_gu, sw_gu, _ = F.fp8_quant_w_128x128(W.to_bf16_tensor(d["w_gu"].reshape(E * N, K)).to(dev()))
    wq_dn, sw_dn, _ = F.fp8_quant_w_128x128(W.to_bf16_tensor(d["w_dn"].reshape(E * N2, K2)).to(dev()))
    wq_gu, sw_gu = wq_gu.view(E, N, K), sw_gu.view(E, N // 128, K // 128)
    wq_dn, sw_dn = wq_dn.view(E, N2, K2), sw_dn.view(E, N2 // 128, K2 // 128)
    offd = torch.from_numpy(off).to(dev())
    blk = F.RECIPE_BLOCK128
    y_gu = F.fp8_grouped_gemm(xq, sx, wq_gu, sw_gu, offd, recipe=blk, out_dtype=torch.bfloat16)
    y_dn = F.fp8_grouped_gemm(hq, sh, wq_dn, sw_dn, offd, recipe=blk, out_dtype=torch.float32)
    counts = np.diff(off)
    experts = sorted(set([int(np.argmax(counts)), int(np.argmin(counts))] + _sample(len(counts), 4, 12).tolist()))
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.array([lo, lo + 1, (lo + hi) // 2, hi - 2, hi - 1]).clip(lo, hi - 1))
        for name, xin, q, s, wfull, wq, sw, y, f32 in (
                ("gate/up", d["x_perm"], xq, sx, d["w_gu"], wq_gu, sw_gu, y_gu, False),
                ("down", d["h"], hq, sh, d["w_dn"], wq_dn, sw_dn, y_dn, True)):
            rq, rs = OQ.quant_act_1x128(xin[rows])
            assert_bytes_equal(_rows_of(q, rows), rq, f"{name} xq rows expert {e}")
            assert_bytes_equal(_rows_of(s, rows), rs, f"{name} sx rows expert {e}")
            rwq, rws = OQ.quant_w_128x128(wfull[e])
            assert_bytes_equal(wq[e], rwq, f"{name} wq expert {e}")
            assert_bytes_equal(sw[e], rws, f"{name} sw expert {e}")
            ref = OG.gemm_fwd(rq, rs, rwq, rws)
            got = host(_rows_of(y, rows))
            rms = float(np.sqrt(np.mean(ref ** 2)))
            if f32:
                assert_gemm_close(got, ref, f"{name} expert {e}", rms=rms)
            else:
                half_ulp = np.ldexp(1.0, np.frexp(np.abs(got.astype(np.float64)))[1] - 9)
                assert np.all(np.abs(got - ref) <= 2e-3 * rms + half_ulp), f"{name} expert {e} outside tolerance"


def test_producers_full_size():
    """Fused SwiGLU -> FP8 (GU 8192x24576, rows + cols) and RMSNorm -> FP8 (X 8192x4096, rows
    + cols) as the producers workload runs them; sampled rows (1x128 groups, r) and sampled
    columns (128x1 groups over all rows) against the oracle."""
    from oracle import producers as OP
    d = W.fused_producers()
    gu = W.to_bf16_tensor(d["gu"]).to(dev())
    x = W.to_bf16_tensor(d["x"]).to(dev())
    gamma = W.to_bf16_tensor(d["gamma"]).to(dev())
    M = d["gu"].shape[0]
    hq, hs, hqt, hst = F.fp8_swiglu_quant_1x128(gu, colwise=True)
    xq, xs, xqt, xst, rstd = F.fp8_rmsnorm_quant_1x128(x, gamma, d["eps"], colwise=True)
    rows = _sample(M, 16, 40)
    rq, rs = OP.swiglu_quant_1x128(d["gu"][rows])
    assert_bytes_equal(_rows_of(hq, rows), rq, "swiglu q rows")
    assert_bytes_equal(_rows_of(hs, rows), rs, "swiglu s rows")
    Fh = d["gu"].shape[1] // 2
    cols = _sample(Fh, 6, 41)
    h_cols = OP.swiglu_bf16(np.concatenate([d["gu"][:, cols], d["gu"][:, Fh + cols]], axis=1))
    rqt, rst = OQ.quant_act_128x1(h_cols)
    assert_bytes_equal(_rows_of(hqt, cols), rqt, "swiglu qt columns")
    assert_bytes_equal(_rows_of(hst, cols), rst, "swiglu st columns")
    ry, rr, amb = OP.rmsnorm_bf16(d["x"][rows], d["gamma"], d["eps"])
    assert not amb.any()
    assert_bytes_equal(_rows_of(rstd, rows), rr, "rstd rows")
    rq2, rs2 = OQ.quant_act_1x128(ry)
    assert_bytes_equal(_rows_of(xq, rows), rq2, "rmsnorm q rows")
    assert_bytes_equal(_rows_of(xs, rows), rs2, "rmsnorm s rows")


def test_mx_dense_full_size(dense):
    """The MXFP8 dense gate/up layer as the mx_dense workload runs it: quantized bytes of
    sampled rows / columns and sampled outputs of the forward, DGrad and WGrad GEMMs."""
    d, t = dense
    dy_np = W.dense_backward()["dy"]
    dy = W.to_bf16_tensor(dy_np).to(dev())
    M, K = d["x"].shape
    N = d["w_gu"].shape[0]
    xq, ex, xqt, ext = F.mxfp8_quant_act_1x32(t["x"], colwise=True)
    wq, ew, wqt, ewt = F.mxfp8_quant_act_1x32(t["w_gu"], colwise=True)
    dyq, edy, dyqt, edyt = F.mxfp8_quant_act_1x32(dy, colwise=True)
    y = F.fp8_gemm_mxfp8_fwd(xq, ex, wq, ew, out_dtype=torch.float32)
    dx = F.fp8_gemm_mxfp8_dgrad(dyq, edy, wqt, ewt, out_dtype=torch.float32)
    dw = F.fp8_gemm_mxfp8_wgrad(dyqt, edyt, xqt, ext)
    rows, ns, ks = _sample(M, 8, 42), _sample(N, 8, 43), _sample(K, 8, 44)
    rxq, rex = OQ.quant_mx_1x32(d["x"][rows])
    rwq, rew = OQ.quant_mx_1x32(d["w_gu"][ns])
    assert_bytes_equal(_rows_of(xq, rows), rxq, "mx xq rows")
    assert_bytes_equal(_rows_of(wq, ns), rwq, "mx wq rows")
    assert_gemm_close(host(_rows_of(y, rows))[:, ns], OG.gemm_mx_fwd(rxq, rex, rwq, rew), "mx fwd")
    rdyq, redy = OQ.quant_mx_1x32(dy_np[rows])
    rwqt, rewt = OQ.quant_mx_1x32(np.ascontiguousarray(d["w_gu"][:, ks].T))
    assert_bytes_equal(_rows_of(wqt, ks), rwqt, "mx wqt columns")
    assert_bytes_equal(_rows_of(ewt, ks), rewt, "mx ewt columns")
    assert_gemm_close(host(_rows_of(dx, rows))[:, ks], OG.gemm_mx_dgrad(rdyq, redy, rwqt, rewt), "mx dgrad")
    rdyqt, redyt = OQ.quant_mx_1x32(np.ascontiguousarray(dy_np[:, ns].T))
    rxqt, rext = OQ.quant_mx_1x32(np.ascontiguousarray(d["x"][:, ks].T))
    assert_bytes_equal(_rows_of(dyqt, ns), rdyqt, "mx dyqt columns")
    assert_gemm_close(host(_rows_of(dw, ns))[:, ks], OG.gemm_mx_wgrad(rdyqt, redyt, rxqt, rext), "mx wgrad")


def test_fp8_param_full_size():
    """fp8_param requantization of the gate/up fp32 master (24576x4096, as the fp8_param
    workload builds it): sampled 128x128 blocks, their scales and transposed bytes."""
    from oracle import fp8_param as OP8
    d = W.dense_forward(with_down=False)
    rng = np.random.default_rng(7)
    m32 = (d["w_gu"] + rng.standard_normal(d["w_gu"].shape, dtype=np.float32) * np.float32(1e-6)).astype(np.float32)
    q, s, qt = F.fp8_quant_w_128x128_f32(torch.from_numpy(m32).to(dev()), transpose=True)
    N, K = m32.shape
    for bi in _sample(N // 128, 3, 45):
        rows = np.arange(bi * 128, (bi + 1) * 128)
        rq, rs = OP8.quant_w_128x128_f32(m32[rows])
        assert_bytes_equal(_rows_of(q, rows), rq, f"q block row {bi}")
        assert_bytes_equal(_rows_of(s, np.array([bi])), rs, f"s block row {bi}")
        got_t = host(qt)[:, rows]
        assert np.array_equal(got_t, rq.T), f"qt block row {bi}"
