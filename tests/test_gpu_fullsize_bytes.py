"""Every quantized byte and scale at the workloads' full sizes, against the oracle: the
dense layer's X (rows and 128x1 columns), X2, W_gu (with its byte transpose) and W_dn, in
both scale recipes; the backward pass's dY (rows and columns); the fused producers' outputs
(SwiGLU and RMSNorm, rows, columns and r); the MoE layer's routed rows, H and both expert
stacks (MXFP8); the MXFP8 dense layer's X and W. The GPU quantizes each whole tensor in one
call, as the benchmark does; the oracle recomputes it in 128-row-aligned chunks in a process
pool (identical results: every quantizer is local to 128-row blocks)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
import workloads as W
from oracle import producers as OP
from oracle import quantize as OQ
from oracle_pool import map_rows, rows_then_cols
from gpu_util import assert_bytes_equal, dev

pytestmark = pytest.mark.gpu


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _eq(gpu, ref, what):
    g = _np(gpu) if isinstance(gpu, torch.Tensor) else gpu
    ref = np.asarray(ref)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    if g.dtype == np.float32:
        g, ref = g.view(np.uint32), np.asarray(ref, np.float32).view(np.uint32)
    bad = int(np.count_nonzero(g != ref))
    assert bad == 0, f"{what}: {bad} of {g.size} differ"


def _act_rows_cols(x, pow2=False):
    rows_fn = OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128
    cols_fn = OQ.quant_act_128x1_pow2 if pow2 else OQ.quant_act_128x1
    q, s = rows_then_cols(map_rows(rows_fn, x), 2, 0)
    qt, st = rows_then_cols(map_rows(cols_fn, x), 0, 2)
    return q, s, qt, st


def _check_act(x, pow2, what, colwise=True):
    quant = F.fp8_quant_act_1x128_pow2 if pow2 else F.fp8_quant_act_1x128
    q, s, qt, st = quant(W.to_bf16_tensor(x).to(dev()), rowwise=True, colwise=colwise)
    if colwise:
        rq, rs, rqt, rst = _act_rows_cols(x, pow2)
        _eq(qt, rqt, f"{what} qt")
        _eq(st, rst, f"{what} st")
    else:
        rq, rs = rows_then_cols(map_rows(OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128, x), 2, 0)
    _eq(q, rq, f"{what} q")
    _eq(s, rs, f"{what} s")


def _check_w(w, pow2, what, transpose):
    quant = F.fp8_quant_w_128x128_pow2 if pow2 else F.fp8_quant_w_128x128
    q, s, qt = quant(W.to_bf16_tensor(w).to(dev()), transpose=transpose)
    rq, rs = rows_then_cols(map_rows(OQ.quant_w_128x128_pow2 if pow2 else OQ.quant_w_128x128, w), 2, 0)
    _eq(q, rq, f"{what} q")
    _eq(s, rs, f"{what} s")
    if transpose:
        _eq(qt, OQ.transpose_payload(rq), f"{what} qt")


@pytest.fixture(scope="module")
def dense():
    return W.dense_forward(with_down=True)


@pytest.mark.parametrize("pow2", [False, True])
def test_dense_activations_all_bytes(dense, pow2):
    _check_act(dense["x"], pow2, f"X 8192x4096 pow2={pow2}")
    _check_act(dense["x2"], pow2, f"X2 8192x12288 pow2={pow2}", colwise=False)


@pytest.mark.parametrize("pow2", [False, True])
def test_dense_weights_all_bytes(dense, pow2):
    _check_w(dense["w_gu"], pow2, f"W_gu 24576x4096 pow2={pow2}", transpose=True)
    _check_w(dense["w_dn"], pow2, f"W_dn 4096x12288 pow2={pow2}", transpose=False)


def test_backward_dy_all_bytes():
    _check_act(W.dense_backward()["dy"], False, "dY 8192x24576")


def test_producers_all_bytes():
    d = W.fused_producers()
    gu = W.to_bf16_tensor(d["gu"]).to(dev())
    q, s, qt, st = F.fp8_swiglu_quant_1x128(gu, rowwise=True, colwise=True)
    rq, rs, rqt, rst = rows_then_cols(map_rows(OP.swiglu_quant_1x128, d["gu"], colwise=True), 2, 2)
    for g, r, name in ((q, rq, "q"), (s, rs, "s"), (qt, rqt, "qt"), (st, rst, "st")):
        _eq(g, r, f"SwiGLU 8192x12288 {name}")
    del gu, q, s, qt, st
    x = W.to_bf16_tensor(d["x"]).to(dev())
    gamma = W.to_bf16_tensor(d["gamma"]).to(dev())
    q, s, qt, st, r = F.fp8_rmsnorm_quant_1x128(x, gamma, d["eps"], rowwise=True, colwise=True)
    parts = map_rows(OP.rmsnorm_quant_1x128, d["x"], d["gamma"], d["eps"], colwise=True)
    assert not any(np.any(p[5]) for p in parts), "a row's r lies at an fp32 rounding tie"
    rq, rs, rqt, rst = rows_then_cols([p[:4] for p in parts], 2, 2)
    rr = np.concatenate([p[4] for p in parts])
    for g, ref, name in ((q, rq, "q"), (s, rs, "s"), (qt, rqt, "qt"), (st, rst, "st"), (r, rr, "r")):
        _eq(g, ref, f"RMSNorm 8192x4096 {name}")


def test_moe_all_bytes():
    d = W.moe_mxfp8()
    for name, a in (("X_perm", d["x_perm"]), ("H", d["h"]),
                    ("W_gu experts", d["w_gu"].reshape(-1, d["w_gu"].shape[2])),
                    ("W_dn experts", d["w_dn"].reshape(-1, d["w_dn"].shape[2]))):
        q, e = F.mxfp8_quant_1x32(W.to_bf16_tensor(a).to(dev()))
        rq, re = rows_then_cols(map_rows(OQ.quant_mx_1x32, a), 2, 0)
        _eq(q, rq, f"MXFP8 {name} {a.shape} q")
        _eq(e, re, f"MXFP8 {name} {a.shape} e8m0")


def test_mx_dense_all_bytes(dense):
    x = dense["x"]
    q, e, qt, et = F.mxfp8_quant_act_1x32(W.to_bf16_tensor(x).to(dev()), rowwise=True, colwise=True)
    rq, re = rows_then_cols(map_rows(OQ.quant_mx_1x32, x), 2, 0)
    rqt, ret = rows_then_cols(map_rows(OQ.quant_mx_32x1, x), 0, 2)
    for g, r, name in ((q, rq, "q"), (e, re, "e8m0"), (qt, rqt, "qt"), (et, ret, "e8m0t")):
        _eq(g, r, f"MXFP8 X 8192x4096 {name}")
