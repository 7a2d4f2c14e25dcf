"""The chunked oracle of the full-size byte comparisons equals the whole-tensor oracle:
every function it is used with, on chunks of 128 rows, against one call on the whole
array (a 128-row-aligned split leaves each 1x128, 1x32, 128x128, 128x1 and 32x1 group and
each producer row whole)."""

import numpy as np
import pytest

import workloads as W
from oracle import producers as OP
from oracle import quantize as OQ
from oracle_pool import map_rows, rows_then_cols


def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("fn,n_rows,n_cols", [
    (OQ.quant_act_1x128, 2, 0), (OQ.quant_act_128x1, 0, 2), (OQ.quant_act_1x128_pow2, 2, 0),
    (OQ.quant_act_128x1_pow2, 0, 2), (OQ.quant_w_128x128, 2, 0), (OQ.quant_w_128x128_pow2, 2, 0),
    (OQ.quant_mx_1x32, 2, 0), (OQ.quant_mx_32x1, 0, 2)])
def test_chunked_quantizers_equal_whole(fn, n_rows, n_cols):
    x = W.normal_bf16((512, 256), 1.0, 91, 1)
    x[300, 17] = 40.0                                  # one group with a large amax
    whole = fn(x)
    parts = rows_then_cols(map_rows(fn, x, chunk_rows=128), n_rows, n_cols)
    for a, b in zip(parts, whole):
        _same(a, b)


def test_chunked_producers_equal_whole():
    gu = W.normal_bf16((256, 512), 1.0, 92, 1)
    whole = OP.swiglu_quant_1x128(gu, colwise=True)
    for a, b in zip(rows_then_cols(map_rows(OP.swiglu_quant_1x128, gu, chunk_rows=128, colwise=True), 2, 2), whole):
        _same(a, b)
    x = W.normal_bf16((256, 256), 1.0, 93, 1)
    gamma = W.normal_bf16((256,), 0.1, 93, 2) + np.float32(1.0)
    whole = OP.rmsnorm_quant_1x128(x, W.bf16_round(gamma), 1e-6, colwise=True)
    parts = map_rows(OP.rmsnorm_quant_1x128, x, W.bf16_round(gamma), 1e-6, chunk_rows=128, colwise=True)
    for a, b in zip(rows_then_cols([p[:4] for p in parts], 2, 2), whole[:4]):
        _same(a, b)
    _same(np.concatenate([p[4] for p in parts]), whole[4])
