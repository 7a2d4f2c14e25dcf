"""Pins for the oracle's block-scaled GEMMs: an exact-rational triple loop that
decodes codes with torch (a library routine) and looks each scale up by explicit
index arithmetic; it catches a transposed operand, a wrong scale index or block
size, and a dropped term. Plus structural identities of the grouped GEMM."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm as G

_DEC = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
_DEC_FR = [Fraction(float(v)) if np.isfinite(v) else None for v in _DEC]


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)   # no NaN codes


def _scales(rng, shape):
    # fp32 scales spread over many binades, with full mantissas
    return (rng.random(shape) * 2.0 ** rng.integers(-12, 4, size=shape)).astype(np.float32)


def _close(exact: Fraction, mag: Fraction, got: float, K: int):
    tol = mag * Fraction(K + 2) * Fraction(2) ** -52
    assert abs(Fraction(float(got)) - exact) <= tol, (float(exact), got)


def _check(entries, term, got, K):
    for (i, j) in entries:
        terms = [term(i, j, k) for k in range(K)]
        _close(sum(terms, Fraction(0)), sum((abs(t) for t in terms), Fraction(0)), got[i, j], K)


def test_fwd_exact_rational():
    rng = np.random.default_rng(30)
    M, N, K = 5, 256, 384
    xq, sx = _codes(rng, (M, K)), _scales(rng, (M, K // 128))
    wq, sw = _codes(rng, (N, K)), _scales(rng, (N // 128, K // 128))
    y = G.gemm_fwd(xq, sx, wq, sw)
    assert y.shape == (M, N)

    def term(m, n, k):
        return (_DEC_FR[xq[m, k]] * Fraction(float(sx[m, k // 128]))
                * _DEC_FR[wq[n, k]] * Fraction(float(sw[n // 128, k // 128])))
    _check([(0, 0), (1, 127), (2, 128), (4, 255), (3, 200)], term, y, K)


def test_dgrad_exact_rational():
    rng = np.random.default_rng(31)
    M, N, K = 4, 256, 384          # dY [M][N], W [N][K] -> dX [M][K]
    dyq, sdy = _codes(rng, (M, N)), _scales(rng, (M, N // 128))
    wq, sw = _codes(rng, (N, K)), _scales(rng, (N // 128, K // 128))
    dx = G.gemm_dgrad(dyq, sdy, wq, sw)
    assert dx.shape == (M, K)

    def term(m, k, n):
        return (_DEC_FR[dyq[m, n]] * Fraction(float(sdy[m, n // 128]))
                * _DEC_FR[wq[n, k]] * Fraction(float(sw[n // 128, k // 128])))
    _check([(0, 0), (1, 129), (3, 383), (2, 255)], term, dx, N)


def test_wgrad_exact_rational():
    rng = np.random.default_rng(32)
    M, N, K = 256, 5, 6            # tokens M; dYt [N][M], Xt [K][M] -> dW [N][K]
    dyqt, sdyt = _codes(rng, (N, M)), _scales(rng, (N, M // 128))
    xqt, sxt = _codes(rng, (K, M)), _scales(rng, (K, M // 128))
    dw = G.gemm_wgrad(dyqt, sdyt, xqt, sxt)
    assert dw.shape == (N, K)

    def term(n, k, m):
        return (_DEC_FR[dyqt[n, m]] * Fraction(float(sdyt[n, m // 128]))
                * _DEC_FR[xqt[k, m]] * Fraction(float(sxt[k, m // 128])))
    _check([(0, 0), (4, 5), (2, 3)], term, dw, M)


def _mx_setup(rng, T, E, N, K):
    xq, ex = _codes(rng, (T, K)), rng.integers(110, 140, size=(T, K // 32), dtype=np.uint8)
    wq, ew = _codes(rng, (E, N, K)), rng.integers(110, 140, size=(E, N, K // 32), dtype=np.uint8)
    return xq, ex, wq, ew


def test_grouped_mx_exact_rational():
    rng = np.random.default_rng(33)
    T, E, N, K = 7, 3, 4, 96
    xq, ex, wq, ew = _mx_setup(rng, T, E, N, K)
    offsets = np.array([0, 3, 3, 7], np.int32)          # expert 1 is empty
    y = G.grouped_gemm_mx(xq, ex, wq, ew, offsets)
    expert = [0, 0, 0, 2, 2, 2, 2]

    def term(t, n, k):
        e = expert[t]
        return (_DEC_FR[xq[t, k]] * Fraction(2) ** (int(ex[t, k // 32]) - 127)
                * _DEC_FR[wq[e, n, k]] * Fraction(2) ** (int(ew[e, n, k // 32]) - 127))
    _check([(t, n) for t in range(T) for n in range(N)], term, y, K)


def test_grouped_equals_dense_per_expert_and_single_expert():
    rng = np.random.default_rng(34)
    T, E, N, K = 40, 4, 64, 128
    xq, ex, wq, ew = _mx_setup(rng, T, E, N, K)
    offsets = np.array([0, 10, 10, 33, 40], np.int32)
    y = G.grouped_gemm_mx(xq, ex, wq, ew, offsets)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        ref = G.dequant_mx(xq[lo:hi], ex[lo:hi]) @ G.dequant_mx(wq[e], ew[e]).T
        assert np.array_equal(y[lo:hi], ref)
    y1 = G.grouped_gemm_mx(xq, ex, wq[:1], ew[:1], np.array([0, T], np.int32))
    assert np.array_equal(y1, G.dequant_mx(xq, ex) @ G.dequant_mx(wq[0], ew[0]).T)
    with pytest.raises(ValueError):
        G.grouped_gemm_mx(xq, ex, wq, ew, np.array([0, 10, 5, 33, 40], np.int32))


def test_grouped_block_exact_rational():
    """Blockwise grouped GEMM against the exact-rational loop: expert e's 128x128 weight
    block scale is looked up as sw[e][n // 128][k // 128], the row scale as sx[t][k // 128]."""
    rng = np.random.default_rng(36)
    T, E, N, K = 6, 3, 256, 256
    xq, sx = _codes(rng, (T, K)), _scales(rng, (T, K // 128))
    wq, sw = _codes(rng, (E, N, K)), _scales(rng, (E, N // 128, K // 128))
    offsets = np.array([0, 2, 2, 6], np.int32)          # expert 1 is empty
    y = G.grouped_gemm_block(xq, sx, wq, sw, offsets)
    expert = [0, 0, 2, 2, 2, 2]

    def term(t, n, k):
        e = expert[t]
        return (_DEC_FR[xq[t, k]] * Fraction(float(sx[t, k // 128]))
                * _DEC_FR[wq[e, n, k]] * Fraction(float(sw[e, n // 128, k // 128])))
    _check([(0, 0), (1, 200), (2, 127), (3, 128), (5, 255), (4, 7)], term, y, K)


def test_grouped_block_equals_dense_per_expert_and_single_expert():
    rng = np.random.default_rng(37)
    T, E, N, K = 40, 4, 256, 384
    xq, sx = _codes(rng, (T, K)), _scales(rng, (T, K // 128))
    wq, sw = _codes(rng, (E, N, K)), _scales(rng, (E, N // 128, K // 128))
    offsets = np.array([0, 10, 10, 33, 40], np.int32)
    y = G.grouped_gemm_block(xq, sx, wq, sw, offsets)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        assert np.array_equal(y[lo:hi], G.gemm_fwd(xq[lo:hi], sx[lo:hi], wq[e], sw[e]))
    y1 = G.grouped_gemm_block(xq, sx, wq[:1], sw[:1], np.array([0, T], np.int32))
    assert np.array_equal(y1, G.gemm_fwd(xq, sx, wq[0], sw[0]))
    with pytest.raises(ValueError):
        G.grouped_gemm_block(xq, sx, wq, sw, np.array([0, 10, 33, 40], np.int32))


def test_unit_scale_reduces_to_plain_product_of_codes():
    """With every scale 1.0 the block-scaled GEMM is the plain product of decoded
    codes, here computed by torch in float64 from torch-decoded values."""
    rng = np.random.default_rng(35)
    xq, wq = _codes(rng, (16, 256)), _codes(rng, (128, 256))
    y = G.gemm_fwd(xq, np.ones((16, 2), np.float32), wq, np.ones((1, 2), np.float32))
    a = torch.from_numpy(xq).view(torch.float8_e4m3fn).to(torch.float64)
    b = torch.from_numpy(wq).view(torch.float8_e4m3fn).to(torch.float64)
    assert np.allclose(y, (a @ b.T).numpy(), rtol=0, atol=1e-9)


def _e8(rng, shape):
    return rng.integers(100, 150, size=shape, dtype=np.uint8)


def _p2(b):
    return Fraction(2) ** (int(b) - 127)


def test_mx_dense_fwd_dgrad_wgrad_exact_rational():
    rng = np.random.default_rng(34)
    M, N, K = 5, 6, 96
    xq, ex = _codes(rng, (M, K)), _e8(rng, (M, K // 32))
    wq, ew = _codes(rng, (N, K)), _e8(rng, (N, K // 32))
    y = G.gemm_mx_fwd(xq, ex, wq, ew)
    assert y.shape == (M, N)
    _check([(m, n) for m in range(M) for n in range(N)],
           lambda m, n, k: _DEC_FR[xq[m, k]] * _p2(ex[m, k // 32]) * _DEC_FR[wq[n, k]] * _p2(ew[n, k // 32]), y, K)
    # DGrad: dY [M][Nr] (groups along Nr), Wt [K][Nr] (W's 32x1 copy) -> dX [M][K]
    Nr = 64
    dyq, edy = _codes(rng, (M, Nr)), _e8(rng, (M, Nr // 32))
    wqt, ewt = _codes(rng, (K, Nr)), _e8(rng, (K, Nr // 32))
    dx = G.gemm_mx_dgrad(dyq, edy, wqt, ewt)
    assert dx.shape == (M, K)
    _check([(0, 0), (4, 95), (2, 33)],
           lambda m, k, n: _DEC_FR[dyq[m, n]] * _p2(edy[m, n // 32]) * _DEC_FR[wqt[k, n]] * _p2(ewt[k, n // 32]), dx, Nr)
    # WGrad: dYt [N][T], Xt [K][T] -> dW [N][K]
    T = 64
    dyqt, edyt = _codes(rng, (N, T)), _e8(rng, (N, T // 32))
    xqt, ext = _codes(rng, (K, T)), _e8(rng, (K, T // 32))
    dw = G.gemm_mx_wgrad(dyqt, edyt, xqt, ext)
    assert dw.shape == (N, K)
    _check([(0, 0), (5, 95), (3, 40)],
           lambda n, k, t: _DEC_FR[dyqt[n, t]] * _p2(edyt[n, t // 32]) * _DEC_FR[xqt[k, t]] * _p2(ext[k, t // 32]), dw, T)
