"""Python binding of libfp8rl (fine-grained FP8 quantization and block-scaled FP8 GEMMs
for MI355X / gfx950).

The functions here have the names of the C entry points in ``include/fp8rl.h`` and do
argument marshalling only: they check devices, dtypes and shapes, allocate missing
outputs with torch, and pass raw device pointers plus torch's current HIP stream to the
library. Every step of the computation runs in the library's HIP kernels; there is no
fallback path. Importing this package does not load the library; the first call does,
and raises if ``libfp8rl.so`` has not been built
(``python -m fp8_block_scaled_quant_amd.build``).

Tensors: bf16 inputs as ``torch.bfloat16``; FP8 payloads and E8M0 scales as
``torch.uint8`` (raw bytes); fp32 scales as ``torch.float32``. All on the GPU,
contiguous.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Fp8rlError", "RECIPE_BLOCK128", "RECIPE_MXFP8", "OUT_BF16", "OUT_F32", "library_path", "load_library",
    "fp8rl_abi_version", "fp8_quant_act_1x128", "fp8_quant_w_128x128", "mxfp8_quant_1x32",
    "fp8_gemm_blockscaled_fwd", "fp8rl_fwd_workspace_bytes", "fp8_gemm_blockscaled_dgrad",
    "fp8_gemm_blockscaled_wgrad", "fp8_grouped_gemm", "fp8_weight_install",
    "fp8_quant_act_1x128_pow2", "fp8_quant_w_128x128_pow2", "fp8_gemm_blockscaled_pow2_fwd",
    "fp8_gemm_blockscaled_pow2_dgrad", "fp8_gemm_blockscaled_pow2_wgrad",
    "fp8_swiglu_bf16", "fp8_swiglu_quant_1x128", "fp8_rmsnorm_bf16", "fp8_rmsnorm_quant_1x128",
    "mxfp8_quant_act_1x32", "fp8_gemm_mxfp8_fwd", "fp8_gemm_mxfp8_dgrad", "fp8_gemm_mxfp8_wgrad",
    "fp8_quant_w_128x128_f32", "LAYOUT_ROWS", "LAYOUT_DECODE", "fp8_gemm_blockscaled_fwd_decode_layout",
    "fp8_gemm_blockscaled_fwd_decode_layout_noalloc", "NOALLOC_SCRATCH_BYTES",
    "fwd_workspace",
]

RECIPE_BLOCK128 = 0
RECIPE_MXFP8 = 1
LAYOUT_ROWS = 0
LAYOUT_DECODE = 1
OUT_BF16 = 0
OUT_F32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# FP8RL_LIBRARY names another build of the library (the sanitizer test loads one that way).
_LIB_PATH = os.environ.get("FP8RL_LIBRARY") or os.path.join(_HERE, "libfp8rl.so")
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t


class _Weight(ctypes.Structure):
    _fields_ = [("recipe", _int), ("rows", _i64), ("cols", _i64), ("q", _vp), ("s", _vp), ("layout", _int)]


_SIGNATURES = {
    "fp8rl_abi_version": ([], _int),
    "fp8rl_status_str": ([_int], ctypes.c_char_p),
    "fp8_quant_act_1x128": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp], _int),
    "fp8_quant_w_128x128": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp], _int),
    "mxfp8_quant_1x32": ([_vp, _i64, _i64, _vp, _vp, _vp], _int),
    "fp8_gemm_blockscaled_fwd": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _sz, _vp], _int),
    "fp8rl_fwd_workspace_bytes": ([_i64, _i64], _sz),
    "fp8_gemm_blockscaled_fwd_decode_layout": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _sz, _vp],
                                               _int),
    "fp8_gemm_blockscaled_fwd_decode_layout_noalloc": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp],
                                                       _int),
    "fp8_gemm_blockscaled_dgrad": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_gemm_blockscaled_wgrad": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_grouped_gemm": ([_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_weight_install": ([ctypes.POINTER(_Weight), ctypes.POINTER(_Weight), _vp], _int),
    "fp8_quant_act_1x128_pow2": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp], _int),
    "fp8_quant_w_128x128_pow2": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp], _int),
    "fp8_gemm_blockscaled_pow2_fwd": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_gemm_blockscaled_pow2_dgrad": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_gemm_blockscaled_pow2_wgrad": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_swiglu_bf16": ([_vp, _i64, _i64, _vp, _vp], _int),
    "mxfp8_quant_act_1x32": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp], _int),
    "fp8_quant_w_128x128_f32": ([_vp, _i64, _i64, _vp, _vp, _vp, _int, _vp], _int),
    "fp8_gemm_mxfp8_fwd": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_gemm_mxfp8_dgrad": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_gemm_mxfp8_wgrad": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp], _int),
    "fp8_swiglu_quant_1x128": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _int, _vp], _int),
    "fp8_rmsnorm_bf16": ([_vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp, _vp], _int),
    "fp8_rmsnorm_quant_1x128": ([_vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _int, _vp], _int),
}


class Fp8rlError(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = load_library().fp8rl_status_str(status).decode()
        super().__init__(f"{call}: status {status} ({msg})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libfp8rl.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m fp8_block_scaled_quant_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _check(status: int, call: str):
    if status != 0:
        raise Fp8rlError(status, call)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(t, dtype, shape, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(t, dtype, shape, name)


def fp8rl_abi_version() -> int:
    return load_library().fp8rl_abi_version()


def fp8_quant_act_1x128(x, q=None, s=None, qt=None, st=None, *, rowwise=True, colwise=False):
    """1x128 (row-wise) and/or 128x1 (column-wise, transposed) activation quantization.

    Returns (q [M][K] u8, s [M][K/128] f32, qt [K][M] u8, st [K][M/128] f32); outputs not
    requested are None."""
    return _quant_act("fp8_quant_act_1x128", x, q, s, qt, st, rowwise, colwise)


def fp8_quant_act_1x128_pow2(x, q=None, s=None, qt=None, st=None, *, rowwise=True, colwise=False):
    """As fp8_quant_act_1x128, with power-of-two scales (stored as fp32)."""
    return _quant_act("fp8_quant_act_1x128_pow2", x, q, s, qt, st, rowwise, colwise)


def _quant_act(entry, x, q, s, qt, st, rowwise, colwise):
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    dev = x.device
    if rowwise:
        q = _out(q, torch.uint8, (M, K), dev, "q")
        s = _out(s, torch.float32, (M, K // 128), dev, "s")
    else:
        q = s = None
    if colwise:
        qt = _out(qt, torch.uint8, (K, M), dev, "qt")
        st = _out(st, torch.float32, (K, M // 128), dev, "st")
    else:
        qt = st = None
    _check(getattr(lib, entry)(_ptr(x), M, K, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _stream(dev)), entry)
    return q, s, qt, st


def _act_outputs(M, K, dev, q, s, qt, st, rowwise, colwise):
    if rowwise:
        q = _out(q, torch.uint8, (M, K), dev, "q")
        s = _out(s, torch.float32, (M, K // 128), dev, "s")
    else:
        q = s = None
    if colwise:
        qt = _out(qt, torch.uint8, (K, M), dev, "qt")
        st = _out(st, torch.float32, (K, M // 128), dev, "st")
    else:
        qt = st = None
    return q, s, qt, st


def fp8_swiglu_bf16(gu, h=None):
    """h[M][F] = bf16(fl32(bf16(silu(gate)) * up)) for gu [M][2F] = [gate | up] (bf16)."""
    lib = load_library()
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be 2-D with an even number of columns")
    M, F = gu.shape[0], gu.shape[1] // 2
    _need(gu, torch.bfloat16, (M, 2 * F), "gu")
    h = _out(h, torch.bfloat16, (M, F), gu.device, "h")
    _check(lib.fp8_swiglu_bf16(_ptr(gu), M, F, _ptr(h), _stream(gu.device)), "fp8_swiglu_bf16")
    return h


def fp8_swiglu_quant_1x128(gu, q=None, s=None, qt=None, st=None, *, rowwise=True, colwise=False, pow2_scales=False):
    """SwiGLU of gu [M][2F] quantized 1x128 (and/or 128x1, transposed) without a bf16
    round trip. Returns (q, s, qt, st) as fp8_quant_act_1x128 does for h."""
    lib = load_library()
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be 2-D with an even number of columns")
    M, F = gu.shape[0], gu.shape[1] // 2
    _need(gu, torch.bfloat16, (M, 2 * F), "gu")
    q, s, qt, st = _act_outputs(M, F, gu.device, q, s, qt, st, rowwise, colwise)
    _check(lib.fp8_swiglu_quant_1x128(_ptr(gu), M, F, _ptr(q), _ptr(s), _ptr(qt), _ptr(st), 1 if pow2_scales else 0,
                                      _stream(gu.device)), "fp8_swiglu_quant_1x128")
    return q, s, qt, st


def fp8_rmsnorm_bf16(x, gamma, eps=1e-6, y=None, rstd=None):
    """y = bf16(fl32(gamma * bf16(fl32(x * r)))), r = fl32(1/sqrt(mean(x^2) + eps)) per row.
    Returns (y [M][K] bf16, rstd [M] f32)."""
    lib = load_library()
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(gamma, torch.bfloat16, (K,), "gamma")
    y = _out(y, torch.bfloat16, (M, K), x.device, "y")
    rstd = _out(rstd, torch.float32, (M,), x.device, "rstd")
    _check(lib.fp8_rmsnorm_bf16(_ptr(x), _ptr(gamma), M, K, float(eps), _ptr(y), _ptr(rstd), _stream(x.device)),
           "fp8_rmsnorm_bf16")
    return y, rstd


def fp8_rmsnorm_quant_1x128(x, gamma, eps=1e-6, q=None, s=None, qt=None, st=None, rstd=None, *, rowwise=True,
                            colwise=False, pow2_scales=False):
    """RMSNorm of x [M][K] quantized 1x128 (and/or 128x1, transposed) without a bf16 round
    trip. Returns (q, s, qt, st, rstd)."""
    lib = load_library()
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(gamma, torch.bfloat16, (K,), "gamma")
    q, s, qt, st = _act_outputs(M, K, x.device, q, s, qt, st, rowwise, colwise)
    rstd = _out(rstd, torch.float32, (M,), x.device, "rstd")
    _check(lib.fp8_rmsnorm_quant_1x128(_ptr(x), _ptr(gamma), M, K, float(eps), _ptr(rstd), _ptr(q), _ptr(s), _ptr(qt),
                                       _ptr(st), 1 if pow2_scales else 0, _stream(x.device)), "fp8_rmsnorm_quant_1x128")
    return q, s, qt, st, rstd


def fp8_quant_w_128x128(w, q=None, s=None, qt=None, *, transpose=False):
    """128x128-block weight quantization. Returns (q [N][K] u8, s [N/128][K/128] f32,
    qt [K][N] u8 or None)."""
    return _quant_w("fp8_quant_w_128x128", w, q, s, qt, transpose)


def fp8_quant_w_128x128_pow2(w, q=None, s=None, qt=None, *, transpose=False):
    """As fp8_quant_w_128x128, with power-of-two block scales (stored as fp32)."""
    return _quant_w("fp8_quant_w_128x128_pow2", w, q, s, qt, transpose)


def _quant_w(entry, w, q, s, qt, transpose):
    lib = load_library()
    N, K = w.shape
    _need(w, torch.bfloat16, (N, K), "w")
    dev = w.device
    q = _out(q, torch.uint8, (N, K), dev, "q")
    s = _out(s, torch.float32, (N // 128, K // 128), dev, "s")
    qt = _out(qt, torch.uint8, (K, N), dev, "qt") if transpose else None
    _check(getattr(lib, entry)(_ptr(w), N, K, _ptr(q), _ptr(s), _ptr(qt), _stream(dev)), entry)
    return q, s, qt


def mxfp8_quant_1x32(x, q=None, e8m0=None):
    """MXFP8 quantization, one E8M0 scale per 1x32 group. x: [..., K] bf16 (leading dims
    flattened into rows). Returns (q u8 same shape, e8m0 u8 [..., K/32])."""
    lib = load_library()
    K = x.shape[-1]
    R = x.numel() // K if K else 0
    _need(x, torch.bfloat16, tuple(x.shape), "x")
    dev = x.device
    q = _out(q, torch.uint8, tuple(x.shape), dev, "q")
    e8m0 = _out(e8m0, torch.uint8, tuple(x.shape[:-1]) + (K // 32,), dev, "e8m0")
    _check(lib.mxfp8_quant_1x32(_ptr(x), R, K, _ptr(q), _ptr(e8m0), _stream(dev)), "mxfp8_quant_1x32")
    return q, e8m0


def fp8_quant_w_128x128_f32(w, q=None, s=None, qt=None, *, transpose=False, pow2_scales=False):
    """fp8_param requantization: 128x128-block quantization of an fp32 master W [N][K].
    Returns (q [N][K] u8, s [N/128][K/128] f32, qt [K][N] u8 or None)."""
    lib = load_library()
    N, K = w.shape
    _need(w, torch.float32, (N, K), "w")
    dev = w.device
    q = _out(q, torch.uint8, (N, K), dev, "q")
    s = _out(s, torch.float32, (N // 128, K // 128), dev, "s")
    qt = _out(qt, torch.uint8, (K, N), dev, "qt") if transpose else None
    _check(lib.fp8_quant_w_128x128_f32(_ptr(w), N, K, _ptr(q), _ptr(s), _ptr(qt), 1 if pow2_scales else 0,
                                       _stream(dev)), "fp8_quant_w_128x128_f32")
    return q, s, qt


def mxfp8_quant_act_1x32(x, q=None, e8m0=None, qt=None, e8m0t=None, *, rowwise=True, colwise=False):
    """MXFP8 1x32 row groups and/or 32x1 column groups written transposed, of x [R][K] bf16.
    Returns (q [R][K], e8m0 [R][K/32], qt [K][R], e8m0t [K][R/32]); outputs not requested are None."""
    lib = load_library()
    R, K = x.shape
    _need(x, torch.bfloat16, (R, K), "x")
    dev = x.device
    if rowwise:
        q = _out(q, torch.uint8, (R, K), dev, "q")
        e8m0 = _out(e8m0, torch.uint8, (R, K // 32), dev, "e8m0")
    else:
        q = e8m0 = None
    if colwise:
        qt = _out(qt, torch.uint8, (K, R), dev, "qt")
        e8m0t = _out(e8m0t, torch.uint8, (K, R // 32), dev, "e8m0t")
    else:
        qt = e8m0t = None
    _check(lib.mxfp8_quant_act_1x32(_ptr(x), R, K, _ptr(q), _ptr(e8m0), _ptr(qt), _ptr(e8m0t), _stream(dev)),
           "mxfp8_quant_act_1x32")
    return q, e8m0, qt, e8m0t


def fp8_gemm_mxfp8_fwd(xq, ex, wq, ew, *, out_dtype=torch.bfloat16, y=None):
    """Y[M][N] = deq(X) deq(W)^T, MXFP8 operands (1x32 E8M0 scales along K)."""
    lib = load_library()
    M, K = xq.shape
    N = wq.shape[0]
    _need(xq, torch.uint8, (M, K), "xq")
    _need(ex, torch.uint8, (M, K // 32), "ex")
    _need(wq, torch.uint8, (N, K), "wq")
    _need(ew, torch.uint8, (N, K // 32), "ew")
    y = _out(y, out_dtype, (M, N), xq.device, "y")
    _check(lib.fp8_gemm_mxfp8_fwd(_ptr(xq), _ptr(ex), _ptr(wq), _ptr(ew), M, N, K, _ptr(y), _odt(out_dtype),
                                  _stream(xq.device)), "fp8_gemm_mxfp8_fwd")
    return y


def fp8_gemm_mxfp8_dgrad(dyq, edy, wqt, ewt, *, out_dtype=torch.bfloat16, dx=None):
    """dX[M][K] = deq(dY) deq(W); dyq [M][N]; W as its 32x1 copy wqt [K][N], ewt [K][N/32]."""
    lib = load_library()
    M, N = dyq.shape
    K = wqt.shape[0]
    _need(dyq, torch.uint8, (M, N), "dyq")
    _need(edy, torch.uint8, (M, N // 32), "edy")
    _need(wqt, torch.uint8, (K, N), "wqt")
    _need(ewt, torch.uint8, (K, N // 32), "ewt")
    dx = _out(dx, out_dtype, (M, K), dyq.device, "dx")
    _check(lib.fp8_gemm_mxfp8_dgrad(_ptr(dyq), _ptr(edy), _ptr(wqt), _ptr(ewt), M, N, K, _ptr(dx), _odt(out_dtype),
                                    _stream(dyq.device)), "fp8_gemm_mxfp8_dgrad")
    return dx


def fp8_gemm_mxfp8_wgrad(dyqt, edyt, xqt, ext, *, dw=None, accumulate=False):
    """dW[N][K] (fp32) = deq(dY)^T deq(X) from the 32x1 copies dyqt [N][M], xqt [K][M]."""
    lib = load_library()
    N, M = dyqt.shape
    K = xqt.shape[0]
    _need(dyqt, torch.uint8, (N, M), "dyqt")
    _need(edyt, torch.uint8, (N, M // 32), "edyt")
    _need(xqt, torch.uint8, (K, M), "xqt")
    _need(ext, torch.uint8, (K, M // 32), "ext")
    if dw is None:
        dw = (torch.zeros if accumulate else torch.empty)((N, K), dtype=torch.float32, device=dyqt.device)
    _need(dw, torch.float32, (N, K), "dw")
    _check(lib.fp8_gemm_mxfp8_wgrad(_ptr(dyqt), _ptr(edyt), _ptr(xqt), _ptr(ext), M, N, K, _ptr(dw),
                                    1 if accumulate else 0, _stream(dyqt.device)), "fp8_gemm_mxfp8_wgrad")
    return dw


def fp8rl_fwd_workspace_bytes(M: int, K: int) -> int:
    return load_library().fp8rl_fwd_workspace_bytes(M, K)


def _odt(out_dtype):
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    if out_dtype == torch.float32:
        return OUT_F32
    raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")


def fwd_workspace(M, K, device):
    """A workspace for the bf16-input forward calls: the quantized X and its scales (any
    contents; calls running at the same time need one each)."""
    nbytes = load_library().fp8rl_fwd_workspace_bytes(M, K)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _fwd(fn, name, xq, sx, wq, sw, x_bf16, out_dtype, y, workspace, N, K):
    lib = load_library()
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    dev = wq.device
    if x_bf16 is not None:
        M = x_bf16.shape[0]
        _need(x_bf16, torch.bfloat16, (M, K), "x_bf16")
        if xq is not None or sx is not None:
            raise ValueError("give either (xq, sx) or x_bf16")
        if workspace is None:
            workspace = fwd_workspace(M, K, dev)
    else:
        M = xq.shape[0]
        _need(xq, torch.uint8, (M, K), "xq")
        _need(sx, torch.float32, (M, K // 128), "sx")
    y = _out(y, out_dtype, (M, N), dev, "y")
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(getattr(lib, fn)(_ptr(xq), _ptr(sx), _ptr(x_bf16), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), _odt(out_dtype),
                            _ptr(workspace), ws_bytes, _stream(dev)), name)
    return y


def fp8_gemm_blockscaled_fwd(xq=None, sx=None, wq=None, sw=None, *, x_bf16=None, out_dtype=torch.bfloat16, y=None,
                             workspace=None):
    """Y[M][N] = deq(X) deq(W)^T. X as (xq, sx) or, for the fused form, as x_bf16 (then a
    workspace is allocated unless given; see fwd_workspace)."""
    N, K = wq.shape
    _need(wq, torch.uint8, (N, K), "wq")
    return _fwd("fp8_gemm_blockscaled_fwd", "fp8_gemm_blockscaled_fwd", xq, sx, wq, sw, x_bf16, out_dtype, y,
                workspace, N, K)


def fp8_gemm_blockscaled_fwd_decode_layout(xq=None, sx=None, wq=None, sw=None, *, N, K, x_bf16=None,
                                           out_dtype=torch.bfloat16, y=None, workspace=None):
    """The forward product with W's payload in the decode layout (fp8_weight_install with
    layout=LAYOUT_DECODE): wq holds N * K bytes."""
    if wq.dtype != torch.uint8 or not wq.is_cuda or not wq.is_contiguous() or wq.numel() != N * K:
        raise ValueError(f"wq must be a contiguous GPU uint8 tensor of {N} * {K} bytes")
    return _fwd("fp8_gemm_blockscaled_fwd_decode_layout", "fp8_gemm_blockscaled_fwd_decode_layout", xq, sx, wq, sw,
                x_bf16, out_dtype, y, workspace, N, K)


NOALLOC_SCRATCH_BYTES = 16 << 20   # FP8RL_NOALLOC_SCRATCH_BYTES


def fp8_gemm_blockscaled_fwd_decode_layout_noalloc(xq=None, sx=None, wq=None, sw=None, *, N, K, x_bf16=None,
                                                   out_dtype=torch.bfloat16, y=None):
    """fp8_gemm_blockscaled_fwd_decode_layout without a workspace: the C call quantizes a bf16
    X into the library's built-in scratch and allocates nothing (pass y to allocate nothing
    here either). Calls that may overlap on one GPU must be serialised by the caller."""
    if wq.dtype != torch.uint8 or not wq.is_cuda or not wq.is_contiguous() or wq.numel() != N * K:
        raise ValueError(f"wq must be a contiguous GPU uint8 tensor of {N} * {K} bytes")
    lib = load_library()
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    dev = wq.device
    if x_bf16 is not None:
        if xq is not None or sx is not None:
            raise ValueError("give either (xq, sx) or x_bf16")
        M = x_bf16.shape[0]
        _need(x_bf16, torch.bfloat16, (M, K), "x_bf16")
    else:
        M = xq.shape[0]
        _need(xq, torch.uint8, (M, K), "xq")
        _need(sx, torch.float32, (M, K // 128), "sx")
    y = _out(y, out_dtype, (M, N), dev, "y")
    _check(lib.fp8_gemm_blockscaled_fwd_decode_layout_noalloc(_ptr(xq), _ptr(sx), _ptr(x_bf16), _ptr(wq), _ptr(sw), M, N,
                                                              K, _ptr(y), _odt(out_dtype), _stream(dev)),
           "fp8_gemm_blockscaled_fwd_decode_layout_noalloc")
    return y


def fp8_gemm_blockscaled_pow2_fwd(xq, sx, wq, sw, *, out_dtype=torch.bfloat16, y=None):
    """Y[M][N] = deq(X) deq(W)^T for power-of-two block scales (FP8 X only)."""
    lib = load_library()
    N, K = wq.shape
    M = xq.shape[0]
    _need(wq, torch.uint8, (N, K), "wq")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    _need(xq, torch.uint8, (M, K), "xq")
    _need(sx, torch.float32, (M, K // 128), "sx")
    y = _out(y, out_dtype, (M, N), wq.device, "y")
    _check(lib.fp8_gemm_blockscaled_pow2_fwd(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(y),
                                             _odt(out_dtype), _stream(wq.device)), "fp8_gemm_blockscaled_pow2_fwd")
    return y


def fp8_gemm_blockscaled_dgrad(dyq, sdy, wqt, sw, *, out_dtype=torch.bfloat16, dx=None):
    """dX[M][K] = deq(dY) deq(W) with wqt = W's byte transpose [K][N], sw [N/128][K/128]."""
    return _dgrad("fp8_gemm_blockscaled_dgrad", dyq, sdy, wqt, sw, out_dtype, dx)


def fp8_gemm_blockscaled_pow2_dgrad(dyq, sdy, wqt, sw, *, out_dtype=torch.bfloat16, dx=None):
    """As fp8_gemm_blockscaled_dgrad, for power-of-two block scales."""
    return _dgrad("fp8_gemm_blockscaled_pow2_dgrad", dyq, sdy, wqt, sw, out_dtype, dx)


def _dgrad(entry, dyq, sdy, wqt, sw, out_dtype, dx):
    lib = load_library()
    M, N = dyq.shape
    K = wqt.shape[0]
    _need(dyq, torch.uint8, (M, N), "dyq")
    _need(sdy, torch.float32, (M, N // 128), "sdy")
    _need(wqt, torch.uint8, (K, N), "wqt")
    _need(sw, torch.float32, (N // 128, K // 128), "sw")
    dx = _out(dx, out_dtype, (M, K), dyq.device, "dx")
    _check(getattr(lib, entry)(_ptr(dyq), _ptr(sdy), _ptr(wqt), _ptr(sw), M, N, K, _ptr(dx), _odt(out_dtype),
                               _stream(dyq.device)), entry)
    return dx


def fp8_gemm_blockscaled_wgrad(dyqt, sdyt, xqt, sxt, *, dw=None, accumulate=False):
    """dW[N][K] (fp32) = deq(dY)^T deq(X) from the column-wise copies dyqt [N][M], xqt [K][M]."""
    return _wgrad("fp8_gemm_blockscaled_wgrad", dyqt, sdyt, xqt, sxt, dw, accumulate)


def fp8_gemm_blockscaled_pow2_wgrad(dyqt, sdyt, xqt, sxt, *, dw=None, accumulate=False):
    """As fp8_gemm_blockscaled_wgrad, for power-of-two scales."""
    return _wgrad("fp8_gemm_blockscaled_pow2_wgrad", dyqt, sdyt, xqt, sxt, dw, accumulate)


def _wgrad(entry, dyqt, sdyt, xqt, sxt, dw, accumulate):
    lib = load_library()
    N, M = dyqt.shape
    K = xqt.shape[0]
    _need(dyqt, torch.uint8, (N, M), "dyqt")
    _need(sdyt, torch.float32, (N, M // 128), "sdyt")
    _need(xqt, torch.uint8, (K, M), "xqt")
    _need(sxt, torch.float32, (K, M // 128), "sxt")
    if accumulate and dw is None:
        raise ValueError("accumulate=True needs dw")
    dw = _out(dw, torch.float32, (N, K), dyqt.device, "dw")
    _check(getattr(lib, entry)(_ptr(dyqt), _ptr(sdyt), _ptr(xqt), _ptr(sxt), M, N, K, _ptr(dw),
                               1 if accumulate else 0, _stream(dyqt.device)), entry)
    return dw


def fp8_grouped_gemm(xq, sx, wq, sw, offsets, *, recipe=RECIPE_MXFP8, out_dtype=torch.bfloat16, y=None):
    """Grouped GEMM, offsets int32 [E+1] on the GPU. Returns y [T][N].
    RECIPE_MXFP8:    xq [T][K] u8, sx [T][K/32] u8, wq [E][N][K] u8, sw [E][N][K/32] u8.
    RECIPE_BLOCK128: xq [T][K] u8, sx [T][K/128] f32, wq [E][N][K] u8, sw [E][N/128][K/128] f32."""
    lib = load_library()
    T, K = xq.shape
    E, N, _ = wq.shape
    _need(xq, torch.uint8, (T, K), "xq")
    _need(wq, torch.uint8, (E, N, K), "wq")
    if recipe == RECIPE_BLOCK128:
        _need(sx, torch.float32, (T, K // 128), "sx")
        _need(sw, torch.float32, (E, N // 128, K // 128), "sw")
    else:
        _need(sx, torch.uint8, (T, K // 32), "sx")
        _need(sw, torch.uint8, (E, N, K // 32), "sw")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    y = _out(y, out_dtype, (T, N), xq.device, "y")
    _check(lib.fp8_grouped_gemm(recipe, _ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(offsets), T, E, N, K, _ptr(y),
                                _odt(out_dtype), _stream(xq.device)), "fp8_grouped_gemm")
    return y


def fp8_weight_install(src_q, src_s, dst_q, dst_s, *, recipe=RECIPE_BLOCK128, layout=LAYOUT_ROWS,
                       src_layout=LAYOUT_ROWS):
    """Install a quantized weight's payload and scales into the destination buffers, with no
    quantizer: verbatim, or regrouped into the decode layout (layout=LAYOUT_DECODE)."""
    lib = load_library()
    rows = src_q.shape[0] if src_q.dim() == 2 else src_q.numel() // src_q.shape[-1]
    cols = src_q.shape[-1]
    drows = dst_q.shape[0] if dst_q.dim() == 2 else dst_q.numel() // dst_q.shape[-1]
    for t, name in ((src_q, "src_q"), (src_s, "src_s"), (dst_q, "dst_q"), (dst_s, "dst_s")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    for qt_, st_, r_, name in ((src_q, src_s, rows, "src"), (dst_q, dst_s, drows, "dst")):
        if qt_.dtype != torch.uint8:
            raise ValueError(f"{name}_q must be uint8")
        if recipe == RECIPE_BLOCK128:
            need = (r_ // 128) * (cols // 128) * 4
        elif recipe == RECIPE_MXFP8:
            need = r_ * (cols // 32)
        else:
            need = 0
        if st_.numel() * st_.element_size() < need:
            raise ValueError(f"{name}_s holds {st_.numel() * st_.element_size()} bytes, the recipe needs {need}")
    src = _Weight(recipe, rows, cols, src_q.data_ptr(), src_s.data_ptr(), src_layout)
    dst = _Weight(recipe, drows, dst_q.shape[-1], dst_q.data_ptr(), dst_s.data_ptr(), layout)
    _check(lib.fp8_weight_install(ctypes.byref(src), ctypes.byref(dst), _stream(src_q.device)), "fp8_weight_install")
    return dst_q, dst_s
