"""CPU tests of the C-ABI boundary: the library loads, exports every function that
include/fp8rl.h declares under its C name, and rejects invalid arguments with the
documented status codes before making any HIP call (no GPU needed: the pointers below are
never dereferenced)."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

import fp8_block_scaled_quant_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8rl.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_RECIPE, ERR_DEVICE, ERR_LAUNCH, ERR_WORKSPACE, ERR_VALUE = range(9)
P = 0x10000          # an aligned, never-dereferenced fake device address
P2 = 0x20000
MIS = 0x10008        # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(fp8\w*|mxfp8\w*)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.library_path()):
        pytest.fail("libfp8rl.so is not built (run __graft_entry__.build())")
    return F.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["fp8_quant_act_1x128", "fp8_quant_w_128x128", "mxfp8_quant_1x32", "fp8_gemm_blockscaled_fwd",
              "fp8_gemm_blockscaled_dgrad", "fp8_gemm_blockscaled_wgrad", "fp8_grouped_gemm", "fp8_weight_install",
              "fp8rl_abi_version", "fp8rl_status_str", "fp8rl_fwd_workspace_bytes", "fp8_quant_act_1x128_pow2",
              "fp8_quant_w_128x128_pow2", "fp8_gemm_blockscaled_pow2_fwd", "fp8_gemm_blockscaled_pow2_dgrad",
              "fp8_gemm_blockscaled_pow2_wgrad", "fp8_swiglu_bf16", "fp8_swiglu_quant_1x128", "fp8_rmsnorm_bf16",
              "fp8_rmsnorm_quant_1x128", "mxfp8_quant_act_1x32", "fp8_gemm_mxfp8_fwd", "fp8_gemm_mxfp8_dgrad",
              "fp8_gemm_mxfp8_wgrad", "fp8_quant_w_128x128_f32", "fp8_gemm_blockscaled_fwd_decode_layout",
              "fp8_gemm_blockscaled_fwd_decode_layout_noalloc"]:
        assert n in names


def test_every_declared_function_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    if shutil.which("nm"):
        out = subprocess.run(["nm", "-D", "--defined-only", F.library_path()], capture_output=True, text=True).stdout
        exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
        for n in declared_functions():
            assert n in exported, f"{n} not exported with C linkage"


def test_version_and_status_strings(lib):
    assert lib.fp8rl_abi_version() == 7
    for code in range(9):
        assert len(lib.fp8rl_status_str(code)) > 0
    assert lib.fp8rl_status_str(99) == b"unknown status"


def test_workspace_size(lib):
    # the quantized X padded to 256 bytes, then its fp32 scales
    assert lib.fp8rl_fwd_workspace_bytes(256, 4096) == 256 * 4096 + 256 * 32 * 4
    assert lib.fp8rl_fwd_workspace_bytes(3, 128) == 512 + 3 * 4
    assert lib.fp8rl_fwd_workspace_bytes(0, 128) == 0
    assert lib.fp8rl_fwd_workspace_bytes(4, 100) == 0


def test_quant_act_validation(lib):
    f = lib.fp8_quant_act_1x128
    assert f(P, 4, 256, P, None, None, None, None) == ERR_NULL          # half a pair
    assert f(P, 4, 256, None, None, None, None, None) == ERR_NULL       # nothing requested
    assert f(P, 4, 100, P, P, None, None, None) == ERR_SHAPE            # K % 128
    assert f(P, -1, 128, P, P, None, None, None) == ERR_SHAPE
    assert f(P, 100, 128, None, None, P, P, None) == ERR_SHAPE          # column groups need M % 128
    assert f(MIS, 4, 128, P, P, None, None, None) == ERR_ALIGN
    assert f(P, 4, 128, MIS, P, None, None, None) == ERR_ALIGN
    assert f(P, 4, 128, P, P + 2, None, None, None) == ERR_ALIGN
    assert f(None, 4, 128, P, P, None, None, None) == ERR_NULL
    assert f(None, 0, 128, P, P, None, None, None) == OK                # empty: no device work


def test_quant_w_and_mx_validation(lib):
    assert lib.fp8_quant_w_128x128(P, 128, 128, None, P, None, None) == ERR_NULL
    assert lib.fp8_quant_w_128x128(P, 100, 128, P, P, None, None) == ERR_SHAPE
    assert lib.fp8_quant_w_128x128(P, 128, 64, P, P, None, None) == ERR_SHAPE
    assert lib.fp8_quant_w_128x128(P, 128, 128, P, P, MIS, None) == ERR_ALIGN
    assert lib.fp8_quant_w_128x128(None, 0, 128, P, P, None, None) == OK
    assert lib.mxfp8_quant_1x32(P, 4, 48, P, P, None) == ERR_SHAPE
    assert lib.mxfp8_quant_1x32(P, 4, 64, None, P, None) == ERR_NULL
    assert lib.mxfp8_quant_1x32(P, 4, 64, MIS, P, None) == ERR_ALIGN
    assert lib.mxfp8_quant_1x32(None, 0, 64, P, P, None) == OK


def test_gemm_validation(lib):
    fwd = lib.fp8_gemm_blockscaled_fwd
    assert fwd(P, P, P, P, P, 4, 128, 128, P, 0, None, 0, None) == ERR_NULL      # both forms of X
    assert fwd(None, None, None, P, P, 4, 128, 128, P, 0, None, 0, None) == ERR_NULL
    assert fwd(P, None, None, P, P, 4, 128, 128, P, 0, None, 0, None) == ERR_NULL
    assert fwd(P, P, None, P, P, 4, 128, 128, P, 7, None, 0, None) == ERR_RECIPE
    assert fwd(P, P, None, P, P, 4, 128, 100, P, 0, None, 0, None) == ERR_SHAPE   # K % 128
    assert fwd(P, P, None, P, P, 4, 100, 128, P, 0, None, 0, None) == ERR_SHAPE   # N % 128
    assert fwd(P, P, None, P, P, 0, 128, 128, P, 0, None, 0, None) == OK
    assert fwd(P, P, None, MIS, P, 4, 128, 128, P, 0, None, 0, None) == ERR_ALIGN
    assert fwd(None, None, P, P, P, 4, 128, 128, P, 0, None, 0, None) == ERR_WORKSPACE
    assert fwd(None, None, P, P, P, 4, 128, 128, P, 0, P2, 100, None) == ERR_WORKSPACE
    assert fwd(None, None, P, P, P, 4, 128, 128, P, 0, MIS, 1 << 20, None) == ERR_ALIGN
    # the decode-layout forward: same rules, plus 32-bit offsets (M K and N K below 2^32)
    fd = lib.fp8_gemm_blockscaled_fwd_decode_layout
    assert fd(P, P, P, P, P, 4, 128, 128, P, 0, None, 0, None) == ERR_NULL
    assert fd(P, P, None, P, P, 4, 100, 128, P, 0, None, 0, None) == ERR_SHAPE
    assert fd(P, P, None, P, P, 4, 1 << 21, 1 << 11, P, 0, None, 0, None) == ERR_SHAPE   # N K = 2^32
    assert fd(P, P, None, P, P, 1 << 21, 128, 1 << 11, P, 0, None, 0, None) == ERR_SHAPE  # M K = 2^32
    assert fd(None, None, P, P, P, 4, 128, 128, P, 0, P2, 100, None) == ERR_WORKSPACE
    assert fd(P, P, None, P, P, 0, 128, 128, P, 0, None, 0, None) == OK
    # bf16-input form of the general forward: M K below 2^32 (a larger M goes to the tiled GEMM)
    assert fwd(None, None, P, P, P, 1 << 21, 128, 1 << 11, P, 0, P2, 1 << 40, None) == ERR_SHAPE
    dg = lib.fp8_gemm_blockscaled_dgrad
    assert dg(P, P, None, P, 4, 128, 128, P, 0, None) == ERR_NULL
    assert dg(P, P, P, P, 4, 100, 128, P, 0, None) == ERR_SHAPE
    assert dg(P, P, P, P, 4, 128, 100, P, 0, None) == ERR_SHAPE
    assert dg(P, P, P, P, 4, 128, 128, P, 3, None) == ERR_RECIPE
    assert dg(P, P, P, P, 0, 128, 128, P, 0, None) == OK
    wg = lib.fp8_gemm_blockscaled_wgrad
    assert wg(P, P, P, P, 100, 128, 128, P, 0, None) == ERR_SHAPE                  # tokens % 128
    assert wg(P, P, P, P, 128, 128, 128, None, 0, None) == ERR_NULL
    assert wg(P, P, P, P, 128, 128, 128, MIS, 0, None) == ERR_ALIGN
    assert wg(P, P, P, P, 128, 0, 128, P, 0, None) == OK


def test_producer_validation(lib):
    sb = lib.fp8_swiglu_bf16
    assert sb(P, 4, 100, P, None) == ERR_SHAPE                          # F % 128
    assert sb(None, 4, 128, P, None) == ERR_NULL
    assert sb(P, 4, 128, None, None) == ERR_NULL
    assert sb(MIS, 4, 128, P, None) == ERR_ALIGN
    assert sb(P, 0, 128, None, None) == OK
    sq = lib.fp8_swiglu_quant_1x128
    assert sq(P, 4, 128, P, None, None, None, 0, None) == ERR_NULL      # half a pair
    assert sq(P, 4, 128, None, None, None, None, 0, None) == ERR_NULL   # nothing requested
    assert sq(P, 100, 128, None, None, P, P, 0, None) == ERR_SHAPE      # column groups need M % 128
    assert sq(P, 4, 128, P, P + 2, None, None, 1, None) == ERR_ALIGN
    assert sq(P, -1, 128, P, P, None, None, 0, None) == ERR_SHAPE
    rb = lib.fp8_rmsnorm_bf16
    assert rb(P, P, 4, 128, 0.0, P, P, None) == ERR_VALUE               # eps must be positive
    assert rb(P, P, 4, 128, float("nan"), P, P, None) == ERR_VALUE
    assert rb(P, P, 4, 128, float("inf"), P, P, None) == ERR_VALUE
    assert rb(P, P, 4, 100, 1e-6, P, P, None) == ERR_SHAPE
    assert rb(P, P, 4, 65536 + 128, 1e-6, P, P, None) == ERR_SHAPE      # K <= 65536
    assert rb(P, None, 4, 128, 1e-6, P, P, None) == ERR_NULL
    assert rb(P, P, 4, 128, 1e-6, P, None, None) == ERR_NULL            # rstd required
    assert rb(P, P, 4, 128, 1e-6, MIS, P, None) == ERR_ALIGN
    rq = lib.fp8_rmsnorm_quant_1x128
    assert rq(P, P, 4, 128, 1e-6, P, None, None, P, P, 0, None) == ERR_SHAPE     # qt needs M % 128
    assert rq(P, P, 4, 128, 1e-6, P, None, None, None, None, 0, None) == ERR_NULL
    assert rq(P, P, 4, 128, -1.0, P, P, P, None, None, 0, None) == ERR_VALUE
    assert rq(P, P, 0, 128, 1e-6, None, P, P, None, None, 0, None) == OK


def test_fp8_param_validation(lib):
    f = lib.fp8_quant_w_128x128_f32
    assert f(P, 128, 128, None, P, None, 0, None) == ERR_NULL
    assert f(P, 100, 128, P, P, None, 0, None) == ERR_SHAPE
    assert f(P, 128, 64, P, P, None, 1, None) == ERR_SHAPE
    assert f(MIS, 128, 128, P, P, None, 0, None) == ERR_ALIGN
    assert f(P, 128, 128, P, P, MIS, 0, None) == ERR_ALIGN
    assert f(None, 128, 128, P, P, None, 0, None) == ERR_NULL
    assert f(None, 0, 128, P, P, None, 0, None) == OK


def test_mx_dense_validation(lib):
    qa = lib.mxfp8_quant_act_1x32
    assert qa(P, 4, 48, P, P, None, None, None) == ERR_SHAPE               # K % 32
    assert qa(P, 4, 64, P, None, None, None, None) == ERR_NULL             # half a pair
    assert qa(P, 4, 64, None, None, None, None, None) == ERR_NULL          # nothing requested
    assert qa(P, 100, 128, None, None, P, P, None) == ERR_SHAPE            # columns need R % 128
    assert qa(P, 128, 96, None, None, P, P, None) == ERR_SHAPE             # ... and K % 128
    assert qa(MIS, 4, 64, P, P, None, None, None) == ERR_ALIGN
    assert qa(P, 0, 64, None, None, None, None, None) == OK
    f = lib.fp8_gemm_mxfp8_fwd
    assert f(P, P, P, P, 4, 128, 128, P, 7, None) == ERR_RECIPE
    assert f(P, P, P, P, 4, 128, 96, P, 0, None) == ERR_SHAPE              # K % 128
    assert f(P, P, P, P, 4, 100, 128, P, 0, None) == ERR_SHAPE             # N % 128
    assert f(P, None, P, P, 4, 128, 128, P, 0, None) == ERR_NULL
    assert f(P, P + 2, P, P, 4, 128, 128, P, 0, None) == ERR_ALIGN         # E8M0 rows read as dwords
    assert f(P, P, P, P, 0, 128, 128, P, 0, None) == OK
    d = lib.fp8_gemm_mxfp8_dgrad
    assert d(P, P, P, P, 4, 100, 128, P, 0, None) == ERR_SHAPE             # N % 128 (contraction)
    assert d(P, P, P, P, 4, 128, 100, P, 0, None) == ERR_SHAPE             # K % 128 (output columns)
    w = lib.fp8_gemm_mxfp8_wgrad
    assert w(P, P, P, P, 100, 128, 128, P, 0, None) == ERR_SHAPE           # tokens % 128
    assert w(P, P, P, P, 128, 128, 128, None, 0, None) == ERR_NULL
    assert w(P, P, P, P, 128, 0, 128, P, 0, None) == OK


def test_reduction_length_limit(lib):
    """Reduction lengths past 2^23 are rejected before any HIP call (the kernels address a
    tile's 256 rows with 32-bit byte offsets)."""
    big = (1 << 23) + 128
    assert lib.fp8_gemm_blockscaled_fwd(P, P, None, P, P, 4, 128, big, P, 0, None, 0, None) == ERR_SHAPE
    assert lib.fp8_gemm_blockscaled_pow2_fwd(P, P, P, P, 4, 128, big, P, 0, None) == ERR_SHAPE
    assert lib.fp8_gemm_blockscaled_dgrad(P, P, P, P, 4, big, 128, P, 0, None) == ERR_SHAPE
    assert lib.fp8_gemm_blockscaled_wgrad(P, P, P, P, big, 128, 128, P, 0, None) == ERR_SHAPE
    assert lib.fp8_gemm_mxfp8_fwd(P, P, P, P, 4, 128, big, P, 0, None) == ERR_SHAPE
    assert lib.fp8_grouped_gemm(F.RECIPE_MXFP8, P, P, P, P, P, 64, 2, 128, big, P, 0, None) == ERR_SHAPE
    # at the limit the shape rules pass: a zero-row call is OK without touching the device
    assert lib.fp8_gemm_blockscaled_fwd(P, P, None, P, P, 0, 128, 1 << 23, P, 0, None, 0, None) == OK


def test_grouped_validation(lib):
    g = lib.fp8_grouped_gemm
    assert g(7, P, P, P, P, P, 64, 2, 128, 128, P, 0, None) == ERR_RECIPE                # unknown recipe
    assert g(F.RECIPE_BLOCK128, P, P, P, P, P, 64, 2, 144, 128, P, 0, None) == ERR_SHAPE  # N % 128 (blocks)
    assert g(F.RECIPE_BLOCK128, P, P, P, P, P, 64, 2, 128, 128, P, 2, None) == ERR_RECIPE  # output dtype
    assert g(F.RECIPE_BLOCK128, P, P, P, P, P, 0, 2, 128, 128, P, 0, None) == OK
    assert g(F.RECIPE_MXFP8, P, P, P, P, P, 64, 0, 128, 128, P, 0, None) == ERR_SHAPE
    assert g(F.RECIPE_MXFP8, P, P, P, P, P, 64, 2, 128, 96, P, 0, None) == ERR_SHAPE   # K % 128
    assert g(F.RECIPE_MXFP8, P, P, P, P, P, 64, 2, 120, 128, P, 0, None) == ERR_SHAPE  # N % 16
    assert g(F.RECIPE_MXFP8, P, P, P, P, None, 64, 2, 128, 128, P, 0, None) == ERR_NULL
    assert g(F.RECIPE_MXFP8, P, P, P, P, P + 2, 64, 2, 128, 128, P, 0, None) == ERR_ALIGN
    assert g(F.RECIPE_MXFP8, P, P, P, P, P, 0, 2, 128, 128, P, 0, None) == OK


def test_install_validation(lib):
    W = F._Weight
    a = W(F.RECIPE_BLOCK128, 256, 256, P, P)
    assert lib.fp8_weight_install(ctypes.byref(a), ctypes.byref(W(F.RECIPE_MXFP8, 256, 256, P2, P2)), None) == ERR_RECIPE
    assert lib.fp8_weight_install(ctypes.byref(a), ctypes.byref(W(F.RECIPE_BLOCK128, 128, 256, P2, P2)), None) == ERR_RECIPE
    assert lib.fp8_weight_install(ctypes.byref(a), None, None) == ERR_NULL
    bad = W(F.RECIPE_BLOCK128, 100, 256, P, P)
    assert lib.fp8_weight_install(ctypes.byref(bad), ctypes.byref(W(F.RECIPE_BLOCK128, 100, 256, P2, P2)), None) == ERR_SHAPE
    mx = W(F.RECIPE_MXFP8, 3, 48, P, P)
    assert lib.fp8_weight_install(ctypes.byref(mx), ctypes.byref(W(F.RECIPE_MXFP8, 3, 48, P2, P2)), None) == ERR_SHAPE
    odd = W(7, 128, 128, P, P)
    assert lib.fp8_weight_install(ctypes.byref(odd), ctypes.byref(W(7, 128, 128, P2, P2)), None) == ERR_RECIPE
    nul = W(F.RECIPE_BLOCK128, 128, 128, None, P)
    assert lib.fp8_weight_install(ctypes.byref(nul), ctypes.byref(W(F.RECIPE_BLOCK128, 128, 128, P2, P2)), None) == ERR_NULL
    e = W(F.RECIPE_BLOCK128, 0, 128, None, None)
    assert lib.fp8_weight_install(ctypes.byref(e), ctypes.byref(W(F.RECIPE_BLOCK128, 0, 128, None, None)), None) == OK
    # layouts: the decode layout is BLOCK128 only, and a decode-layout payload never goes back to rows
    rows_to_dec = W(F.RECIPE_BLOCK128, 256, 256, P2, P2, F.LAYOUT_DECODE)
    dec = W(F.RECIPE_BLOCK128, 256, 256, P, P, F.LAYOUT_DECODE)
    assert lib.fp8_weight_install(ctypes.byref(dec), ctypes.byref(W(F.RECIPE_BLOCK128, 256, 256, P2, P2)), None) == ERR_RECIPE
    mxa = W(F.RECIPE_MXFP8, 256, 256, P, P)
    assert lib.fp8_weight_install(ctypes.byref(mxa), ctypes.byref(W(F.RECIPE_MXFP8, 256, 256, P2, P2, F.LAYOUT_DECODE)), None) == ERR_RECIPE
    assert lib.fp8_weight_install(ctypes.byref(a), ctypes.byref(W(F.RECIPE_BLOCK128, 256, 256, P2, P2, 5)), None) == ERR_RECIPE
    assert lib.fp8_weight_install(ctypes.byref(bad), ctypes.byref(W(F.RECIPE_BLOCK128, 100, 256, P2, P2, F.LAYOUT_DECODE)), None) == ERR_SHAPE
    del rows_to_dec


def _gpu_present():
    return os.path.exists("/dev/kfd")


@pytest.mark.skipif(_gpu_present(), reason="checks the no-GPU error path; a GPU is present")
def test_valid_call_without_a_gpu_reports_device_error(lib):
    # Arguments pass validation; the device query then fails on a host without a GPU.
    assert lib.fp8_quant_act_1x128(P, 4, 128, P, P, None, None, None) == ERR_DEVICE
