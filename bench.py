"""Benchmark of the FP8 block-scaled hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-also] [--no-graph]
                    [--workload dense|dense_pow2|decode|backward|backward_pow2|moe|moe_block128|install|producers|mx_dense|fp8_param] [--no-cpu-baseline]

A step is one pass of the hot path over one batch of synthetic input, inputs resident in
HBM. The default workload is the dense layer shaped like a ~9B model's MLP
(X 8192x4096 with 0.1% outlier channels x50, fused gate/up W 24576x4096, down
W 4096x12288, down input 8192x12288):
    quantize X 1x128 row-wise + 128x1 column-wise (the copy WGrad consumes),
    quantize W_gu and W_dn per 128x128 block (re-quantized each optimizer step),
    Y_gu = X . W_gu^T (FP8 MFMA, fp32 accumulation, bf16 out),
    quantize the down input 1x128, Y_dn = X2 . W_dn^T.
`value` = GEMM FLOPs of the step / step time (TFLOP/s, whole step including the
quantizers). The step time is that of K steps captured once into a HIP graph and replayed
(one untimed replay first); `ms_per_step_eager` is the same K steps launched call by call,
the pass in which every kernel is also timed by HIP events (`--no-graph`: eager only).
`roofline` reports the dominant kernel (the gate/up GEMM) from the HIP events of the eager
pass, recorded on the stream the library launches on, against the 5.0 PFLOP/s dense FP8
MFMA peak; `quant_roofline` the X quantizer against 8 TB/s HBM.

The default run also measures one short pass (10 steps) of each of the decode, backward and
MoE workloads with their own rooflines, under "also" (--no-also skips them); the decode
pass carries the weight-sync figures: the installed weights' error (0: the rollout runs on
the trainer's bytes, and trainer and rollout outputs are compared bit for bit) and the naive
dequantize -> bf16 -> per-tensor requantize path's mean relative error and Frobenius ratio
per weight, computed with the oracle on the host before the GPU is used.

Other workloads (--workload) time the decode, backward, MoE and weight-install paths the
same way; dense_pow2 and backward_pow2 run the dense layer with power-of-two block scales,
which the scaled MFMA applies itself; moe_block128 runs the MoE layer in the blockwise recipe. HBM-bound workloads (decode, install) cycle through copies of their inputs that
together exceed 1 GiB, so the 256 MB last-level cache cannot serve a launch from the previous
one. `roofline.traffic` is the dominant kernel's HBM bytes per launch from rocprofv3
FETCH_SIZE + WRITE_SIZE counter runs (scaled by what the same counters read for the install
copy of known size); it is reported only while the kernel's sources hash to the ones the
counters were taken on, else null.
Prints ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s (% of FP8 MFMA peak); quantizer GB/s (% of HBM)"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
ROTATE_BYTES = 1 << 30          # HBM-bound inputs cycle through at least this many bytes

CSRC = os.path.join(ROOT, "fp8_block_scaled_quant_amd", "csrc")

# HBM bytes per launch of each workload's dominant kernel, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs of this script, each scaled by the ratio of known bytes to counted bytes of the
# install copy. Keyed by the sha256 of the kernel's sources at the time of the counter runs.
# FETCH_SIZE counts half the bytes the install copy reads (factor 1.999); WRITE_SIZE counts them
# (factor 0.999). Both count L2 <-> fabric transfers, so lines served by the 256 MB
# last-level cache are included.
MEASURED_TRAFFIC = {
    "gemm_gu": {"sha": "d1d74be00594d11b", "gb": 1.6388},  # read 1.2365 + write 0.4024
    "gemm_gu_pow2": {"sha": "d1d74be00594d11b", "gb": 1.6388},  # read 1.2365 + write 0.4024
    "dgrad": {"sha": "d1d74be00594d11b", "gb": 1.3244},  # read 1.2574 + write 0.0671
    "dgrad_pow2": {"sha": "d1d74be00594d11b", "gb": 1.3240},  # read 1.2569 + write 0.0671
    "mx_fwd": {"sha": "d1d74be00594d11b", "gb": 1.6483},  # read 1.2460 + write 0.4024
    "decode_n24576": {"sha": "c2e3de9b37813cfe", "gb": 0.1221},  # read 0.1095 + write 0.0126 (the GEMM launch of the call)
    "grouped_gu": {"sha": "d1d74be00594d11b", "gb": 0.3147},  # read 0.2476 + write 0.0671
    "grouped_gu_block": {"sha": "d1d74be00594d11b", "gb": 0.3079},  # read 0.2409 + write 0.0671
    "install_gu": {"sha": "f3a49985734351c2", "gb": 0.2014},  # read 0.1007 + write 0.1007 (calibration copy)
    "swiglu_fp8": {"sha": "4ad7ed3ca95264b9", "gb": 0.6228},  # read 0.4035 + write 0.2193
    "requant_gu": {"sha": "ff1a9e3db15c1481", "gb": 0.6040},  # read 0.4026 + write 0.2014
    "quant_x": {"sha": "df969eae54a17cf5", "gb": 0.1375},  # read 0.0672 + write 0.0703
    "quant_x_pow2": {"sha": "df969eae54a17cf5", "gb": 0.1374},  # read 0.0672 + write 0.0703
    "quant_dy": {"sha": "df969eae54a17cf5", "gb": 0.8382},  # read 0.4026 + write 0.4356
    "quant_dy_pow2": {"sha": "df969eae54a17cf5", "gb": 0.8387},  # read 0.4026 + write 0.4361
    "quant_dy_mx": {"sha": "df969eae54a17cf5", "gb": 0.8399},  # read 0.4026 + write 0.4373
    "quant_xperm_mx": {"sha": "df969eae54a17cf5", "gb": 0.2038},  # read 0.1346 + write 0.0692
    "quant_xperm_rows": {"sha": "df969eae54a17cf5", "gb": 0.2038},  # read 0.1346 + write 0.0692
}


def _sources_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gemm_gu": ("gemm.hip", "device.hpp"),
    "gemm_gu_pow2": ("gemm.hip", "device.hpp"),
    "dgrad": ("gemm.hip", "device.hpp"),
    "dgrad_pow2": ("gemm.hip", "device.hpp"),
    "mx_fwd": ("gemm.hip", "device.hpp"),
    "decode_n24576": ("decode.hip", "device.hpp"),
    "grouped_gu": ("gemm.hip", "device.hpp"),
    "grouped_gu_block": ("gemm.hip", "device.hpp"),
    "install_gu": ("install.hip", "device.hpp"),
    "swiglu_fp8": ("producers.hip", "quant_kernels.hpp", "device.hpp"),
    "requant_gu": ("fp8_param.hip", "device.hpp"),
    "quant_x": ("quant.hip", "quant_kernels.hpp", "device.hpp"),
    "quant_x_pow2": ("quant.hip", "quant_kernels.hpp", "device.hpp"),
    "quant_dy": ("quant.hip", "quant_kernels.hpp", "device.hpp"),
    "quant_dy_pow2": ("quant.hip", "quant_kernels.hpp", "device.hpp"),
    "quant_dy_mx": ("quant.hip", "quant_kernels.hpp", "device.hpp"),
    "quant_xperm_mx": ("quant.hip", "quant_kernels.hpp", "device.hpp"),
    "quant_xperm_rows": ("quant.hip", "quant_kernels.hpp", "device.hpp"),
}


def _traffic(kernel):
    """(GB per launch, sources sha) if the counters were taken on the current sources, else (None, sha)."""
    sha = _sources_sha(KERNEL_SOURCES[kernel]) if kernel in KERNEL_SOURCES else None
    rec = MEASURED_TRAFFIC.get(kernel)
    if rec is not None and rec["sha"] == sha:
        return rec["gb"], sha
    return None, sha


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense", choices=["dense", "dense_pow2", "decode", "backward", "backward_pow2", "moe",
                                                         "moe_block128", "install", "producers", "mx_dense", "fp8_param"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time the eager steps only (no HIP graph replay)")
    ap.add_argument("--no-also", action="store_true",
                    help="dense workload only: skip the extra decode, backward and MoE passes")
    ap.add_argument("--no-weight-sync-errors", action="store_true",
                    help="skip the host computation of the naive weight-sync errors (decode)")
    return ap.parse_args()


class EventTimer:
    """Pairs of HIP events recorded on the current stream around one kernel's launches."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def per_launch_ms(self):
        """Median over the launches (one host stall between a pair of events, e.g. the first call
        of a pass waiting on the host, would otherwise dominate a mean over a few calls)."""
        ts = [a.elapsed_time(b) for a, b in self.pairs]
        return float(np.median(ts)) if ts else float("nan")


# ---------------------------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------------------------

def dense_setup(torch, F, W, dev, pow2=False):
    d = W.dense_forward(with_down=True)
    if pow2:
        quant_act, quant_w, gemm = F.fp8_quant_act_1x128_pow2, F.fp8_quant_w_128x128_pow2, F.fp8_gemm_blockscaled_pow2_fwd
    else:
        quant_act, quant_w, gemm = F.fp8_quant_act_1x128, F.fp8_quant_w_128x128, F.fp8_gemm_blockscaled_fwd
    t = {k: W.to_bf16_tensor(v).to(dev) for k, v in d.items()}
    M, K = t["x"].shape
    N = t["w_gu"].shape[0]
    N2, K2 = t["w_dn"].shape
    u8, f32 = torch.uint8, torch.float32
    b = dict(
        xq=torch.empty((M, K), dtype=u8, device=dev), sx=torch.empty((M, K // 128), dtype=f32, device=dev),
        xqt=torch.empty((K, M), dtype=u8, device=dev), sxt=torch.empty((K, M // 128), dtype=f32, device=dev),
        wq_gu=torch.empty((N, K), dtype=u8, device=dev), sw_gu=torch.empty((N // 128, K // 128), dtype=f32, device=dev),
        wq_dn=torch.empty((N2, K2), dtype=u8, device=dev),
        sw_dn=torch.empty((N2 // 128, K2 // 128), dtype=f32, device=dev),
        x2q=torch.empty((M, K2), dtype=u8, device=dev), sx2=torch.empty((M, K2 // 128), dtype=f32, device=dev),
        y_gu=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        y_dn=torch.empty((M, N2), dtype=torch.bfloat16, device=dev),
    )
    timers = {k: EventTimer(torch) for k in ("quant_x", "quant_w", "gemm_gu", "quant_x2", "gemm_dn")}

    def step(timed):
        tm = timers if timed else None
        if tm: tm["quant_x"].start()
        quant_act(t["x"], q=b["xq"], s=b["sx"], qt=b["xqt"], st=b["sxt"], rowwise=True, colwise=True)
        if tm: tm["quant_x"].stop(); tm["quant_w"].start()
        quant_w(t["w_gu"], q=b["wq_gu"], s=b["sw_gu"])
        quant_w(t["w_dn"], q=b["wq_dn"], s=b["sw_dn"])
        if tm: tm["quant_w"].stop(); tm["gemm_gu"].start()
        gemm(b["xq"], b["sx"], b["wq_gu"], b["sw_gu"], y=b["y_gu"])
        if tm: tm["gemm_gu"].stop(); tm["quant_x2"].start()
        quant_act(t["x2"], q=b["x2q"], s=b["sx2"])
        if tm: tm["quant_x2"].stop(); tm["gemm_dn"].start()
        gemm(b["x2q"], b["sx2"], b["wq_dn"], b["sw_dn"], y=b["y_dn"])
        if tm: tm["gemm_dn"].stop()

    flops_gu = 2.0 * M * N * K
    flops_dn = 2.0 * M * N2 * K2
    info = dict(
        config={"workload": "dense_layer_forward_9b" + ("_pow2" if pow2 else ""), "tokens_M": M, "hidden_K": K,
                "gate_up_N": N, "down_N": N2, "down_K": K2,
                "recipe": "blockwise 1x128 act / 128x128 weight, E4M3, "
                          + ("power-of-two scales applied by the scaled MFMA" if pow2 else "fp32 scales"),
                "out": "bf16"},
        flops=flops_gu + flops_dn,
        dominant=("gemm_gu", "mfma", flops_gu / 1e12, "TFLOP/s", PEAK_FP8_TFLOPS,
                  f"2*M*N*K = {flops_gu:.4g} FLOP per launch"),
        # quant X: 2 B read + 1 B row + 1 B column payload + 4 B per 128 per direction
        quant=("quant_x", (M * K * (2 + 1 + 1) + 2 * M * K // 128 * 4) / 1e9,
               "bf16 read 2 B + row and column E4M3 payloads 1 B each + fp32 scales per element"),
        gemm_keys=("gemm_gu", "gemm_dn"),
        traffic_key="gemm_gu_pow2" if pow2 else "gemm_gu",
        quant_traffic_key="quant_x_pow2" if pow2 else "quant_x",
    )
    return step, timers, info


_DECODE_DATA = {}


def decode_data(W):
    """The decode workload's synthetic activations and weights (generated once per process)."""
    if not _DECODE_DATA:
        _DECODE_DATA.update(W.decode_rollout())
    return _DECODE_DATA


def decode_setup(torch, F, W, dev):
    d = decode_data(W)
    x = W.to_bf16_tensor(d["x"]).to(dev)
    M, K = x.shape
    set_bytes = sum(n * K + (n // 128) * (K // 128) * 4 for n in W.DECODE_N)
    n_sets = -(-ROTATE_BYTES // set_bytes)
    sets = [dict() for _ in range(n_sets)]
    ys = {}
    bitwise = {}
    for n in W.DECODE_N:
        wq, sw, _ = F.fp8_quant_w_128x128(W.to_bf16_tensor(d[f"w{n}"]).to(dev))
        for st in sets:     # installed (rollout-owned) copies in the decode layout, the trainer's bytes
            iq, is_ = torch.empty_like(wq), torch.empty_like(sw)
            F.fp8_weight_install(wq, sw, iq, is_, layout=F.LAYOUT_DECODE)
            st[n] = (iq, is_)
        ys[n] = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        # trainer forward (row-major payload) vs rollout forward (installed copy), outside the timed steps
        y_train = F.fp8_gemm_blockscaled_fwd(wq=wq, sw=sw, x_bf16=x)
        y_roll = F.fp8_gemm_blockscaled_fwd_decode_layout(wq=sets[0][n][0], sw=sets[0][n][1], x_bf16=x, N=n, K=K)
        bitwise[str(n)] = bool(torch.equal(y_train.view(torch.int16), y_roll.view(torch.int16)))
        del wq, sw, y_train, y_roll
    ws = F.fwd_workspace(M, K, dev)
    timers = {f"decode_n{n}": EventTimer(torch) for n in W.DECODE_N}
    it = [0]

    def step(timed):
        st = sets[it[0] % n_sets]
        it[0] += 1
        for n, (iq, is_) in st.items():
            if timed: timers[f"decode_n{n}"].start()
            F.fp8_gemm_blockscaled_fwd_decode_layout(wq=iq, sw=is_, x_bf16=x, N=n, K=K, y=ys[n], workspace=ws)
            if timed: timers[f"decode_n{n}"].stop()

    nmax = max(W.DECODE_N)
    info = dict(
        config={"workload": "decode_rollout", "rows_M": M, "K": K, "N": list(W.DECODE_N),
                "activations": "bf16, quantized 1x128 inside each call (quantizer launch + GEMM launch)",
                "weights": "installed E4M3 128x128, decode layout (16x128 tiles in MFMA operand order)",
                "weight_copies": n_sets},
        flops=sum(2.0 * M * n * K for n in W.DECODE_N),
        dominant=(f"decode_n{nmax}", "hbm", (nmax * K + nmax * K // 128 // 128 * 4) / 1e9, "GB/s", PEAK_HBM_GBS,
                  "weight stream: E4M3 payload + fp32 block scales per call (the call is the 1x128 quantizer "
                  "launch + the GEMM launch)"),
        quant=None,
        gemm_keys=tuple(timers),
        weight_sync={"installed_rel_error": 0.0, "installed_output_bitwise_equal": bitwise},
    )
    return step, timers, info


# The naive weight-sync control ([SkyRL-FP8] "When independent quantization breaks policy
# consistency", Fig. 2): each decode weight quantized 128x128, dequantized to bf16 and
# requantized per tensor, its mean relative error and Frobenius ratio against the trainer's
# dequantized weight. Oracle arithmetic on the host, over 1024-row chunks in a process pool
# forked before the GPU is touched: pass 1 quantizes and finds the tensor maximum, pass 2
# requantizes with the tensor's scale and sums the errors.
_NAIVE_W = {}


def _naive_pass1(task):
    from oracle import quantize as OQ, weight_sync as WS
    n, r0, r1 = task
    q, s = OQ.quant_w_128x128(_NAIVE_W[n][r0:r1])
    return n, q, s, float(np.max(np.abs(WS.dequant_to_bf16(q, s))))


def _naive_pass2(task):
    from oracle import weight_sync as WS
    n, q, s, s_t = task
    q2 = WS.requant_per_tensor(WS.dequant_to_bf16(q, s), s_t)
    a = WS.weight_value_block(q, s)
    d = WS.weight_value_tensor(q2, s_t) - a
    return n, float(np.sum(np.abs(d))), float(np.sum(np.abs(a))), float(np.sum(d * d)), float(np.sum(a * a))


def naive_weight_sync_errors(W):
    import multiprocessing as mp
    from oracle import weight_sync as WS
    t0 = time.perf_counter()
    d = decode_data(W)
    _NAIVE_W.update({n: d[f"w{n}"] for n in W.DECODE_N})
    tasks = [(n, r, min(r + 1024, w.shape[0])) for n, w in _NAIVE_W.items() for r in range(0, w.shape[0], 1024)]
    procs = max(1, min(16, os.cpu_count() or 1))
    with mp.get_context("fork").Pool(procs) as pool:
        p1 = pool.map(_naive_pass1, tasks)
        amax = {}
        for n, _, _, m in p1:
            amax[n] = max(amax.get(n, 0.0), m)
        s_t = {n: WS.per_tensor_scale(amax[n]) for n in amax}
        p2 = pool.map(_naive_pass2, [(n, q, s, s_t[n]) for n, q, s, _ in p1])
    _NAIVE_W.clear()
    acc = {}
    for n, ad, aa, dd, a2 in p2:
        t = acc.setdefault(n, [0.0, 0.0, 0.0, 0.0])
        t[0] += ad; t[1] += aa; t[2] += dd; t[3] += a2
    out = {str(n): {"mean_rel_error": round(t[0] / t[1], 5), "frobenius_ratio": round(float(np.sqrt(t[2] / t[3])), 5),
                    "per_tensor_scale": float(s_t[n])} for n, t in sorted(acc.items())}
    return {"naive_rel_error": out, "processes": procs, "seconds": round(time.perf_counter() - t0, 1),
            "how": "oracle: 128x128 quantization, dequantize to bf16, per-tensor requantization (amax/448); "
                   "error = sum|w_naive - w_trainer| / sum|w_trainer|, Frobenius ratio ||w_naive - w_trainer|| / "
                   "||w_trainer||; the page quotes 0.038 on a 4B model"}


def backward_setup(torch, F, W, dev, pow2=False):
    d = W.dense_forward(with_down=False)
    if pow2:
        quant_act, quant_w = F.fp8_quant_act_1x128_pow2, F.fp8_quant_w_128x128_pow2
        dgrad, wgrad = F.fp8_gemm_blockscaled_pow2_dgrad, F.fp8_gemm_blockscaled_pow2_wgrad
    else:
        quant_act, quant_w = F.fp8_quant_act_1x128, F.fp8_quant_w_128x128
        dgrad, wgrad = F.fp8_gemm_blockscaled_dgrad, F.fp8_gemm_blockscaled_wgrad
    dy = W.to_bf16_tensor(W.dense_backward()["dy"]).to(dev)
    x = W.to_bf16_tensor(d["x"]).to(dev)
    w = W.to_bf16_tensor(d["w_gu"]).to(dev)
    M, K = x.shape
    N = w.shape[0]
    _, _, xqt, sxt = quant_act(x, rowwise=False, colwise=True)      # saved from the forward
    wq, sw, wqt = quant_w(w, transpose=True)
    u8, f32 = torch.uint8, torch.float32
    b = dict(dyq=torch.empty((M, N), dtype=u8, device=dev), sdy=torch.empty((M, N // 128), dtype=f32, device=dev),
             dyqt=torch.empty((N, M), dtype=u8, device=dev), sdyt=torch.empty((N, M // 128), dtype=f32, device=dev),
             dx=torch.empty((M, K), dtype=torch.bfloat16, device=dev), dw=torch.empty((N, K), dtype=f32, device=dev))
    timers = {k: EventTimer(torch) for k in ("quant_dy", "dgrad", "wgrad")}

    def step(timed):
        if timed: timers["quant_dy"].start()
        quant_act(dy, q=b["dyq"], s=b["sdy"], qt=b["dyqt"], st=b["sdyt"], rowwise=True, colwise=True)
        if timed: timers["quant_dy"].stop(); timers["dgrad"].start()
        dgrad(b["dyq"], b["sdy"], wqt, sw, dx=b["dx"])
        if timed: timers["dgrad"].stop(); timers["wgrad"].start()
        wgrad(b["dyqt"], b["sdyt"], xqt, sxt, dw=b["dw"])
        if timed: timers["wgrad"].stop()

    fl = 2.0 * M * N * K
    info = dict(
        config={"workload": "dense_layer_backward_gate_up" + ("_pow2" if pow2 else ""), "tokens_M": M, "N": N, "K": K,
                "scales": "power-of-two, applied by the scaled MFMA" if pow2 else "fp32", "dgrad_out": "bf16",
                "wgrad_out": "fp32"},
        flops=2 * fl,
        dominant=("dgrad", "mfma", fl / 1e12, "TFLOP/s", PEAK_FP8_TFLOPS, f"2*M*N*K = {fl:.4g} FLOP per launch"),
        quant=("quant_dy", (M * N * 4 + 2 * M * N // 128 * 4) / 1e9,
               "bf16 read 2 B + row and column E4M3 payloads + fp32 scales per element"),
        gemm_keys=("dgrad", "wgrad"),
        traffic_key="dgrad_pow2" if pow2 else "dgrad",
        quant_traffic_key="quant_dy_pow2" if pow2 else "quant_dy",
    )
    return step, timers, info


def mx_dense_setup(torch, F, W, dev):
    """The dense gate/up layer (X 8192x4096, W 24576x4096, dY 8192x24576) forward and backward
    in the MXFP8 recipe: 1x32 E8M0 groups along each GEMM's contraction dimension, so X, W and
    dY are each quantized row-wise and column-wise (32x1, transposed) from bf16; then the
    forward, DGrad and WGrad GEMMs on the scaled MFMA."""
    d = W.dense_forward(with_down=False)
    x = W.to_bf16_tensor(d["x"]).to(dev)
    w = W.to_bf16_tensor(d["w_gu"]).to(dev)
    del d
    dy = W.to_bf16_tensor(W.dense_backward()["dy"]).to(dev)
    M, K = x.shape
    N = w.shape[0]
    u8 = torch.uint8

    def qbufs(R, C):
        return (torch.empty((R, C), dtype=u8, device=dev), torch.empty((R, C // 32), dtype=u8, device=dev),
                torch.empty((C, R), dtype=u8, device=dev), torch.empty((C, R // 32), dtype=u8, device=dev))
    bx, bw, bdy = qbufs(M, K), qbufs(N, K), qbufs(M, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    timers = {k: EventTimer(torch) for k in ("quant_x", "quant_w", "fwd", "quant_dy", "dgrad", "wgrad")}

    def step(timed):
        tm = timers if timed else None
        if tm: tm["quant_x"].start()
        F.mxfp8_quant_act_1x32(x, *bx, colwise=True)
        if tm: tm["quant_x"].stop(); tm["quant_w"].start()
        F.mxfp8_quant_act_1x32(w, *bw, colwise=True)
        if tm: tm["quant_w"].stop(); tm["fwd"].start()
        F.fp8_gemm_mxfp8_fwd(bx[0], bx[1], bw[0], bw[1], y=y)
        if tm: tm["fwd"].stop(); tm["quant_dy"].start()
        F.mxfp8_quant_act_1x32(dy, *bdy, colwise=True)
        if tm: tm["quant_dy"].stop(); tm["dgrad"].start()
        F.fp8_gemm_mxfp8_dgrad(bdy[0], bdy[1], bw[2], bw[3], dx=dx)
        if tm: tm["dgrad"].stop(); tm["wgrad"].start()
        F.fp8_gemm_mxfp8_wgrad(bdy[2], bdy[3], bx[2], bx[3], dw=dw)
        if tm: tm["wgrad"].stop()

    fl = 2.0 * M * N * K
    info = dict(
        config={"workload": "dense_layer_fwd_bwd_mxfp8_9b", "tokens_M": M, "gate_up_N": N, "hidden_K": K,
                "recipe": "MXFP8: E4M3 + E8M0 per 1x32 along each contraction (32x1 transposed copies)",
                "out": "Y, dX bf16; dW fp32"},
        flops=3 * fl,
        dominant=("fwd", "mfma", fl / 1e12, "TFLOP/s", PEAK_FP8_TFLOPS, f"2*M*N*K = {fl:.4g} FLOP per launch"),
        quant=("quant_dy", (M * N * 4 + 2 * M * N // 32) / 1e9,
               "bf16 read 2 B + row and column E4M3 payloads + E8M0 scales per element"),
        gemm_keys=("fwd", "dgrad", "wgrad"),
        traffic_key="mx_fwd",
        quant_traffic_key="quant_dy_mx",
    )
    return step, timers, info


def fp8_param_setup(torch, F, W, dev):
    """fp8_param requantization after an optimizer step: the FP32 masters of the dense layer's
    gate/up (24576x4096) and down (4096x12288) weights quantized per 128x128 block into FP8
    storage, with the byte-transposed copy DGrad reads. The masters are the dense workload's
    weights in fp32 plus a small fp32 perturbation (all 24 significand bits in use)."""
    d = W.dense_forward(with_down=True)
    rng = np.random.default_rng(7)
    masters = []
    for k in ("w_gu", "w_dn"):
        m32 = d[k] + (rng.standard_normal(d[k].shape, dtype=np.float32) * np.float32(1e-6))
        masters.append(torch.from_numpy(m32.astype(np.float32)).to(dev))
    del d
    outs = []
    for m in masters:
        N, K = m.shape
        outs.append((torch.empty((N, K), dtype=torch.uint8, device=dev),
                     torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev),
                     torch.empty((K, N), dtype=torch.uint8, device=dev)))
    timers = {k: EventTimer(torch) for k in ("requant_gu", "requant_dn")}

    def step(timed):
        for name, m, (q, s_, qt) in zip(("requant_gu", "requant_dn"), masters, outs):
            if timed: timers[name].start()
            F.fp8_quant_w_128x128_f32(m, q=q, s=s_, qt=qt, transpose=True)
            if timed: timers[name].stop()

    per = [m.numel() * (4 + 2) + (m.numel() // (128 * 128)) * 4 for m in masters]
    info = dict(
        config={"workload": "fp8_param_requant_dense_layer_9b", "masters": ["gate_up 24576x4096 fp32",
                                                                          "down 4096x12288 fp32"],
                "recipe": "128x128 blocks, fp32 scales, row + byte-transposed E4M3"},
        flops=None,
        bytes=sum(per),
        dominant=("requant_gu", "hbm", per[0] / 1e9, "GB/s", PEAK_HBM_GBS,
                  f"fp32 read 4 B + E4M3 row and transposed copies 2 B per element + scales = {per[0]} B"),
        quant=None,
        gemm_keys=(),
    )
    return step, timers, info


def moe_setup(torch, F, W, dev):
    d = W.moe_mxfp8()
    xp = W.to_bf16_tensor(d["x_perm"]).to(dev)
    h = W.to_bf16_tensor(d["h"]).to(dev)
    wq_gu, sw_gu = F.mxfp8_quant_1x32(W.to_bf16_tensor(d["w_gu"]).to(dev))
    wq_dn, sw_dn = F.mxfp8_quant_1x32(W.to_bf16_tensor(d["w_dn"]).to(dev))
    off = torch.from_numpy(d["offsets"]).to(dev)
    T, K = xp.shape
    E, N, _ = wq_gu.shape
    _, N2, K2 = wq_dn.shape
    u8 = torch.uint8
    b = dict(xq=torch.empty((T, K), dtype=u8, device=dev), sx=torch.empty((T, K // 32), dtype=u8, device=dev),
             hq=torch.empty((T, K2), dtype=u8, device=dev), sh=torch.empty((T, K2 // 32), dtype=u8, device=dev),
             y_gu=torch.empty((T, N), dtype=torch.bfloat16, device=dev),
             y_dn=torch.empty((T, N2), dtype=torch.bfloat16, device=dev))
    timers = {k: EventTimer(torch) for k in ("quant_x", "grouped_gu", "quant_h", "grouped_dn")}

    def step(timed):
        if timed: timers["quant_x"].start()
        F.mxfp8_quant_1x32(xp, q=b["xq"], e8m0=b["sx"])
        if timed: timers["quant_x"].stop(); timers["grouped_gu"].start()
        F.fp8_grouped_gemm(b["xq"], b["sx"], wq_gu, sw_gu, off, y=b["y_gu"])
        if timed: timers["grouped_gu"].stop(); timers["quant_h"].start()
        F.mxfp8_quant_1x32(h, q=b["hq"], e8m0=b["sh"])
        if timed: timers["quant_h"].stop(); timers["grouped_dn"].start()
        F.fp8_grouped_gemm(b["hq"], b["sh"], wq_dn, sw_dn, off, y=b["y_dn"])
        if timed: timers["grouped_dn"].stop()

    fl_gu, fl_dn = 2.0 * T * N * K, 2.0 * T * N2 * K2
    info = dict(
        config={"workload": "moe_mxfp8_grouped", "routed_rows_T": T, "experts": E, "gate_up": [N, K],
                "down": [N2, K2], "routing": "Zipf(1.1) top-8",
                "weights": "expert weights MXFP8-quantized once before the timed steps (as installed for a rollout); "
                           "the step quantizes the activations and runs both grouped GEMMs"},
        flops=fl_gu + fl_dn,
        dominant=("grouped_gu", "mfma", fl_gu / 1e12, "TFLOP/s", PEAK_FP8_TFLOPS,
                  f"2*T*N*K = {fl_gu:.4g} FLOP per launch"),
        quant=("quant_x", T * K * (2 + 1 + 1 / 32) / 1e9, "bf16 read 2 B + E4M3 1 B + E8M0 1/32 B per element"),
        quant_traffic_key="quant_xperm_mx",
        gemm_keys=("grouped_gu", "grouped_dn"),
        # X_perm and the expert stack once (E4M3 + E8M0) and Y once (bf16)
        algorithmic_gb=(T * K * (1 + 1 / 32) + E * N * K * (1 + 1 / 32) + T * N * 2) / 1e9,
    )
    return step, timers, info


def moe_block128_setup(torch, F, W, dev):
    """The MoE layer of the MXFP8 workload (same routed rows, experts and weights) in the
    blockwise recipe: activations in 1x128 groups, each expert's weights in 128x128 blocks."""
    d = W.moe_mxfp8()
    xp = W.to_bf16_tensor(d["x_perm"]).to(dev)
    h = W.to_bf16_tensor(d["h"]).to(dev)
    E, N, K = d["w_gu"].shape
    _, N2, K2 = d["w_dn"].shape
    wq_gu, sw_gu, _ = F.fp8_quant_w_128x128(W.to_bf16_tensor(d["w_gu"].reshape(E * N, K)).to(dev))
    wq_dn, sw_dn, _ = F.fp8_quant_w_128x128(W.to_bf16_tensor(d["w_dn"].reshape(E * N2, K2)).to(dev))
    wq_gu, sw_gu = wq_gu.view(E, N, K), sw_gu.view(E, N // 128, K // 128)
    wq_dn, sw_dn = wq_dn.view(E, N2, K2), sw_dn.view(E, N2 // 128, K2 // 128)
    off = torch.from_numpy(d["offsets"]).to(dev)
    T = xp.shape[0]
    u8, f32 = torch.uint8, torch.float32
    b = dict(xq=torch.empty((T, K), dtype=u8, device=dev), sx=torch.empty((T, K // 128), dtype=f32, device=dev),
             hq=torch.empty((T, K2), dtype=u8, device=dev), sh=torch.empty((T, K2 // 128), dtype=f32, device=dev),
             y_gu=torch.empty((T, N), dtype=torch.bfloat16, device=dev),
             y_dn=torch.empty((T, N2), dtype=torch.bfloat16, device=dev))
    timers = {k: EventTimer(torch) for k in ("quant_x", "grouped_gu", "quant_h", "grouped_dn")}
    blk = F.RECIPE_BLOCK128

    def step(timed):
        if timed: timers["quant_x"].start()
        F.fp8_quant_act_1x128(xp, q=b["xq"], s=b["sx"])
        if timed: timers["quant_x"].stop(); timers["grouped_gu"].start()
        F.fp8_grouped_gemm(b["xq"], b["sx"], wq_gu, sw_gu, off, recipe=blk, y=b["y_gu"])
        if timed: timers["grouped_gu"].stop(); timers["quant_h"].start()
        F.fp8_quant_act_1x128(h, q=b["hq"], s=b["sh"])
        if timed: timers["quant_h"].stop(); timers["grouped_dn"].start()
        F.fp8_grouped_gemm(b["hq"], b["sh"], wq_dn, sw_dn, off, recipe=blk, y=b["y_dn"])
        if timed: timers["grouped_dn"].stop()

    fl_gu, fl_dn = 2.0 * T * N * K, 2.0 * T * N2 * K2
    info = dict(
        config={"workload": "moe_block128_grouped", "routed_rows_T": T, "experts": E, "gate_up": [N, K],
                "down": [N2, K2], "routing": "Zipf(1.1) top-8"},
        flops=fl_gu + fl_dn,
        dominant=("grouped_gu", "mfma", fl_gu / 1e12, "TFLOP/s", PEAK_FP8_TFLOPS,
                  f"2*T*N*K = {fl_gu:.4g} FLOP per launch"),
        quant=("quant_x", T * K * (2 + 1 + 4 / 128) / 1e9, "bf16 read 2 B + E4M3 1 B + fp32 scale 4/128 B per element"),
        quant_traffic_key="quant_xperm_rows",
        gemm_keys=("grouped_gu", "grouped_dn"),
        # X_perm once (E4M3 + fp32 1x128 scales), the expert stack once (E4M3 + fp32 128x128
        # block scales) and Y once (bf16)
        algorithmic_gb=(T * K * (1 + 4 / 128) + E * N * K * (1 + 4 / 128 ** 2) + T * N * 2) / 1e9,
        traffic_key="grouped_gu_block",
    )
    return step, timers, info


def install_setup(torch, F, W, dev):
    """Weight install of the dense layer's gate/up and down weights (payload + fp32 block scales),
    the rollout side's whole per-sync work for that layer. A plain copy of known size, so its
    counter readings also calibrate the FETCH_SIZE / WRITE_SIZE figures of the other kernels."""
    d = W.dense_forward(with_down=True)
    srcs = []
    for k in ("w_gu", "w_dn"):
        wq, sw, _ = F.fp8_quant_w_128x128(W.to_bf16_tensor(d[k]).to(dev))
        srcs.append((wq, sw))
    del d
    per_set = sum(q.numel() + s_.numel() * 4 for q, s_ in srcs)
    n_sets = -(-ROTATE_BYTES // (2 * per_set))
    pairs = []
    for _ in range(n_sets):
        pairs.append([(q.clone(), s_.clone(), torch.empty_like(q), torch.empty_like(s_)) for q, s_ in srcs])
    del srcs
    names = ("install_gu", "install_dn")
    timers = {k: EventTimer(torch) for k in names}
    it = [0]

    def step(timed):
        ps = pairs[it[0] % n_sets]
        it[0] += 1
        for k, (sq, ss, dq, ds) in zip(names, ps):
            if timed: timers[k].start()
            F.fp8_weight_install(sq, ss, dq, ds)
            if timed: timers[k].stop()

    gu_bytes = 2 * (pairs[0][0][0].numel() + pairs[0][0][1].numel() * 4)
    info = dict(
        config={"workload": "weight_install_dense_layer_9b", "tensors": ["gate_up 24576x4096", "down 4096x12288"],
                "recipe": "blockwise 128x128, E4M3 payload + fp32 scales", "copies": n_sets},
        flops=None,
        bytes=2 * per_set,
        dominant=("install_gu", "hbm", gu_bytes / 1e9, "GB/s", PEAK_HBM_GBS,
                  f"read + write of the gate/up payload and scales = {gu_bytes} B per launch"),
        quant=None,
        gemm_keys=(),
    )
    return step, timers, info


def producers_setup(torch, F, W, dev):
    """The fused producers of the dense layer, each writing the row-wise FP8 copy the next
    GEMM reads and the column-wise (128x1, transposed) copy its WGrad reads:
    RMSNorm of the residual stream X 8192x4096 -> FP8 (input of the gate/up GEMM), and
    SwiGLU of the gate/up output GU 8192x24576 -> FP8 H 8192x12288 (input of the down GEMM).
    The unfused chains (bf16 producer, then the quantizer) are timed after the timed steps
    for comparison."""
    d = W.fused_producers()
    gu = W.to_bf16_tensor(d["gu"]).to(dev)
    x0 = W.to_bf16_tensor(d["x"]).to(dev)
    gamma = W.to_bf16_tensor(d["gamma"]).to(dev)
    eps = d["eps"]
    del d
    M, F2 = gu.shape
    Fh = F2 // 2
    K = x0.shape[1]
    n_x = max(1, -(-ROTATE_BYTES // (x0.numel() * 2)))          # X copies: the step reads >= 1 GiB of X
    xs = [x0.clone() for _ in range(n_x)]
    del x0
    u8, f32 = torch.uint8, torch.float32
    b = dict(hq=torch.empty((M, Fh), dtype=u8, device=dev), hs=torch.empty((M, Fh // 128), dtype=f32, device=dev),
             hqt=torch.empty((Fh, M), dtype=u8, device=dev), hst=torch.empty((Fh, M // 128), dtype=f32, device=dev),
             xq=torch.empty((M, K), dtype=u8, device=dev), xs=torch.empty((M, K // 128), dtype=f32, device=dev),
             xqt=torch.empty((K, M), dtype=u8, device=dev), xst=torch.empty((K, M // 128), dtype=f32, device=dev),
             rstd=torch.empty((M,), dtype=f32, device=dev))
    timers = {k: EventTimer(torch) for k in ("rmsnorm_fp8", "swiglu_fp8")}
    it = [0]

    def step(timed):
        x = xs[it[0] % n_x]
        it[0] += 1
        if timed: timers["rmsnorm_fp8"].start()
        F.fp8_rmsnorm_quant_1x128(x, gamma, eps, q=b["xq"], s=b["xs"], qt=b["xqt"], st=b["xst"], rstd=b["rstd"],
                                  colwise=True)
        if timed: timers["rmsnorm_fp8"].stop(); timers["swiglu_fp8"].start()
        F.fp8_swiglu_quant_1x128(gu, q=b["hq"], s=b["hs"], qt=b["hqt"], st=b["hst"], colwise=True)
        if timed: timers["swiglu_fp8"].stop()

    def unfused(reps=10):
        """Mean microseconds of the unfused chains: bf16 producer, then the quantizer."""
        t = {k: EventTimer(torch) for k in ("rmsnorm_bf16", "quant_y", "swiglu_bf16", "quant_h")}
        h = torch.empty((M, Fh), dtype=torch.bfloat16, device=dev)
        y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        for i in range(reps + 2):
            x = xs[i % n_x]
            tm = t if i >= 2 else None
            if tm: tm["rmsnorm_bf16"].start()
            F.fp8_rmsnorm_bf16(x, gamma, eps, y=y, rstd=b["rstd"])
            if tm: tm["rmsnorm_bf16"].stop(); tm["quant_y"].start()
            F.fp8_quant_act_1x128(y, q=b["xq"], s=b["xs"], qt=b["xqt"], st=b["xst"], colwise=True)
            if tm: tm["quant_y"].stop(); tm["swiglu_bf16"].start()
            F.fp8_swiglu_bf16(gu, h=h)
            if tm: tm["swiglu_bf16"].stop(); tm["quant_h"].start()
            F.fp8_quant_act_1x128(h, q=b["hq"], s=b["hs"], qt=b["hqt"], st=b["hst"], colwise=True)
            if tm: tm["quant_h"].stop()
        torch.cuda.synchronize()
        return {k: round(v.per_launch_ms() * 1e3, 2) for k, v in t.items()}

    # algorithmic bytes: bf16 inputs once, both FP8 copies, both scale sets (+ gamma, r)
    sw_bytes = M * F2 * 2 + 2 * M * Fh + 2 * (M * Fh // 128) * 4
    rms_bytes = M * K * 2 + K * 2 + 2 * M * K + 2 * (M * K // 128) * 4 + M * 4
    info = dict(
        config={"workload": "fused_producers_dense_layer_9b", "rmsnorm": f"X {M}x{K} -> FP8 rows + cols",
                "swiglu": f"GU {M}x{F2} -> FP8 H {M}x{Fh} rows + cols", "recipe": "1x128 / 128x1, fp32 scales",
                "x_copies": n_x},
        flops=None,
        bytes=sw_bytes + rms_bytes,
        dominant=("swiglu_fp8", "hbm", sw_bytes / 1e9, "GB/s", PEAK_HBM_GBS,
                  f"bf16 GU read 4 B + two E4M3 copies 2 B + fp32 scales per output element = {sw_bytes} B"),
        quant=("rmsnorm_fp8", rms_bytes / 1e9, "bf16 X read 2 B + two E4M3 copies 2 B + scales and r per element"),
        gemm_keys=(),
        extra=unfused,
    )
    return step, timers, info


# ---------------------------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample of the same workload
# ---------------------------------------------------------------------------------------------

def _repeat(chunk, budget_s):
    reps = 0
    t0 = time.perf_counter()
    while True:
        chunk()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            return reps, dt


def cpu_baseline(workload: str, budget_s: float = 12.0):
    """Time the oracle (as it stands) on a bounded sample of the workload: one chunk of the
    layer, repeated until about `budget_s` seconds of CPU work have been done."""
    import workloads as W
    from oracle import gemm as OG
    from oracle import quantize as OQ
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    if workload == "producers":
        from oracle import producers as OP
        m, f, k = 128, 12288, 4096
        gu = W.bf16_round(rng.standard_normal((m, 2 * f)).astype(np.float32))
        x = W.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
        gamma = W.bf16_round(np.float32(1.0) + rng.standard_normal(k).astype(np.float32) * np.float32(0.1))
        nbytes = (m * 2 * f * 2 + 2 * m * f + 2 * (m * f // 128) * 4) + (m * k * 2 + 2 * m * k + 2 * (m * k // 128) * 4)
        OP.silu_bf16_table()                       # built once per process, outside the timing

        def chunk():
            OP.swiglu_quant_1x128(gu, colwise=True)
            OP.rmsnorm_quant_1x128(x, gamma, 1e-6, colwise=True)
        reps, dt = _repeat(chunk, budget_s)
        return {"value": reps * nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{reps} x oracle SwiGLU -> FP8 (rows + cols) of GU {m}x{2 * f} and RMSNorm -> FP8 "
                          f"(rows + cols) of X {m}x{k}, 128 token rows of the dense layer", "seconds": round(dt, 2)}
    if workload == "mx_dense":
        m, n, k = 256, 2048, 4096
        x = W.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
        w = W.bf16_round(rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02))

        def chunk():
            xq, ex = OQ.quant_mx_1x32(x)
            wq, ew = OQ.quant_mx_1x32(w)
            OG.gemm_mx_fwd(xq, ex, wq, ew)
        reps, dt = _repeat(chunk, budget_s)
        return {"value": reps * 2.0 * m * n * k / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
                "kind": "oracle", "sample": f"{reps} x oracle MXFP8 quantization of both operands + fp64 dequantized "
                f"forward GEMM, {m}x{n}x{k} chunk of the gate/up layer", "seconds": round(dt, 2)}
    if workload == "moe":
        m, n, k = 512, 1024, 2048
        x = W.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
        w = W.bf16_round(rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02))

        def chunk():
            xq, ex = OQ.quant_mx_1x32(x)
            wq, ew = OQ.quant_mx_1x32(w)
            OG.grouped_gemm_mx(xq, ex, wq[None], ew[None], np.array([0, m], np.int64))
        what = f"oracle MXFP8 quantization of both operands + fp64 dequantized GEMM, {m}x{n}x{k} (one expert)"
    elif workload == "moe_block128":
        m, n, k = 512, 1024, 2048
        x = W.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
        w = W.bf16_round(rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02))

        def chunk():
            xq, sx = OQ.quant_act_1x128(x)
            wq, sw = OQ.quant_w_128x128(w)
            OG.grouped_gemm_block(xq, sx, wq[None], sw[None], np.array([0, m], np.int64))
        what = f"oracle 1x128 / 128x128 quantization + fp64 dequantized GEMM, {m}x{n}x{k} (one expert)"
    else:
        # 256 token rows x 2048 output features of the dense gate/up projection, K = 4096
        m, n, k = 256, 2048, 4096
        x = W.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
        w = W.bf16_round(rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02))

        pow2 = workload.endswith("_pow2")
        quant_act = OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128
        quant_w = OQ.quant_w_128x128_pow2 if pow2 else OQ.quant_w_128x128

        def chunk():
            xq, sx = quant_act(x)
            wq, sw = quant_w(w)
            OG.gemm_fwd(xq, sx, wq, sw)
        what = (f"oracle 1x128 + 128x128 {'power-of-two scale ' if pow2 else ''}quantization and fp64 dequantized "
                f"GEMM, {m}x{n}x{k} chunk of the gate/up layer")
    reps, dt = _repeat(chunk, budget_s)
    return {"value": reps * 2.0 * m * n * k / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} x {what}", "seconds": round(dt, 2)}


def measure(workload, steps, warmup, no_graph, torch, F, W, dev):
    """Set up one workload, run `warmup` untimed steps, time `steps` eager steps (HIP events around
    every kernel on the library's stream), then the next `steps` steps captured into one HIP
    graph (one untimed replay, one timed replay). Returns the workload's part of the JSON line."""
    setup = {"dense": dense_setup, "dense_pow2": lambda *args: dense_setup(*args, pow2=True), "decode": decode_setup,
             "backward": backward_setup, "backward_pow2": lambda *args: backward_setup(*args, pow2=True),
             "moe": moe_setup, "moe_block128": moe_block128_setup, "install": install_setup,
             "producers": producers_setup, "mx_dense": mx_dense_setup, "fp8_param": fp8_param_setup}[workload]
    step, timers, info = setup(torch, F, W, dev)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    ms_per_step_eager = (time.perf_counter() - t0) / steps * 1e3
    ms_per_step = ms_per_step_eager
    if not no_graph:
        # The same calls (continuing any input rotation) captured once, which removes the launch
        # gaps between dependent kernels.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                step(False)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) / steps * 1e3
        del graph

    breakdown = {k: round(v.per_launch_ms() * 1e3, 2) for k, v in timers.items()}          # microseconds
    name, bound, per_launch, unit, peak, per_unit = info["dominant"]
    dom_ms = timers[name].per_launch_ms()
    achieved = per_launch / (dom_ms * 1e-3)
    gemm_ms = sum(timers[k].per_launch_ms() for k in info["gemm_keys"])
    traffic, sha = _traffic(info.get("traffic_key", name))
    if info["flops"] is not None:
        value, vunit = round(info["flops"] / (ms_per_step * 1e-3) / 1e12, 2), "TFLOP/s"
    else:
        value, vunit = round(info["bytes"] / (ms_per_step * 1e-3) / 1e9, 1), "GB/s"
    rec = {
        "value": value,
        "unit": vunit,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(ms_per_step_eager, 4),
        "step_launch": "eager" if no_graph else "hip_graph",
        "config": info["config"],
        "roofline": {"bound": bound, "kernel": name, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic, "traffic_unit": "GB per launch (HBM)",
                     "sources_sha": sha, "per_launch": per_unit},
        "kernel_us": breakdown,
    }
    if info["gemm_keys"]:
        rec["gemm_tflops"] = round(info["flops"] / (gemm_ms * 1e-3) / 1e12, 2)
    if info["quant"] is not None:
        qname, qgb, qdesc = info["quant"]
        qms = timers[qname].per_launch_ms()
        qkey = info.get("quant_traffic_key")
        qtraffic, qsha = _traffic(qkey) if qkey else (None, None)
        rec["quant_roofline"] = {"bound": "hbm", "kernel": qname, "achieved": round(qgb / (qms * 1e-3), 1),
                                 "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(qgb / (qms * 1e-3) / PEAK_HBM_GBS, 4),
                                 "traffic": qtraffic, "traffic_unit": "GB per launch (HBM)", "sources_sha": qsha,
                                 "per_launch": qdesc}
    if "algorithmic_gb" in info:
        # A GEMM whose arithmetic intensity sits below the ridge (flops per HBM byte under
        # peak FLOP/s / peak B/s) cannot reach the MFMA peak: report the attainable rate too.
        ai = info["dominant"][2] * 1e12 / (info["algorithmic_gb"] * 1e9)
        attainable = min(peak, ai * PEAK_HBM_GBS / 1e3)
        rec["roofline"]["arithmetic_intensity"] = round(ai, 1)
        rec["roofline"]["attainable"] = round(attainable, 1)
        rec["roofline"]["frac_attainable"] = round(achieved / attainable, 4)
    if "extra" in info:
        rec["unfused_kernel_us"] = info["extra"]()
    if "weight_sync" in info:
        rec["weight_sync"] = info["weight_sync"]
    return rec


# Workloads the default run (the dense layer) also measures, one short pass each, so that
# one line carries the decode, backward and MoE figures next to the headline.
ALSO = ("decode", "backward", "moe")


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the path runs on a single MI355X).",
              file=sys.stderr)
        sys.exit(2)
    import workloads as W

    also = ALSO if (a.workload == "dense" and not a.no_also) else ()
    naive = None
    if (a.workload == "decode" or "decode" in also) and not a.no_weight_sync_errors:
        naive = naive_weight_sync_errors(W)      # host work in forked processes, before any GPU use

    import gc

    import torch

    import fp8_block_scaled_quant_amd as F

    dev = torch.device("cuda", 0)
    F.load_library()
    rec = measure(a.workload, a.steps, a.warmup, a.no_graph, torch, F, W, dev)
    out = {"metric": METRIC, "value": rec.pop("value"), "unit": rec.pop("unit"), "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": rec.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8_e4m3 x fp8_e4m3 -> fp32 accumulate", "data": "synthetic"}
    out.update(rec)
    if a.workload == "decode" and naive:
        out["weight_sync"].update(naive)
    if also:
        out["also"] = {}
        for wl in also:
            gc.collect()
            torch.cuda.empty_cache()
            steps, warmup = min(a.steps, 10), min(a.warmup, 2)
            r = measure(wl, steps, warmup, a.no_graph, torch, F, W, dev)
            r["steps"], r["warmup"] = steps, warmup
            if wl == "decode" and naive:
                r["weight_sync"].update(naive)
            out["also"][wl] = r
    if not a.no_cpu_baseline and a.workload not in ("install", "fp8_param"):
        out["cpu_baseline"] = cpu_baseline(a.workload)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
