"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds only input recipes (random draws, outlier injection, bf16
storage of the draws, MoE routing); it contains none of the quantization or
GEMM arithmetic. Both the CPU oracle's callers and the HIP path's callers take
their inputs from here, so the two sides always see the same bytes.

Recipe: ``numpy.random.default_rng([config, tensor_id])``; draws are
``standard_normal(float32) * sigma``; outlier multipliers are applied in fp32;
then each value is rounded once to bf16 (round to nearest even). Arrays are
returned as float32 holding bf16-exact values (``to_bf16_tensor`` gives the
torch bf16 tensor of the same values).

Workload shapes follow the pages' settings: a ~9B dense layer's linear GEMMs,
32 prompts x 8 samples for decode, and a routed-expert MoE layer.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round", "normal_bf16", "with_outlier_entries", "with_outlier_channels",
    "zipf_topk_routing", "to_bf16_tensor",
    "tiny_forward", "dense_forward", "decode_rollout", "dense_backward", "moe_mxfp8",
]


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Store fp32 draws as bf16 (round to nearest even) and return them as fp32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def to_bf16_tensor(a: np.ndarray):
    """torch bf16 CPU tensor holding the same (bf16-exact) values."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _rng(config: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([config, tid])


def _normal32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)


def normal_bf16(shape, sigma: float, config: int, tid: int) -> np.ndarray:
    """N(0, sigma^2) draws stored as bf16."""
    return bf16_round(_normal32(_rng(config, tid), shape, sigma))


def with_outlier_entries(a32: np.ndarray, frac: float, mult: float, rng: np.random.Generator) -> np.ndarray:
    """Multiply round(frac * size) entries, chosen without replacement, by ``mult`` (fp32, in place)."""
    n = int(np.rint(frac * a32.size))
    idx = rng.choice(a32.size, size=n, replace=False)
    flat = a32.reshape(-1)
    flat[idx] *= np.float32(mult)
    return a32


def with_outlier_channels(a32: np.ndarray, frac: float, mult: float, rng: np.random.Generator) -> np.ndarray:
    """Multiply round(frac * K) columns (channels), chosen without replacement, by ``mult`` (fp32, in place)."""
    K = a32.shape[1]
    n = int(np.rint(frac * K))
    cols = np.sort(rng.choice(K, size=n, replace=False))
    a32[:, cols] *= np.float32(mult)
    return a32


def zipf_topk_routing(n_tokens: int, n_experts: int, topk: int, alpha: float, rng: np.random.Generator):
    """Zipf(alpha)-skewed top-k routing.

    Expert e has weight p_e proportional to r_e**-alpha over a seeded rank
    permutation r. Each token takes ``topk`` distinct experts by Gumbel-top-k on
    log p (sampling without replacement). Routed rows are grouped by expert
    (ascending), tokens ascending within an expert.

    Returns (perm int64 [n_tokens*topk]: source token of each routed row,
    offsets int32 [n_experts+1]).
    """
    ranks = rng.permutation(n_experts) + 1
    logp = -alpha * np.log(ranks.astype(np.float64))
    logp -= np.log(np.sum(np.exp(logp)))
    scores = logp[None, :] + rng.gumbel(size=(n_tokens, n_experts))
    chosen = np.argsort(-scores, axis=1, kind="stable")[:, :topk]          # [tokens][topk]
    tok = np.repeat(np.arange(n_tokens, dtype=np.int64), topk)
    exp = chosen.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, exp))                                          # by expert, then token
    perm = tok[order]
    counts = np.bincount(exp, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return perm, offsets


# --------------------------------------------------------------------------------------
# The five workloads. Each returns a dict of float32 (bf16-exact) arrays plus metadata.
# --------------------------------------------------------------------------------------

def tiny_forward():
    """Tiny blockwise forward: X 256x512 ~ N(0,1); W 512x512 ~ N(0,0.02) with 1% of
    entries multiplied by 20."""
    x = normal_bf16((256, 512), 1.0, 1, 0)
    w32 = _normal32(_rng(1, 1), (512, 512), 0.02)
    w32 = with_outlier_entries(w32, 0.01, 20.0, _rng(1, 2))
    return {"x": x, "w": bf16_round(w32)}


def dense_forward(with_down: bool = True):
    """Dense layer shaped like a ~9B model's MLP: X 8192x4096 ~ N(0,1) with 0.1% of
    channels x50; fused gate/up W 24576x4096 and down W 4096x12288 ~ N(0,0.02);
    the down projection's input X2 8192x12288 ~ N(0,1) with 0.1% channels x50."""
    x32 = _normal32(_rng(2, 0), (8192, 4096), 1.0)
    x = bf16_round(with_outlier_channels(x32, 0.001, 50.0, _rng(2, 1)))
    del x32
    out = {"x": x, "w_gu": normal_bf16((24576, 4096), 0.02, 2, 2)}
    if with_down:
        out["w_dn"] = normal_bf16((4096, 12288), 0.02, 2, 3)
        x2 = _normal32(_rng(2, 4), (8192, 12288), 1.0)
        out["x2"] = bf16_round(with_outlier_channels(x2, 0.001, 50.0, _rng(2, 5)))
    return out


DECODE_N = (4096, 12288, 24576)


def decode_rollout(ns=DECODE_N):
    """Decode step: 32 prompts x 8 samples = 256 rows, K = 4096, N in {4096, 12288, 24576}."""
    out = {"x": normal_bf16((256, 4096), 1.0, 3, 0)}
    for i, n in enumerate(DECODE_N):
        if n in ns:
            out[f"w{n}"] = normal_bf16((n, 4096), 0.02, 3, 1 + i)
    return out


def dense_backward():
    """Backward of the dense gate/up layer: dY 8192x24576 ~ N(0, 1e-3); X and W_gu from
    the dense forward workload."""
    return {"dy": normal_bf16((8192, 24576), 1e-3, 4, 0)}


def moe_mxfp8(n_tokens=4096, hidden=2048, n_experts=64, topk=8, n_gu=1024, n_dn=2048, k_dn=512, alpha=1.1,
              config=5):
    """MoE layer, MXFP8 recipe: tokens ~ N(0,1), Zipf(1.1) top-8 routing over 64 experts,
    per-expert gate/up W [1024][2048] and down W [2048][512] ~ N(0,0.02), down input
    H [T*8][512] ~ N(0,1)."""
    x = normal_bf16((n_tokens, hidden), 1.0, config, 0)
    perm, offsets = zipf_topk_routing(n_tokens, n_experts, topk, alpha, _rng(config, 1))
    return {
        "x": x, "perm": perm, "offsets": offsets, "x_perm": np.ascontiguousarray(x[perm]),
        "w_gu": normal_bf16((n_experts, n_gu, hidden), 0.02, config, 2),
        "w_dn": normal_bf16((n_experts, n_dn, k_dn), 0.02, config, 3),
        "h": normal_bf16((n_tokens * topk, k_dn), 1.0, config, 4),
    }


def fused_producers(m=8192, hidden=4096, f=12288, config=6):
    """Inputs of the fused producers in the dense layer: the gate/up GEMM output
    GU [M][2F] = [gate | up] ~ N(0,1) with 0.1% of channels x50 (the SwiGLU producer's
    input, M = 8192 tokens, F = 12288), the residual stream X [M][4096] ~ N(0,1) with 0.1%
    of channels x50 and the RMSNorm weight gamma [4096] = 1 + N(0, 0.1) (the RMSNorm
    producer's inputs); eps = 1e-6."""
    gu32 = _normal32(_rng(config, 0), (m, 2 * f), 1.0)
    gu = bf16_round(with_outlier_channels(gu32, 0.001, 50.0, _rng(config, 1)))
    del gu32
    x32 = _normal32(_rng(config, 2), (m, hidden), 1.0)
    x = bf16_round(with_outlier_channels(x32, 0.001, 50.0, _rng(config, 3)))
    gamma = bf16_round(np.float32(1.0) + _normal32(_rng(config, 4), (hidden,), 0.1))
    return {"gu": gu, "x": x, "gamma": gamma, "eps": 1e-6}
