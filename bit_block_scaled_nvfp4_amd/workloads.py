"""Seeded synthetic inputs for the NVFP4 quantize + GEMM path.

This module only draws random numbers and casts them; it holds none of the
quantization or GEMM arithmetic, so both the HIP path and the CPU oracle may
use it.  Everything is generated on the host with numpy's PCG64
(``numpy.random.default_rng``) in float32 and then rounded to BF16 with
torch's round-to-nearest-even cast, so the same host bytes feed both sides.

The workloads stand in for the layers the pages talk about (no datasets or
trained weights are needed or used):

* ``tiny``: a 256x256 by 256x256 FP32 product, seed 0.
* ``fprop_3b``: one linear layer of a ~3B transformer (the model size of
  "Full-Stack FP4 ...", section 4): X 8192x3072 (batch 4 x seq 2048), 1% of
  columns x20 as outlier channels; W 3072x3072 with std 0.02.
* ``mlp_up_12b``: the MLP up-projection of a 12B hybrid model ("NVFP4 Treina
  com Precisao de 16 Bits ...", TL;DR): X 16384x5120 with 0.5% of columns x30,
  W 20480x5120 with std 0.015.
* ``linear_train``: a full linear training step, M=8192, K=N=4096; X N(0,1),
  W std 0.02, dY a Student-t(3) gradient scaled by 1e-3 (heavy tailed).
* ``attn_scores``: attention scores QK^T ("Full-Stack FP4 ...", section 2.4):
  Q, K [4][32][4096][128], each (batch, head) slice scaled by a per-head RMS
  drawn log-uniformly in [0.5, 4].
* ``attn_bwd``: the backward through dS of the same attention: Q, K as
  above and dS [128][4096][4096], N(0, 1) times 1e-4 times a per-head factor
  log-uniform in [0.25, 4].
* ``adamw_state``: FP32 AdamW moments m, v of a 20480x5120 weight, heavy
  tailed with a per-row gradient scale.
* ``ns_3b``: a 3072x8192 BF16 weight gradient for Newton-Schulz in NVFP4.
* ``lora_3b``: the fprop_3b layer split as W_res + beta L2 L1, rank 64.
"""
from __future__ import annotations

import os

import numpy as np
import torch


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 numpy array -> torch.bfloat16 CPU tensor (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw BF16 bit patterns of a CPU bfloat16 tensor as numpy uint16."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def normal(shape, seed: int, std: float = 1.0, outlier_frac: float = 0.0,
           outlier_scale: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) with round(outlier_frac * cols) distinct columns
    multiplied by outlier_scale."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_frac > 0.0:
        cols = shape[-1]
        k = int(round(outlier_frac * cols))
        idx = rng.choice(cols, k, replace=False)
        x[..., idx] *= np.float32(outlier_scale)
    return x


def student_t(shape, seed: int, df: float = 3.0, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_t(df, size=shape) * scale).astype(np.float32)


# --- the five workloads ----------------------------------------------------

def tiny(seed: int = 0):
    """A and B, 256x256 FP32 N(0,1), drawn in that order.  B is K x N."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((256, 256)).astype(np.float32)
    b = rng.standard_normal((256, 256)).astype(np.float32)
    return {"A": torch.from_numpy(a), "B": torch.from_numpy(b)}


def fprop_3b(seed: int = 1, m: int = 8192, k: int = 3072, n: int = 3072):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    idx = rng.choice(k, int(round(0.01 * k)), replace=False)
    x[:, idx] *= np.float32(20.0)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return {"X": to_bf16(x), "W": to_bf16(w)}


def mlp_up_12b(seed: int = 2, m: int = 16384, k: int = 5120, n: int = 20480):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    idx = rng.choice(k, int(round(0.005 * k)), replace=False)
    x[:, idx] *= np.float32(30.0)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.015)
    return {"X": to_bf16(x), "W": to_bf16(w)}


LINEAR_SR_SEED = 0x5EED0004
LINEAR_RHT_SEED = 0x4AD40004


def linear_train(seed: int = 3, m: int = 8192, k: int = 4096, n: int = 4096):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    dy = (rng.standard_t(3.0, size=(m, n)) * 1e-3).astype(np.float32)
    return {"X": to_bf16(x), "W": to_bf16(w), "dY": to_bf16(dy),
            "sr_seed": LINEAR_SR_SEED, "rht_seed": LINEAR_RHT_SEED}


def attn_scores(seed: int = 4, b: int = 4, h: int = 32, s: int = 4096, d: int = 128):
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("Q", "K"):
        t = rng.standard_normal((b, h, s, d), dtype=np.float32)
        rms = np.exp(rng.uniform(np.log(0.5), np.log(4.0), size=(b, h, 1, 1))).astype(np.float32)
        t *= rms
        out[name] = to_bf16(t)
    out["alpha"] = float(np.float32(1.0 / np.sqrt(float(d))))  # 1/sqrt(128) -> 0x3DB504F3
    return out


ATTN_BWD_SR_SEED = 0x5EED0006


def attn_bwd(seed: int = 5, b: int = 4, h: int = 32, s: int = 4096, d: int = 128, heads: int | None = None):
    """The attention backward through dS ("Full-Stack FP4 ...", section 2.4):
    per (batch, head) slice i, drawn from its own stream default_rng([seed,
    i]): Q and K N(0, 1) times a per-slice RMS log-uniform in [0.5, 4] (as in
    attn_scores), and dS, the gradient of the scores, N(0, 1) times 1e-4 times
    a per-slice factor log-uniform in [0.25, 4].  `heads` keeps the first
    slices only (the same values as in the full draw)."""
    bh = b * h if heads is None else heads
    q = torch.empty((bh, s, d), dtype=torch.bfloat16)
    k = torch.empty((bh, s, d), dtype=torch.bfloat16)
    ds = torch.empty((bh, s, s), dtype=torch.bfloat16)
    def draw(i):
        rng = np.random.default_rng([seed, i])
        for t in (q, k):
            x = rng.standard_normal((s, d), dtype=np.float32)
            x *= np.float32(np.exp(rng.uniform(np.log(0.5), np.log(4.0))))
            t[i] = to_bf16(x)
        scale = np.float32(1e-4 * np.exp(rng.uniform(np.log(0.25), np.log(4.0))))
        ds[i] = to_bf16(rng.standard_normal((s, s), dtype=np.float32) * scale)

    # slices are independent streams, so they can be drawn side by side
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        list(ex.map(draw, range(bh)))
    return {"Q": q, "K": k, "dS": ds, "alpha": float(np.float32(1.0 / np.sqrt(float(d)))),
            "sr_seed": ATTN_BWD_SR_SEED}


ADAMW_RHT_SEED = 0x4AD40007
ADAMW_SR_SEED = 0x5EED0007


def adamw_state(seed: int = 7, rows: int = 20480, cols: int = 5120):
    """AdamW moments of one weight matrix (the 12B MLP up-projection's shape),
    for the NVFP4 state codec ("Full-Stack FP4 ...", section 2.2): per row a
    gradient scale g_r log-uniform in [1e-5, 1e-2]; m = g_r * Student-t(3)
    (heavy tailed), v = (g_r * Student-t(3))^2 + (1e-3 g_r)^2 (a second,
    independent draw, so v >= 0 and never exactly zero).  Row r comes from
    default_rng([seed, r // 1024]) in chunks of 1024 rows."""
    m = np.empty((rows, cols), np.float32)
    v = np.empty((rows, cols), np.float32)

    def draw(c):
        r0, r1 = 1024 * c, min(rows, 1024 * (c + 1))
        rng = np.random.default_rng([seed, c])
        g = np.exp(rng.uniform(np.log(1e-5), np.log(1e-2), size=(r1 - r0, 1)))
        m[r0:r1] = (rng.standard_t(3.0, size=(r1 - r0, cols)) * g).astype(np.float32)
        t = rng.standard_t(3.0, size=(r1 - r0, cols)) * g
        v[r0:r1] = (t * t + (1e-3 * g) ** 2).astype(np.float32)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        list(ex.map(draw, range((rows + 1023) // 1024)))
    return {"m": torch.from_numpy(m), "v": torch.from_numpy(v), "rht_seed": ADAMW_RHT_SEED,
            "sr_seed": ADAMW_SR_SEED}


NS_COEFFS = [(1.875, -1.25, 0.375)] * 5


def ns_3b(seed: int = 8, m: int = 3072, n: int = 8192):
    """A weight gradient for Newton-Schulz orthogonalization in NVFP4
    ("Full-Stack FP4 ...", section 2.3): the [3072][8192] MLP weight of the
    3B model, G = 1e-3 N(0, 1) times a per-row scale log-uniform in [0.5, 2],
    with 0.1% of entries times 20 as outliers, in BF16; five steps of the
    textbook quintic (a, b, c) = (15/8, -10/8, 3/8), clipping X at p99."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((m, n), dtype=np.float32) * np.float32(1e-3)
    g *= np.exp(rng.uniform(np.log(0.5), np.log(2.0), size=(m, 1))).astype(np.float32)
    idx = rng.choice(m * n, int(round(0.001 * m * n)), replace=False)
    g.reshape(-1)[idx] *= np.float32(20.0)
    return {"G": to_bf16(g), "coeffs": NS_COEFFS, "clip_quantile": 0.99, "clip_mask": 1}


def lora_3b(seed: int = 10, m: int = 8192, k: int = 3072, n: int = 3072, r: int = 64):
    """The fprop_3b layer as W = W_res + beta L2 L1 ("Full-Stack FP4 ...",
    section 2.1): X as in fprop_3b (1% of columns x20), W_res std 0.02, L1
    [r][K] N(0, 1/K), L2 [N][r] N(0, 0.05^2), beta 0.5, rank 64, all BF16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    idx = rng.choice(k, int(round(0.01 * k)), replace=False)
    x[:, idx] *= np.float32(20.0)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    l1 = rng.standard_normal((r, k), dtype=np.float32) * np.float32(1.0 / np.sqrt(k))
    l2 = rng.standard_normal((n, r), dtype=np.float32) * np.float32(0.05)
    return {"X": to_bf16(x), "W_res": to_bf16(w), "L1": to_bf16(l1), "L2": to_bf16(l2), "beta": 0.5}


WORKLOADS = {
    "tiny": tiny,
    "fprop_3b": fprop_3b,
    "mlp_up_12b": mlp_up_12b,
    "linear_train": linear_train,
    "attn_scores": attn_scores,
    "attn_bwd": attn_bwd,
    "adamw_state": adamw_state,
    "ns_3b": ns_3b,
    "lora_3b": lora_3b,
}
