"""GPU parity of the linear-layer driver (Fprop, Dgrad, Wgrad in one C-ABI
call) with the oracle composed step by step: the six quantized views with
the same seeds and stream tags, then three reference GEMMs."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, compare_output, oracle_quant, to_oracle_view

pytestmark = pytest.mark.gpu


def oracle_linear(x, w, dy, sr_seed, rht_seed, wgrad_sr_x=True):
    """The six quantized views of the step, in nv.LINEAR_VIEWS order: X, W
    (Fprop, RNE), dY (SR, stream 1), W^T (Dgrad), dY^T and X^T (Wgrad, RHT,
    SR streams 2 and 3)."""
    return [oracle_quant(x),
            oracle_quant(w),
            oracle_quant(dy, rounding=O.SR, sr_seed=sr_seed, sr_stream=1),
            oracle_quant(w, axis=O.ALONG_ROWS),
            oracle_quant(dy, axis=O.ALONG_ROWS, rounding=O.SR, sr_seed=sr_seed, sr_stream=2,
                         rht=True, rht_seed=rht_seed),
            oracle_quant(x, axis=O.ALONG_ROWS, rounding=O.SR if wgrad_sr_x else O.RNE,
                         sr_seed=sr_seed, sr_stream=3, rht=True, rht_seed=rht_seed)]


GEMMS = ((0, 1, "Y"), (2, 3, "dX"), (4, 5, "dW"))


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """k seeded distinct rows of 0..n-1 (all when k >= n), always with the first and last."""
    if k >= n:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, k, replace=False)]))


def compare_linear(x, w, dy, sr_seed, rht_seed, nrows=None, wgrad_sr_x=True, dw_dtype=torch.bfloat16, seed=0):
    """Run the step through the C ABI; check the six quantized views it
    leaves in its workspace bit-exact, then `nrows` seeded rows (all rows
    when None) of each output, drawn over that output's own row range."""
    M, K = x.shape
    N = w.shape[0]
    ws = nv.new_workspace(nv.nvfp4_linear_workspace_size(M, N, K), DEV)
    y, dx, dw = nv.linear_fwd_bwd(x.to(DEV), w.to(DEV), dy.to(DEV), sr_seed, rht_seed,
                                  wgrad_sr_x=wgrad_sr_x, dw_dtype=dw_dtype, workspace=ws)
    torch.cuda.synchronize()
    views = oracle_linear(x, w, dy, sr_seed, rht_seed, wgrad_sr_x)
    for i, want in enumerate(views):
        assert_quant_equal(to_oracle_view(nv.linear_view(ws, M, N, K, i)), want, f"view {nv.LINEAR_VIEWS[i]}")
    stats = {}
    for (ia, ib, name), out in zip(GEMMS, (y, dx, dw)):
        rows = np.arange(out.shape[0]) if nrows is None else sample_rows(out.shape[0], nrows, seed + ia)
        stats[name] = compare_output(out.unsqueeze(0), views[ia], views[ib], 1.0, out.dtype == torch.bfloat16,
                                     name, rows=rows)
        assert stats[name]["rows"] == rows.size
    return stats


@pytest.mark.parametrize("M,N,K", [(16, 16, 16), (64, 48, 32), (160, 96, 80), (256, 512, 384)])
def test_linear_small(M, N, K):
    rng = np.random.default_rng(M + N + K)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    dy = torch.from_numpy((rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32)).to(torch.bfloat16)
    compare_linear(x, w, dy, 0x5EED0004, 0x4AD40004)


def test_linear_rne_x_and_fp32_dw():
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((128, 64)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((32, 64)).astype(np.float32)).to(torch.bfloat16)
    dy = torch.from_numpy(rng.standard_normal((128, 32)).astype(np.float32)).to(torch.bfloat16)
    compare_linear(x, w, dy, 11, 22, wgrad_sr_x=False, dw_dtype=torch.float32)
