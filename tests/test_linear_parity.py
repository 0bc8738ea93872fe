"""GPU parity of the linear-layer driver (Fprop, Dgrad, Wgrad in one C-ABI
call) with the oracle composed step by step: the six quantized views with
the same seeds and stream tags, then three reference GEMMs."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from oracle import oracle as O

from .parity import DEV, check_gemm, oracle_quant

pytestmark = pytest.mark.gpu


def oracle_linear(x, w, dy, sr_seed, rht_seed, wgrad_sr_x=True):
    qx = oracle_quant(x)
    qw = oracle_quant(w)
    qdy = oracle_quant(dy, rounding=O.SR, sr_seed=sr_seed, sr_stream=1)
    qwt = oracle_quant(w, axis=O.ALONG_ROWS)
    qdyt = oracle_quant(dy, axis=O.ALONG_ROWS, rounding=O.SR, sr_seed=sr_seed, sr_stream=2,
                        rht=True, rht_seed=rht_seed)
    qxt = oracle_quant(x, axis=O.ALONG_ROWS, rounding=O.SR if wgrad_sr_x else O.RNE,
                       sr_seed=sr_seed, sr_stream=3, rht=True, rht_seed=rht_seed)
    return (qx, qw), (qdy, qwt), (qdyt, qxt)


def compare_linear(x, w, dy, sr_seed, rht_seed, rows=None, wgrad_sr_x=True, dw_dtype=torch.bfloat16):
    y, dx, dw = nv.linear_fwd_bwd(x.to(DEV), w.to(DEV), dy.to(DEV), sr_seed, rht_seed,
                                  wgrad_sr_x=wgrad_sr_x, dw_dtype=dw_dtype)
    torch.cuda.synchronize()
    pairs = oracle_linear(x, w, dy, sr_seed, rht_seed, wgrad_sr_x)
    for (qa, qb), out, name in zip(pairs, (y, dx, dw), ("Y", "dX", "dW")):
        sel = np.arange(qa.rows) if rows is None else np.unique(np.asarray(rows) % qa.rows)
        y_ref, sabs = O.gemm_ref(qa, qb, 1.0, 0, sel)
        got = out[torch.as_tensor(sel, device=out.device)].float().cpu().numpy()
        check_gemm(got, y_ref, sabs, out.dtype == torch.bfloat16, name)


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
