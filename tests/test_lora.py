"""GPU parity of the LoRA-style forward ("Full-Stack FP4 ...", section 2.1:
W = W_res + beta L2 L1, the residual in NVFP4 and the subspace in BF16)
against the oracle:

* the NVFP4 view of X bit-exact;
* T = BF16(X L1^T) within the BF16 rule of the GEMM acceptance (the RNE of
  the FP64 value or a neighbour);
* Y within the FP32 accumulation tolerance of s X^ W^^T + beta T L2^T,
  computed from the GPU's T once T is checked."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, check_gemm, host_threads, oracle_quant, to_oracle_view

pytestmark = pytest.mark.gpu


def _bf16(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16)


def _check(x, w_view, l1, l2, beta, y, ws, r, rows=None, what=""):
    M, K = x.shape
    xv, t = nv.lora_internals(ws, M, K, r)
    assert_quant_equal(to_oracle_view(xv), oracle_quant(x), f"{what}: X view")
    sel = np.arange(M) if rows is None else np.asarray(rows)
    xb, l1b, l2b = W.bf16_bits(x), W.bf16_bits(l1), W.bf16_bits(l2)
    t_gpu = W.bf16_bits(t.cpu())
    t_ref, t_abs = O.lora_down_ref(xb, l1b, sel)
    st = check_gemm(O.bf16_values(t_gpu[sel]), t_ref, t_abs, True, f"{what}: T")
    qx, qw = to_oracle_view(xv), to_oracle_view(w_view)
    chunks = [c for c in np.array_split(sel, max(1, min(host_threads(), sel.size // 16))) if c.size]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(chunks)) as ex:
        refs = list(ex.map(lambda c: O.lora_forward_ref(qx, qw, t_gpu, l2b, beta, c), chunks))
    y_ref = np.concatenate([a for a, _ in refs])
    sabs = np.concatenate([b for _, b in refs])
    yy = y[torch.as_tensor(sel, device=y.device)].float().cpu().numpy()
    sy = check_gemm(yy, y_ref, sabs, y.dtype == torch.bfloat16, f"{what}: Y")
    return st, sy


@pytest.mark.parametrize("M,N,K,r", [(1, 1, 16, 16), (16, 16, 16, 16), (48, 80, 32, 32), (160, 272, 96, 48),
                                     (512, 384, 1024, 64), (300, 200, 256, 128), (33, 64, 128, 96),
                                     (1000, 520, 4096, 16)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_lora_forward_matches_oracle(M, N, K, r, out_dtype):
    x = _bf16((M, K), M + K, 2.0)
    w = _bf16((N, K), N + K, 0.05)
    l1 = _bf16((r, K), r + K, 1.0 / np.sqrt(K))
    l2 = _bf16((N, r), N + r, 0.1)
    wv = nv.quantize(w.to(DEV))
    ws = nv.new_workspace(nv.nvfp4_lora_workspace_size(M, K, r), DEV)
    y = nv.lora_forward(x.to(DEV), wv, l1.to(DEV), l2.to(DEV), -0.75, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    _check(x, wv, l1, l2, -0.75, y, ws, r, what=f"lora {M}x{N}x{K} r{r}")


def test_lora_forward_zero_input_and_strided_output():
    M, N, K, r = 64, 96, 128, 32
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    w = _bf16((N, K), 3)
    l1 = _bf16((r, K), 4)
    l2 = _bf16((N, r), 5)
    wv = nv.quantize(w.to(DEV))
    ws = nv.new_workspace(nv.nvfp4_lora_workspace_size(M, K, r), DEV)
    out = torch.full((M, 128), 7.0, device=DEV)
    nv.lora_forward(x.to(DEV), wv, l1.to(DEV), l2.to(DEV), 2.0, out=out[:, :N], workspace=ws)
    torch.cuda.synchronize()
    assert (out[:, :N] == 0).all() and (out[:, N:] == 7.0).all()
    # a nonzero X after a zero one reuses the workspace
    x = _bf16((M, K), 6)
    y = nv.lora_forward(x.to(DEV), wv, l1.to(DEV), l2.to(DEV), 2.0, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    _check(x, wv, l1, l2, 2.0, y, ws, r, what="reuse")


def test_lora_forward_full_size():
    """lora_3b: 8192 x 3072 x 3072, rank 64; X view in full, T and Y on 1024
    rows."""
    t = W.lora_3b()
    x, w, l1, l2, beta = t["X"], t["W_res"], t["L1"], t["L2"], t["beta"]
    M, K = x.shape
    r = l1.shape[0]
    wv = nv.quantize(w.to(DEV))
    ws = nv.new_workspace(nv.nvfp4_lora_workspace_size(M, K, r), DEV)
    y = nv.lora_forward(x.to(DEV), wv, l1.to(DEV), l2.to(DEV), beta, workspace=ws)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(11).choice(M, 1024, replace=False))
    st, sy = _check(x, wv, l1, l2, beta, y, ws, r, rows=rows, what="lora_3b")
    print(f"\nparity lora_3b: T {st}, Y {sy}", flush=True)
