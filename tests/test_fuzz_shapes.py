"""Seeded random shapes and options through every entry point, against the
oracle: ragged sizes (rows and columns that are not multiples of any tile,
batches, strides), both dtypes, both roundings, the transform, every GEMM
output type.  Each case draws its own shapes from default_rng([case]); a
failure names the case and the shapes."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, check_gemm, oracle_quant, to_oracle_view

pytestmark = pytest.mark.gpu


def _tensor(rng, shape, dtype):
    scale = float(np.exp(rng.uniform(-6, 6)))
    x = (rng.standard_t(4, size=shape) * scale).astype(np.float32)
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("case", range(24))
def test_quantize_random(case):
    rng = np.random.default_rng([101, case])
    axis = int(rng.integers(0, 2))
    batch = int(rng.integers(1, 4))
    a, b = int(rng.integers(1, 400)), 16 * int(rng.integers(1, 40))
    rows, cols = (a, b) if axis == O.ALONG_COLS else (b, a)
    dtype = ["bf16", "f32"][int(rng.integers(0, 2))]
    rnd = int(rng.integers(0, 2))
    rht = bool(rng.integers(0, 2))
    x = _tensor(rng, (batch, rows, cols), dtype)
    seed, stream = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
    what = f"case {case}: {dtype} [{batch}][{rows}][{cols}] axis {axis} rnd {rnd} rht {rht}"
    got = nv.quantize(x.to(DEV), axis=axis, rounding=rnd, sr_seed=seed, sr_stream=stream, rht=rht, rht_seed=seed ^ 5)
    want = oracle_quant(x, axis=axis, rounding=rnd, sr_seed=seed, sr_stream=stream, rht=rht, rht_seed=seed ^ 5)
    assert_quant_equal(to_oracle_view(got), want, what)


@pytest.mark.parametrize("case", range(16))
def test_gemm_random(case):
    rng = np.random.default_rng([102, case])
    batch = int(rng.integers(1, 3))
    M, N, K = int(rng.integers(1, 700)), int(rng.integers(1, 700)), 16 * int(rng.integers(1, 50))
    a = nv.quantize(_tensor(rng, (batch, M, K), "bf16").to(DEV))
    b = nv.quantize(_tensor(rng, (batch, N, K), "f32").to(DEV))
    alpha = float(np.float32(rng.uniform(-2, 2)))
    out = [torch.float32, torch.bfloat16][int(rng.integers(0, 2))]
    y = nv.gemm(a, b, out_dtype=out, alpha=alpha)
    torch.cuda.synchronize()
    y3 = y if y.dim() == 3 else y.unsqueeze(0)
    qa, qb = to_oracle_view(a), to_oracle_view(b)
    for bi in range(batch):
        y_ref, sabs = O.gemm_ref(qa, qb, alpha, bi)
        check_gemm(y3[bi].float().cpu().numpy(), y_ref, sabs, out == torch.bfloat16,
                   f"case {case}: [{batch}] {M}x{N}x{K} alpha {alpha} {out}")


@pytest.mark.parametrize("case", range(8))
def test_dual_and_axpby_random(case):
    rng = np.random.default_rng([103, case])
    R, C = 16 * int(rng.integers(1, 30)), 16 * int(rng.integers(1, 30))
    dtype = ["bf16", "f32"][case % 2]
    x = _tensor(rng, (R, C), dtype)
    rr, cr = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    row, col = nv.quantize_dual(x.to(DEV), row_rounding=rr, col_rounding=cr, sr_seed=case, row_stream=1,
                                col_stream=2)
    assert_quant_equal(to_oracle_view(row), oracle_quant(x, rounding=rr, sr_seed=case, sr_stream=1), f"case {case} row")
    assert_quant_equal(to_oracle_view(col), oracle_quant(x, axis=O.ALONG_ROWS, rounding=cr, sr_seed=case,
                                                         sr_stream=2), f"case {case} col")
    c_in = torch.from_numpy(rng.standard_normal((R, R)).astype(np.float32))
    beta = float(np.float32(rng.uniform(-3, 3)))
    y = nv.gemm_axpby(row, row, c_in.to(DEV), beta, alpha=0.5)
    torch.cuda.synchronize()
    y_ref, sabs = O.gemm_axpby_ref(to_oracle_view(row), to_oracle_view(row), 0.5, c_in.numpy(), beta)
    check_gemm(y[0].cpu().numpy(), y_ref, sabs, False, f"case {case} axpby {R}x{R}x{C}")


@pytest.mark.parametrize("case", range(6))
def test_state_codec_and_lora_random(case):
    rng = np.random.default_rng([104, case])
    R, C = int(rng.integers(1, 300)), 16 * int(rng.integers(1, 40))
    m = _tensor(rng, (R, C), "f32")
    v = _tensor(rng, (R, C), "f32") ** 2
    st = nv.qadamw_encode(m.to(DEV), v.to(DEV), case + 1, case + 2, case)
    gm, gv = nv.qadamw_decode(st, case + 1)
    torch.cuda.synchronize()
    want = O.qadamw_encode(m.numpy(), v.numpy(), case + 1, case + 2, case)
    assert_quant_equal(to_oracle_view(st.m), want.m, f"case {case} m")
    assert_quant_equal(to_oracle_view(st.v), want.v, f"case {case} v")
    wm, wv = O.qadamw_decode(want, case + 1)
    assert (gm.cpu().numpy().view(np.uint32) == wm.view(np.uint32)).all(), f"case {case} decoded m"
    assert (gv.cpu().numpy().view(np.uint32) == wv.view(np.uint32)).all(), f"case {case} decoded v"
    # LoRA: random rank and sizes
    M, N, K, r = int(rng.integers(1, 300)), int(rng.integers(1, 300)), 16 * int(rng.integers(1, 20)), \
        16 * int(rng.integers(1, 9))
    x = _tensor(rng, (M, K), "bf16")
    w = nv.quantize(_tensor(rng, (N, K), "bf16").to(DEV))
    l1 = _tensor(rng, (r, K), "bf16")
    l2 = _tensor(rng, (N, r), "bf16")
    beta = float(np.float32(rng.uniform(0.1, 2)))
    ws = nv.new_workspace(nv.nvfp4_lora_workspace_size(M, K, r), DEV)
    y = nv.lora_forward(x.to(DEV), w, l1.to(DEV), l2.to(DEV), beta, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    xv, t = nv.lora_internals(ws, M, K, r)
    from bit_block_scaled_nvfp4_amd import workloads as W
    tb = W.bf16_bits(t.cpu())
    t_ref, t_abs = O.lora_down_ref(W.bf16_bits(x), W.bf16_bits(l1))
    check_gemm(O.bf16_values(tb), t_ref, t_abs, True, f"case {case} T {M}x{K} r{r}")
    y_ref, sabs = O.lora_forward_ref(to_oracle_view(xv), to_oracle_view(w), tb, W.bf16_bits(l2), beta)
    check_gemm(y.cpu().numpy(), y_ref, sabs, False, f"case {case} lora {M}x{N}x{K} r{r}")
