"""GPU parity of the attention backward through dS in NVFP4 ("Full-Stack FP4
...", section 2.4: QK^T and dS in NVFP4, quantized views of Q and K reused
between forward and backward) with the oracle composed step by step:

* nvfp4_quantize_dual: both orientations from one read, each view
  bit-identical to the oracle's quantize along that axis with its own
  rounding and stream, one tensor scale;
* nvfp4_attention_ds_grads: dS quantized along the keys (SR, stream 4) and
  along the queries (SR, stream 5), dQ = alpha dS K and dK = alpha dS^T Q
  against the oracle's FP64 reference on the oracle's views.

At the full 128-head shape the oracle quantizes a prefix of the heads
(every view's first slices, whose stochastic-rounding counters and, with the
tensor maximum planted in the first slice, tensor scale are those of the
full tensor), and the GEMM outputs are checked on 8 rows of every slice."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, compare_output, oracle_quant, to_oracle_view

pytestmark = pytest.mark.gpu


def _bf16(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("shape", [(1, 16, 16), (3, 48, 80), (2, 160, 96), (1, 512, 1024), (2, 272, 384)])
@pytest.mark.parametrize("rows_rnd,cols_rnd", [(O.RNE, O.RNE), (O.SR, O.SR), (O.RNE, O.SR)])
def test_quantize_dual_matches_oracle_both_views(shape, rows_rnd, cols_rnd):
    x = _bf16(shape, sum(shape), 3.0)
    row, col = nv.quantize_dual(x.to(DEV), row_rounding=rows_rnd, col_rounding=cols_rnd, sr_seed=77,
                                row_stream=4, col_stream=5)
    want_r = oracle_quant(x, rounding=rows_rnd, sr_seed=77, sr_stream=4)
    want_c = oracle_quant(x, axis=O.ALONG_ROWS, rounding=cols_rnd, sr_seed=77, sr_stream=5)
    assert_quant_equal(to_oracle_view(row), want_r, f"row view {shape}")
    assert_quant_equal(to_oracle_view(col), want_c, f"transposed view {shape}")


def test_quantize_dual_fp32_strided_and_zero():
    base = _bf16((2, 48, 96), 3).float()
    big = torch.zeros(2, 56, 128)
    big[:, :48, :96] = base
    row, col = nv.quantize_dual(big.to(DEV)[:, :48, :96], row_rounding=O.SR, sr_seed=5, row_stream=1)
    assert_quant_equal(to_oracle_view(row), oracle_quant(base, rounding=O.SR, sr_seed=5, sr_stream=1), "fp32 row")
    assert_quant_equal(to_oracle_view(col), oracle_quant(base, axis=O.ALONG_ROWS), "fp32 transposed")
    z = torch.zeros(64, 32, dtype=torch.bfloat16)
    row, col = nv.quantize_dual(z.to(DEV))
    torch.cuda.synchronize()
    assert row.tensor_scale.item() == 0.0 and col.tensor_scale.item() == 0.0
    assert_quant_equal(to_oracle_view(col), oracle_quant(z, axis=O.ALONG_ROWS), "zeros")


def test_quantize_dual_refuses_the_transform():
    x = _bf16((32, 48), 1).to(DEV)
    with pytest.raises(nv.NVFP4Error) as e:
        outs = (nv.QTensor.empty(1, 32, 48, DEV), nv.QTensor.empty(1, 48, 32, DEV))
        args, keep, _ = nv._dual_args(x, O.RNE, O.RNE, 0, 0, 0, outs, None)
        keep[0].rht = 1
        nv._check(nv.lib().nvfp4_quantize_dual(*args), "dual")
    assert e.value.status == nv.EUNSUPPORTED


def _oracle_attention(q, k, ds, alpha, sr_seed, rnd=O.SR):
    q_seq = oracle_quant(q, axis=O.ALONG_ROWS)
    k_seq = oracle_quant(k, axis=O.ALONG_ROWS)
    ds_row = oracle_quant(ds, rounding=rnd, sr_seed=sr_seed, sr_stream=4)
    ds_col = oracle_quant(ds, axis=O.ALONG_ROWS, rounding=rnd, sr_seed=sr_seed, sr_stream=5)
    return q_seq, k_seq, ds_row, ds_col


@pytest.mark.parametrize("bh,sq,sk,d", [(1, 16, 16, 16), (2, 48, 80, 32), (3, 160, 96, 64), (2, 512, 384, 128)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_attention_ds_grads_small(bh, sq, sk, d, out_dtype):
    q = _bf16((bh, sq, d), 10 + d)
    k = _bf16((bh, sk, d), 11 + d, 2.0)
    ds = _bf16((bh, sq, sk), 12 + d, 1e-4)
    alpha = float(np.float32(1.0 / np.sqrt(d)))
    # forward: Q and K in both orientations from one read each; QK^T uses the head-dim views
    q_hd, q_seq = nv.quantize_dual(q.to(DEV))
    k_hd, k_seq = nv.quantize_dual(k.to(DEV))
    ws = nv.new_workspace(nv.nvfp4_attention_ds_workspace_size(bh, sq, sk), DEV)
    dq, dk = nv.attention_ds_grads(ds.to(DEV), q_seq, k_seq, alpha, 0x5EED0006, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    oq, ok_, ods_r, ods_c = _oracle_attention(q, k, ds, alpha, 0x5EED0006)
    assert_quant_equal(to_oracle_view(q_seq), oq, "Q^T view")
    assert_quant_equal(to_oracle_view(k_seq), ok_, "K^T view")
    assert_quant_equal(to_oracle_view(q_hd), oracle_quant(q), "Q head-dim view")
    assert_quant_equal(to_oracle_view(nv.attention_ds_view(ws, bh, sq, sk, 0)), ods_r, "dS along keys")
    assert_quant_equal(to_oracle_view(nv.attention_ds_view(ws, bh, sq, sk, 1)), ods_c, "dS along queries")
    bf16 = out_dtype == torch.bfloat16
    s1 = compare_output(dq, ods_r, ok_, alpha, bf16, "dQ")
    s2 = compare_output(dk, ods_c, oq, alpha, bf16, "dK")
    assert s1["n"] == bh * sq * d and s2["n"] == bh * sk * d


def test_attention_ds_grads_full_size():
    """128 (batch, head) slices of 4096 x 4096 scores, head_dim 128."""
    t = W.attn_bwd()
    q, k, ds, alpha, seed = t["Q"], t["K"], t["dS"], t["alpha"], t["sr_seed"]
    bh, sq, sk, d = 128, 4096, 4096, 128
    # the tensor maximum, planted in the first slice, so the prefix's tensor scale is the tensor's
    top = float(ds.float().abs().max())
    ds[0, 5, 7] = torch.tensor(-2.0 * top, dtype=torch.bfloat16)
    q_hd, q_seq = nv.quantize_dual(q.to(DEV))
    k_hd, k_seq = nv.quantize_dual(k.to(DEV))
    dds = ds.to(DEV)
    ws = nv.new_workspace(nv.nvfp4_attention_ds_workspace_size(bh, sq, sk), DEV)
    dq, dk = nv.attention_ds_grads(dds, q_seq, k_seq, alpha, seed, workspace=ws)
    torch.cuda.synchronize()
    del dds
    # Q and K views in full (the forward views too)
    for got, x, axis, what in ((q_hd, q, O.ALONG_COLS, "Q"), (q_seq, q, O.ALONG_ROWS, "Q^T"),
                               (k_hd, k, O.ALONG_COLS, "K"), (k_seq, k, O.ALONG_ROWS, "K^T")):
        assert_quant_equal(to_oracle_view(got), oracle_quant(x, axis=axis), what)
    # dS views: the first 4 slices
    pre = 4
    gr = to_oracle_view(nv.attention_ds_view(ws, bh, sq, sk, 0))
    gc = to_oracle_view(nv.attention_ds_view(ws, bh, sq, sk, 1))
    wr = oracle_quant(ds[:pre], rounding=O.SR, sr_seed=seed, sr_stream=4)
    wc = oracle_quant(ds[:pre], axis=O.ALONG_ROWS, rounding=O.SR, sr_seed=seed, sr_stream=5)
    for g, w, what in ((gr, wr, "dS along keys"), (gc, wc, "dS along queries")):
        g_pre = O.QTensor(g.codes[:pre], g.scales[:pre], g.tensor_scale, pre, g.rows, g.cols)
        assert_quant_equal(g_pre, w, f"{what}, first {pre} slices")
    # dQ and dK: 8 rows of every slice, reference from the checked views
    rng = np.random.default_rng(6)
    per = {b: np.sort(rng.choice(4096, 8, replace=False)) for b in range(bh)}
    s1 = compare_output(dq, gr, to_oracle_view(k_seq), alpha, True, "dQ", rows_per_batch=per)
    s2 = compare_output(dk, gc, to_oracle_view(q_seq), alpha, True, "dK", rows_per_batch=per)
    assert s1["rows"] == s2["rows"] == 8 * bh
    print(f"\nparity attn_bwd dQ: {s1}\nparity attn_bwd dK: {s2}", flush=True)
