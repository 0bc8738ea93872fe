"""End-to-end parity on the five workloads at their full sizes, in the launch
configuration the benchmark uses.  Quantized views are compared bit-exact in
full (all six views of the linear training step included); GEMM outputs on
every element for the 256x256 case and, elsewhere, on at least 1024 seeded
rows drawn over each output's own row range (for the attention scores, 8
rows in every one of the 128 (batch, head) products).  The FP64 reference
runs in host threads over row chunks."""
import numpy as np
import pytest
import torch

from bit_block_scaled_nvfp4_amd import workloads as W

from .parity import assert_quant_equal, gemm_vs_oracle, gpu_quant, oracle_quant, to_oracle_view
from .test_linear_parity import compare_linear, sample_rows

pytestmark = pytest.mark.gpu

NROWS = 1024


def _report(name, stats):
    print(f"\nparity {name}: {stats}", flush=True)


def test_fprop_3b():
    t = W.fprop_3b()
    qx, qw = gpu_quant(t["X"]), gpu_quant(t["W"])
    assert_quant_equal(to_oracle_view(qx), oracle_quant(t["X"]), "X")
    assert_quant_equal(to_oracle_view(qw), oracle_quant(t["W"]), "W")
    rows = sample_rows(8192, NROWS, 1)
    s = gemm_vs_oracle(qx, qw, out_dtype=torch.bfloat16, rows=rows, what="fprop_3b")
    assert s["rows"] >= NROWS
    _report("fprop_3b Y", s)


def test_mlp_up_12b():
    t = W.mlp_up_12b()
    qx, qw = gpu_quant(t["X"]), gpu_quant(t["W"])
    assert_quant_equal(to_oracle_view(qx), oracle_quant(t["X"]), "X")
    assert_quant_equal(to_oracle_view(qw), oracle_quant(t["W"]), "W")
    rows = sample_rows(16384, NROWS, 2)
    s = gemm_vs_oracle(qx, qw, out_dtype=torch.bfloat16, rows=rows, what="mlp_up_12b")
    assert s["rows"] >= NROWS
    _report("mlp_up_12b Y", s)


def test_linear_train():
    t = W.linear_train()
    stats = compare_linear(t["X"], t["W"], t["dY"], t["sr_seed"], t["rht_seed"], nrows=NROWS, seed=3)
    for name, s in stats.items():
        assert s["rows"] >= NROWS
        _report(f"linear_train {name}", s)


def test_attn_scores():
    t = W.attn_scores()
    q = t["Q"].reshape(128, 4096, 128)
    k = t["K"].reshape(128, 4096, 128)
    qq, qk = gpu_quant(q), gpu_quant(k)
    assert_quant_equal(to_oracle_view(qq), oracle_quant(q), "Q")
    assert_quant_equal(to_oracle_view(qk), oracle_quant(k), "K")
    rng = np.random.default_rng(4)
    per_batch = {b: np.unique(np.concatenate([[0, 4095] if b in (0, 127) else [],
                                              rng.choice(4096, NROWS // 128, replace=False)])).astype(np.int64)
                 for b in range(128)}
    s = gemm_vs_oracle(qq, qk, out_dtype=torch.float32, alpha=t["alpha"], rows_per_batch=per_batch,
                       what="attn_scores")
    assert s["rows"] >= NROWS
    _report("attn_scores S", s)
