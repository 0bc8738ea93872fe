"""Pins for the oracle's LoRA-style forward (L1, L2; "Full-Stack FP4 ...",
section 2.1), no GPU: the BF16 decode against torch's bfloat16 cast, and the
composition y = main + beta T L2^T against its special cases (L2 = 0 gives
the plain NVFP4 product; a zero residual gives beta T L2^T; a unit row of X
picks a column of L1)."""
import numpy as np
import torch

from oracle import oracle as O


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_values_match_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    v = O.bf16_values(bits)
    same = (v == t) | (np.isnan(v) & np.isnan(t))
    assert same.all()


def test_lora_reference_special_cases():
    rng = np.random.default_rng(1)
    M, N, K, r = 32, 48, 64, 16
    x = _bf16_bits(rng.standard_normal((M, K)))
    l1 = _bf16_bits(rng.standard_normal((r, K)))
    l2 = _bf16_bits(rng.standard_normal((N, r)))
    qx = O.quantize(x, O.BF16)
    qw = O.quantize(rng.standard_normal((N, K)).astype(np.float32), O.F32)
    t, ts = O.lora_down_ref(x, l1)
    assert (ts >= np.abs(t)).all()
    t_bits = O.bf16_rne_bits(t).astype(np.uint16)
    main, smain = O.gemm_ref(qx, qw)
    y, s = O.lora_forward_ref(qx, qw, t_bits, np.zeros_like(l2), 0.5)
    np.testing.assert_array_equal(y, main)
    np.testing.assert_array_equal(s, smain)
    zw = O.quantize(np.zeros((N, K), np.float32), O.F32)
    y, _ = O.lora_forward_ref(qx, zw, t_bits, l2, -2.0)
    np.testing.assert_array_equal(y, -2.0 * (O.bf16_values(t_bits) @ O.bf16_values(l2).T))
    e = np.zeros((1, K), np.float32)
    e[0, 5] = 1.0
    t1, _ = O.lora_down_ref(_bf16_bits(e), l1)
    np.testing.assert_array_equal(t1[0], O.bf16_values(l1)[:, 5])
    yr, _ = O.lora_forward_ref(qx, qw, t_bits, l2, 0.5, rows=[3, 9])
    yf, _ = O.lora_forward_ref(qx, qw, t_bits, l2, 0.5)
    np.testing.assert_array_equal(yr, yf[[3, 9]])
