"""GPU parity of the grouped quantize (several tensors, one tensor scale
each, one launch) with the CPU oracle: every tensor of a group must come out
bit-exact as the oracle quantizes it alone.  Covers the single-launch path,
the per-tensor fallback (strided views, groups over the single-pass
capacity), empty members and workspace reuse across calls whose group sizes
change."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, oracle_quant, to_oracle_view

pytestmark = pytest.mark.gpu

GROUP_SHAPES = [(129, 1024), (37, 160), (1, 16), (64, 4096)]


def _input(shape, seed, dtype, scale=1.0):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def _check_group(xs, outs, kw, what):
    for i, (x, q) in enumerate(zip(xs, outs)):
        assert_quant_equal(to_oracle_view(q), oracle_quant(x, **kw), f"{what}: tensor {i} {tuple(x.shape)}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", [O.RNE, O.SR])
@pytest.mark.parametrize("rht", [False, True])
def test_group_matches_oracle(dtype, rounding, rht):
    # magnitudes differ by orders so that a shared tensor scale would show
    xs = [_input(s, 200 + i, dtype, 10.0 ** (2 - i)) for i, s in enumerate(GROUP_SHAPES)]
    kw = dict(rounding=rounding, sr_seed=0x5EED0011, sr_stream=3, rht=rht, rht_seed=0x4AD40011)
    for n in (1, 2, 4):
        outs = nv.quantize_group([x.to(DEV) for x in xs[:n]], **kw)
        _check_group(xs[:n], outs, kw, f"{n} tensors")


def test_group_with_empty_zero_and_batched_members():
    xs = [torch.zeros(0, 32, dtype=torch.bfloat16), _input((3, 40, 96), 210, "bf16"),
          torch.zeros(64, 64, dtype=torch.bfloat16), _input((5, 48), 211, "bf16")]
    outs = nv.quantize_group([x.to(DEV) for x in xs], rounding=O.SR, sr_seed=7, sr_stream=1)
    torch.cuda.synchronize()
    assert outs[0].tensor_scale.item() == 0.0 and outs[0].codes.numel() == 0
    kw = dict(rounding=O.SR, sr_seed=7, sr_stream=1)
    _check_group(xs[1:], outs[1:], kw, "mixed")
    assert outs[2].tensor_scale.item() == 0.0
    only_empty = nv.quantize_group([torch.zeros(0, 16, dtype=torch.bfloat16, device=DEV)])
    torch.cuda.synchronize()
    assert only_empty[0].tensor_scale.item() == 0.0


def test_group_strided_member_takes_the_per_tensor_path():
    base = _input((48, 96), 220, "bf16")
    big = torch.zeros(56, 128, dtype=torch.bfloat16)
    big[:48, :96] = base
    other = _input((64, 256), 221, "bf16", 1e-3)
    dev_big = big.to(DEV)
    kw = dict(rounding=O.SR, sr_seed=11, sr_stream=2, rht=True, rht_seed=5)
    outs = nv.quantize_group([dev_big[:48, :96], other.to(DEV)], **kw)
    _check_group([base, other], outs, kw, "strided")


def test_group_workspace_reuse_with_changing_group_sizes():
    """One workspace, calls of 2, 1, 2, 4, 3 and 1 tensors with maxima that
    change between calls: a job index whose maxima slots were left from an
    earlier, larger group must not leak into a later call."""
    ws = nv.new_workspace(nv.nvfp4_quantize_group_workspace_size(), DEV)
    sizes = [2, 1, 2, 4, 3, 1, 2]
    for c, n in enumerate(sizes):
        xs = [_input((96, 512), 300 + 10 * c + i, "bf16", 10.0 ** ((c + i) % 5 - 2)) for i in range(n)]
        outs = nv.quantize_group([x.to(DEV) for x in xs], workspace=ws)
        _check_group(xs, outs, {}, f"call {c}")
    torch.cuda.synchronize()
    # neither the per-tensor control words nor the group barrier's timeout word are left set
    assert int(ws[:16].sum().item()) == 0
    assert int(ws[4096 + 8:4096 + 12].sum().item()) == 0


def test_group_and_single_calls_agree_bit_for_bit():
    xs = [_input((512, 2048), 230, "bf16"), _input((256, 2048), 231, "bf16", 0.02)]
    kw = dict(rounding=O.SR, sr_seed=1, sr_stream=9)
    outs = nv.quantize_group([x.to(DEV) for x in xs], **kw)
    for x, q in zip(xs, outs):
        single = nv.quantize(x.to(DEV), **kw)
        a, b = to_oracle_view(q), to_oracle_view(single)
        assert_quant_equal(a, b, "group vs single")


def test_group_over_single_pass_capacity():
    """Two tensors that each fit one launch but not together (39.8M BF16
    elements): the group runs them one after the other, same results."""
    xs = [_input((2432, 8192), 240, "bf16"), _input((2432, 8192), 241, "bf16", 3.0)]
    outs = nv.quantize_group([x.to(DEV) for x in xs])
    _check_group(xs, outs, {}, "over capacity")


def test_group_fprop_full_size():
    """The activations and weights of the 3B-class fprop (8192x3072 and
    3072x3072 BF16, 34.6M elements) in the one launch the step uses."""
    t = W.fprop_3b()
    xs = [t["X"], t["W"]]
    outs = nv.quantize_group([x.to(DEV) for x in xs])
    _check_group(xs, outs, {}, "fprop")
