"""GPU parity of the quantize kernels with the CPU oracle: codes, block
scales and tensor scale bit-exact, over both layouts, both input dtypes,
both roundings, with and without the Hadamard transform, on ragged shapes,
strided and batched inputs and adversarial values."""
import numpy as np
import pytest
import torch

from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

from .parity import assert_quant_equal, gpu_quant, oracle_quant, to_oracle_view

pytestmark = pytest.mark.gpu


def _input(shape, seed, dtype, kind="normal"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if kind == "wide":  # per-row magnitudes over 2^-40 .. 2^20: subnormal / zero block scales
        x *= (2.0 ** rng.integers(-40, 20, shape[:-1] + (1,))).astype(np.float32)
    elif kind == "ties":  # values on E2M1 midpoints relative to a power-of-two scale
        grid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, -0.0], np.float32)
        x = rng.choice(grid, shape).astype(np.float32) * rng.choice([-1, 1], shape).astype(np.float32)
    elif kind == "heavy":
        x = (rng.standard_t(2.0, shape) * 1e-3).astype(np.float32)
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


ROW_SHAPES = [(1, 16), (3, 48), (37, 160), (129, 1024), (1000, 48), (64, 4096)]
COL_SHAPES = [(16, 1), (32, 7), (48, 37), (160, 1000), (256, 130), (4096, 24)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", [O.RNE, O.SR])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("axis", [O.ALONG_COLS, O.ALONG_ROWS])
def test_quantize_shapes(dtype, rounding, rht, axis):
    shapes = ROW_SHAPES if axis == O.ALONG_COLS else COL_SHAPES
    for i, shape in enumerate(shapes):
        x = _input(shape, 1000 + i, dtype)
        kw = dict(axis=axis, rounding=rounding, sr_seed=0x5EED0004 + i, sr_stream=i, rht=rht,
                  rht_seed=0x4AD40004)
        got = to_oracle_view(gpu_quant(x, **kw))
        assert_quant_equal(got, oracle_quant(x, **kw), f"shape {shape}")


@pytest.mark.parametrize("kind", ["wide", "ties", "heavy"])
@pytest.mark.parametrize("axis", [O.ALONG_COLS, O.ALONG_ROWS])
@pytest.mark.parametrize("rounding", [O.RNE, O.SR])
def test_quantize_adversarial(kind, axis, rounding):
    x = _input((96, 256), 7, "bf16", kind)
    x[5, :32] = 0.0
    x[7, 16:48] = -0.0
    kw = dict(axis=axis, rounding=rounding, sr_seed=123, sr_stream=4, rht=False)
    assert_quant_equal(to_oracle_view(gpu_quant(x, **kw)), oracle_quant(x, **kw), kind)


def test_quantize_zero_and_empty():
    x = torch.zeros(64, 64, dtype=torch.bfloat16)
    x[3, 5] = -0.0
    for axis in (O.ALONG_COLS, O.ALONG_ROWS):
        got = to_oracle_view(gpu_quant(x, axis=axis))
        assert_quant_equal(got, oracle_quant(x, axis=axis), "zeros")
        assert got.tensor_scale == 0
    q = gpu_quant(torch.zeros(0, 32, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert q.tensor_scale.item() == 0.0 and q.codes.numel() == 0


def test_quantize_strided_and_batched():
    base = _input((3, 48, 96), 21, "bf16")          # [batch][rows][cols]
    big = torch.zeros(3, 56, 128, dtype=torch.bfloat16)
    big[:, :48, :96] = base
    view = big[:, :48, :96]                          # ld = 128, batch stride = 56*128
    for axis in (O.ALONG_COLS, O.ALONG_ROWS):
        kw = dict(axis=axis, rounding=O.SR, sr_seed=9, sr_stream=1, rht=axis == O.ALONG_ROWS,
                  rht_seed=77)
        got = to_oracle_view(gpu_quant(view, **kw))
        x3 = base.contiguous()
        want = oracle_quant(x3, **kw)
        assert_quant_equal(got, want, f"strided axis {axis}")


def test_quantize_deterministic_across_calls():
    x = _input((512, 2048), 5, "bf16")
    kw = dict(rounding=O.SR, sr_seed=1, sr_stream=2, rht=True, rht_seed=3)
    for axis in (O.ALONG_COLS, O.ALONG_ROWS):
        a = to_oracle_view(gpu_quant(x, axis=axis, **kw))
        b = to_oracle_view(gpu_quant(x, axis=axis, **kw))
        assert_quant_equal(a, b, "repeat")


def test_workspace_reuse_across_calls():
    """The workspace control words are restored to zero by every call, so one
    workspace serves a sequence of calls with different maxima."""
    import bit_block_scaled_nvfp4_amd as nv
    ws = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), "cuda:0")
    for i, scale in enumerate([100.0, 1.0, 1e-3, 50.0]):
        x = (_input((64, 128), 30 + i, "f32") * scale).to(torch.bfloat16)
        q = nv.quantize(x.to("cuda:0"), workspace=ws)
        assert_quant_equal(to_oracle_view(q), oracle_quant(x), f"call {i}")
    torch.cuda.synchronize()
    assert int(ws[:16].sum().item()) == 0


def test_single_pass_and_two_pass_share_a_workspace():
    """Alternate tensors that fit the single-pass kernel with ones that take
    the two-pass path (more than 37.7M BF16 elements) and with transposing
    calls, all on one workspace: every result stays bit-exact, and neither
    the two-pass words nor the barrier-timeout word are left set."""
    import bit_block_scaled_nvfp4_amd as nv
    ws = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), "cuda:0")
    big = _input((4864, 8192), 40, "bf16")  # 39.8M elements: over the single-pass capacity
    small = [(_input((256, 512), 41 + i, "f32") * 10.0 ** (i - 2)).to(torch.bfloat16) for i in range(4)]
    seq = [small[0], big, small[1], small[2], big, small[3]]
    for i, x in enumerate(seq):
        kw = dict(rounding=O.SR if i % 2 else O.RNE, sr_seed=5, sr_stream=i)
        q = nv.quantize(x.to("cuda:0"), workspace=ws, **kw)
        assert_quant_equal(to_oracle_view(q), oracle_quant(x, **kw), f"call {i}")
        qt = nv.quantize(x.to("cuda:0"), axis=O.ALONG_ROWS, workspace=ws)
        if x is not big:
            assert_quant_equal(to_oracle_view(qt), oracle_quant(x, axis=O.ALONG_ROWS), f"col call {i}")
    torch.cuda.synchronize()
    assert int(ws[:16].sum().item()) == 0
    # the eight two-pass partial maxima (64-byte slots after the 128-byte
    # header, 10 counter lines and 16 single-pass slot lines) are cleared too
    part0 = 128 + 10 * 128 + 16 * 128
    assert int(ws[part0:part0 + 8 * 64].sum().item()) == 0


@pytest.mark.parametrize("rows", [8192, 16384])
def test_transposing_single_pass_and_two_pass(rows):
    """Transposing BF16 quantize with RHT + SR: 8192 x 4096 fills the
    single-pass kernel's grid exactly (256 tiles of 1024 x 128); 16384 x 4096
    needs 512 tiles and takes the two-pass kernels.  Both bit-exact."""
    x = (_input((rows, 4096), 50 + rows // 8192, "f32") * 0.01).to(torch.bfloat16)
    kw = dict(axis=O.ALONG_ROWS, rounding=O.SR, sr_seed=0x5EED0003, sr_stream=3, rht=True, rht_seed=0x4AD40004)
    assert_quant_equal(to_oracle_view(gpu_quant(x, **kw)), oracle_quant(x, **kw), f"{rows}x4096 transposed")


@pytest.mark.parametrize("name", ["fprop_3b"])
def test_quantize_fprop_full_size(name):
    t = W.fprop_3b()
    for key in ("X", "W"):
        got = to_oracle_view(gpu_quant(t[key]))
        assert_quant_equal(got, oracle_quant(t[key]), key)


def test_barrier_counters_start_from_zero_whatever_the_grid():
    """Single-pass calls with different grid sizes on one workspace: a
    transposing call of 8 workgroups, a full-size row call (one workgroup
    per CU, every one holding data), a transposing call of 32 workgroups, a
    row call again.  Each call's barrier counters start from zero, so every
    result is bit-exact, and the arrival and finish counters are back at
    zero afterwards."""
    import bit_block_scaled_nvfp4_amd as nv
    ws = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), "cuda:0")
    full = W.fprop_3b()["X"]                           # 8192 x 3072: six segments per wavefront
    small = _input((512, 1024), 60, "bf16")            # transposed: 8 tiles of 512 x 128
    medium = (_input((2048, 2048), 61, "f32") * 3.0).to(torch.bfloat16)  # transposed: 64 tiles
    seq = [(small, O.ALONG_ROWS), (full, O.ALONG_COLS), (medium, O.ALONG_ROWS), (full, O.ALONG_COLS),
           (small, O.ALONG_COLS)]
    for i, (x, axis) in enumerate(seq):
        kw = dict(axis=axis, rounding=O.SR if i % 2 else O.RNE, sr_seed=17, sr_stream=i)
        q = nv.quantize(x.to("cuda:0"), workspace=ws, **kw)
        assert_quant_equal(to_oracle_view(q), oracle_quant(x, **kw), f"call {i} {tuple(x.shape)} axis {axis}")
    torch.cuda.synchronize()
    w = ws.cpu()
    counters = w[128:128 + 9 * 128].view(-1, 128)      # arrive[0..7] and top: value and finish words
    assert int(counters[:, :12].sum()) == 0
    assert int(w[8:12].view(torch.int32)[0]) == 0       # no time-out
    assert nv.quantize_workspace_check(ws) == nv.OK


def _force_timeout(ws: torch.Tensor, base: int) -> None:
    """Make the single-pass barrier of the control block at byte `base` give
    up at once: poll limit 8, and slot 0's arrival counter preset far beyond
    any grid's slot size, so slot 0 never completes and the release is never
    published.  Every workgroup still runs to its end."""
    ws[base:base + 4].view(torch.int32)[0] = 8
    ws[base + 128:base + 136].view(torch.int64)[0] = 1 << 40


@pytest.mark.parametrize("path", ["row", "col", "group"])
def test_barrier_timeout_poisons_the_tensor_scale(path):
    """A single-pass call whose barrier wait expires (forced from the host
    with a tiny poll limit) returns, finishes every kernel, sets the time-out
    word and publishes a NaN tensor scale, so the GEMM output is NaN; the
    word stays set for later calls on that workspace until it is zeroed."""
    import math
    import bit_block_scaled_nvfp4_amd as nv
    x = _input((512, 1024), 70, "bf16").to("cuda:0")
    if path == "group":
        ws = nv.new_workspace(nv.nvfp4_quantize_group_workspace_size(), "cuda:0")
        _force_timeout(ws, 4096)
        run = lambda: nv.quantize_group([x, x[:256]], workspace=ws)[0]
        word = 4096 + 8
    else:
        ws = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), "cuda:0")
        _force_timeout(ws, 0)
        axis = O.ALONG_ROWS if path == "col" else O.ALONG_COLS
        run = lambda: nv.quantize(x, axis=axis, workspace=ws)
        word = 8
    q = run()
    torch.cuda.synchronize()
    assert math.isnan(q.tensor_scale.item())
    assert int(ws[word:word + 4].view(torch.int32)[0].item()) == 1
    assert nv.quantize_workspace_check(ws) == nv.ETIMEOUT
    y = nv.gemm(q, q, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isnan(y).all())
    q2 = run()  # sticky: still poisoned
    torch.cuda.synchronize()
    assert math.isnan(q2.tensor_scale.item())
    ws.zero_()  # zeroed, the workspace is good again
    q3 = run()
    torch.cuda.synchronize()
    assert not math.isnan(q3.tensor_scale.item())
    assert nv.quantize_workspace_check(ws) == nv.OK
