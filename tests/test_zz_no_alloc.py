"""nvfp4_quantize_noalloc (no workspace argument; the library's static
per-GPU control block) against nvfp4_quantize with a workspace, through the
C ABI: bit-identical codes, scales and tensor scales on two calls in a row,
the second smaller, over the single-pass row, transposing and two-pass
paths, with RNE and with the transform and stochastic rounding."""
import ctypes

import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _x(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16).to(DEV)


def _call(fn_name, x, axis, opts, out, ws=None):
    b, r, c = (1, *x.shape) if x.dim() == 2 else x.shape
    ld = x.stride(-2)
    args = [x.data_ptr(), nv.BF16, b, r, c, ld, r * ld, axis, ctypes.byref(opts), ctypes.byref(out.c_struct())]
    stream = torch.cuda.current_stream().cuda_stream
    if ws is None:
        return getattr(nv.lib(), fn_name)(*args, stream)
    return getattr(nv.lib(), fn_name)(*args, ws.data_ptr(), ws.numel(), stream)


def _views(x, axis):
    r, c = x.shape[-2:]
    return (r, c) if axis == nv.ALONG_COLS else (c, r)


CASES = [  # (first shape, second, smaller, shape)
    ((1024, 4096), (96, 512)),          # single-pass row kernel, then a small single-pass call
    ((8192, 3072), (512, 1024)),        # one workgroup per CU holding data, then 8 workgroups
    ((4864, 8192), (1024, 2048)),       # two-pass (over the single-pass capacity), then single-pass
]


@pytest.mark.parametrize("first,second", CASES)
@pytest.mark.parametrize("axis", [nv.ALONG_COLS, nv.ALONG_ROWS])
@pytest.mark.parametrize("mode", ["rne", "rht_sr"])
def test_noalloc_matches_workspace_entry_point(first, second, axis, mode):
    if mode == "rne":
        opts = nv.QuantOptsC(nv.RNE, 0, 0, 0, 0, 0)
    else:
        opts = nv.QuantOptsC(nv.SR, 1, 0x5EED0005, 0x4AD40005, 7, 0)
    for i, shape in enumerate((first, second)):
        x = _x(shape, 100 + i, scale=10.0 ** (1 - 2 * i))
        qr, qc = _views(x, axis)
        want = nv.QTensor.empty(1, qr, qc, DEV)
        got = nv.QTensor.empty(1, qr, qc, DEV)
        ws = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), DEV)
        assert _call("nvfp4_quantize", x, axis, opts, want, ws) == nv.OK
        assert _call("nvfp4_quantize_noalloc", x, axis, opts, got) == nv.OK
        torch.cuda.synchronize()
        assert torch.equal(got.codes, want.codes), f"call {i} {shape}: codes"
        assert torch.equal(got.scales, want.scales), f"call {i} {shape}: scales"
        assert torch.equal(got.tensor_scale.view(torch.int32), want.tensor_scale.view(torch.int32)), \
            f"call {i} {shape}: tensor scale"


def test_noalloc_argument_errors_before_any_launch():
    x = _x((64, 64), 1)
    out = nv.QTensor.empty(1, 64, 48, DEV)  # wrong view shape
    assert _call("nvfp4_quantize_noalloc", x, nv.ALONG_COLS, nv.QuantOptsC(0, 0, 0, 0, 0, 0), out) == nv.EINVAL
    q = nv.QTensorC()
    assert nv.nvfp4_quantize_noalloc(x.data_ptr(), 7, 1, 64, 64, 64, 4096, 0, None, q, None) == nv.EINVAL
