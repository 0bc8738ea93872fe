"""Python binding of libnvfp4.so, the gfx950 NVFP4 quantize + block-scaled
GEMM library (C ABI in include/nvfp4.h).

This layer only marshals arguments: torch provides device memory and the
current HIP stream, every step of the computation runs in the library's
kernels.  There is no fallback: without the built library every call raises.

Low-level entry points carry the C names (``nvfp4_quantize``, ``nvfp4_gemm``,
``nvfp4_linear_fwd_bwd``, ...) and take raw pointers and sizes exactly as the
C ABI does; ``quantize``, ``gemm`` and ``linear_fwd_bwd`` wrap them for torch
tensors.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "nvfp4.h")

# enums of include/nvfp4.h
OK, EINVAL, ESHAPE, EALIGN, EUNSUPPORTED, EHIP, EWORKSPACE, ETIMEOUT = range(8)
F32, BF16 = 0, 1
RNE, SR = 0, 1
ALONG_COLS, ALONG_ROWS = 0, 1


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class QTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("batch", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class QuantOptsC(ctypes.Structure):
    _fields_ = [("rounding", ctypes.c_int32), ("rht", ctypes.c_int32),
                ("sr_seed", ctypes.c_uint64), ("rht_seed", ctypes.c_uint64),
                ("sr_stream", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class QuantJobC(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("batch", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld", ctypes.c_int64), ("batch_stride", ctypes.c_int64),
                ("out", QTensorC)]


class AttnCfgC(ctypes.Structure):
    _fields_ = [("sr_seed", ctypes.c_uint64), ("ds_rounding", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class QAdamWStateC(ctypes.Structure):
    _fields_ = [("m", QTensorC), ("v", QTensorC), ("v_means", ctypes.c_void_p)]


class NsCfgC(ctypes.Structure):
    _fields_ = [("clip_quantile", ctypes.c_double), ("clip_mask", ctypes.c_uint32), ("product", ctypes.c_uint32)]


class NsStateC(ctypes.Structure):
    _fields_ = [("x_prev", ctypes.c_void_p), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("clip", ctypes.c_void_p * 3), ("inv_norm", ctypes.c_void_p), ("view", QTensorC * 4)]


class LinearCfgC(ctypes.Structure):
    _fields_ = [("sr_seed", ctypes.c_uint64), ("rht_seed", ctypes.c_uint64),
                ("wgrad_sr_x", ctypes.c_int32), ("dw_dtype", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bit_block_scaled_nvfp4_amd.build`"
                " (this package has no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        L.nvfp4_status_string.argtypes = [i32]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_version.restype = i32
        L.nvfp4_quantize_workspace_size.restype = sz
        L.nvfp4_quantize.argtypes = [vp, i32, i64, i64, i64, i64, i64, i32,
                                     ctypes.POINTER(QuantOptsC), ctypes.POINTER(QTensorC), vp, sz, vp]
        L.nvfp4_quantize.restype = i32
        L.nvfp4_quantize_noalloc.argtypes = [vp, i32, i64, i64, i64, i64, i64, i32,
                                             ctypes.POINTER(QuantOptsC), ctypes.POINTER(QTensorC), vp]
        L.nvfp4_quantize_noalloc.restype = i32
        L.nvfp4_quantize_dual.argtypes = [vp, i32, i64, i64, i64, i64, i64, ctypes.POINTER(QuantOptsC),
                                          ctypes.POINTER(QTensorC), ctypes.POINTER(QuantOptsC),
                                          ctypes.POINTER(QTensorC), vp, sz, vp]
        L.nvfp4_quantize_dual.restype = i32
        L.nvfp4_attention_ds_workspace_size.argtypes = [i64, i64, i64]
        L.nvfp4_attention_ds_workspace_size.restype = sz
        L.nvfp4_attention_ds_grads.argtypes = [vp, i32, ctypes.POINTER(QTensorC), ctypes.POINTER(QTensorC), vp, vp,
                                               i32, i64, i64, i64, i64, ctypes.c_float, ctypes.POINTER(AttnCfgC),
                                               vp, sz, vp]
        L.nvfp4_attention_ds_grads.restype = i32
        L.nvfp4_quantize_group_workspace_size.restype = sz
        L.nvfp4_quantize_group.argtypes = [ctypes.POINTER(QuantJobC), i32, i32, ctypes.POINTER(QuantOptsC),
                                           vp, sz, vp]
        L.nvfp4_quantize_group.restype = i32
        L.nvfp4_gemm.argtypes = [ctypes.POINTER(QTensorC), ctypes.POINTER(QTensorC), vp, i32, i64, i64,
                                 ctypes.c_float, vp]
        L.nvfp4_gemm.restype = i32
        L.nvfp4_gemm_ex.argtypes = [ctypes.POINTER(QTensorC), ctypes.POINTER(QTensorC), vp, i32, i64, i64,
                                    ctypes.c_float, i32, i32, vp]
        L.nvfp4_gemm_ex.restype = i32
        L.nvfp4_quantize_workspace_check.argtypes = [vp, sz, vp]
        L.nvfp4_quantize_workspace_check.restype = i32
        L.nvfp4_linear_view.argtypes = [vp, sz, i64, i64, i64, i32, ctypes.POINTER(QTensorC)]
        L.nvfp4_linear_view.restype = i32
        L.nvfp4_linear_workspace_size.argtypes = [i64, i64, i64]
        L.nvfp4_linear_workspace_size.restype = sz
        L.nvfp4_linear_fwd_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                           ctypes.POINTER(LinearCfgC), vp, sz, vp]
        L.nvfp4_linear_fwd_bwd.restype = i32
        L.nvfp4_qadamw_workspace_size.restype = sz
        L.nvfp4_qadamw_encode.argtypes = [vp, vp, i64, i64, i64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.POINTER(QAdamWStateC), vp, sz, vp]
        L.nvfp4_qadamw_encode.restype = i32
        L.nvfp4_qadamw_decode.argtypes = [ctypes.POINTER(QAdamWStateC), ctypes.c_uint64, vp, vp, i64, vp]
        L.nvfp4_qadamw_decode.restype = i32
        L.nvfp4_gemm_axpby.argtypes = [ctypes.POINTER(QTensorC), ctypes.POINTER(QTensorC), vp, i32, i64, i64,
                                       ctypes.c_float, vp, i64, i64, ctypes.c_float, vp]
        L.nvfp4_gemm_axpby.restype = i32
        L.nvfp4_ns_workspace_size.argtypes = [i64, i64]
        L.nvfp4_ns_workspace_size.restype = sz
        L.nvfp4_ns_orthogonalize.argtypes = [vp, i32, i64, i64, i64, vp, i32, ctypes.POINTER(NsCfgC), vp, i64,
                                             vp, sz, vp]
        L.nvfp4_ns_orthogonalize.restype = i32
        L.nvfp4_ns_internals.argtypes = [vp, sz, i64, i64, ctypes.POINTER(NsStateC)]
        L.nvfp4_ns_internals.restype = i32
        L.nvfp4_lora_workspace_size.argtypes = [i64, i64, i64]
        L.nvfp4_lora_workspace_size.restype = sz
        L.nvfp4_lora_forward.argtypes = [vp, ctypes.POINTER(QTensorC), vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                         vp, i32, i64, vp, sz, vp]
        L.nvfp4_lora_forward.restype = i32
        L.nvfp4_lora_internals.argtypes = [vp, sz, i64, i64, i64, ctypes.POINTER(QTensorC),
                                           ctypes.POINTER(ctypes.c_void_p)]
        L.nvfp4_lora_internals.restype = i32
        _lib = L
    return _lib


# --- C-named entry points (raw pointers / sizes) ---------------------------

def nvfp4_status_string(status: int) -> str:
    return lib().nvfp4_status_string(int(status)).decode()


status_string = nvfp4_status_string


def nvfp4_version() -> int:
    return lib().nvfp4_version()


def nvfp4_quantize_workspace_size() -> int:
    return lib().nvfp4_quantize_workspace_size()


def nvfp4_quantize_group_workspace_size() -> int:
    return lib().nvfp4_quantize_group_workspace_size()


def nvfp4_qadamw_workspace_size() -> int:
    return int(lib().nvfp4_qadamw_workspace_size())


def nvfp4_ns_workspace_size(m: int, n: int) -> int:
    return int(lib().nvfp4_ns_workspace_size(m, n))


def nvfp4_linear_workspace_size(M: int, N: int, K: int) -> int:
    return lib().nvfp4_linear_workspace_size(M, N, K)


def nvfp4_quantize(x_ptr, x_dtype, batch, rows, cols, ld, batch_stride, axis, opts, out, workspace,
                   workspace_bytes, stream) -> int:
    return lib().nvfp4_quantize(x_ptr, x_dtype, batch, rows, cols, ld, batch_stride, axis,
                                ctypes.byref(opts) if opts is not None else None,
                                ctypes.byref(out) if out is not None else None,
                                workspace, workspace_bytes, stream)


def nvfp4_quantize_noalloc(x_ptr, x_dtype, batch, rows, cols, ld, batch_stride, axis, opts, out, stream) -> int:
    return lib().nvfp4_quantize_noalloc(x_ptr, x_dtype, batch, rows, cols, ld, batch_stride, axis,
                                        ctypes.byref(opts) if opts is not None else None,
                                        ctypes.byref(out) if out is not None else None, stream)


def nvfp4_quantize_dual(x_ptr, x_dtype, batch, rows, cols, ld, batch_stride, row_opts, row_out, col_opts, col_out,
                        workspace, workspace_bytes, stream) -> int:
    ref = lambda o: ctypes.byref(o) if o is not None else None
    return lib().nvfp4_quantize_dual(x_ptr, x_dtype, batch, rows, cols, ld, batch_stride, ref(row_opts), ref(row_out),
                                     ref(col_opts), ref(col_out), workspace, workspace_bytes, stream)


def nvfp4_attention_ds_workspace_size(bh: int, sq: int, sk: int) -> int:
    return lib().nvfp4_attention_ds_workspace_size(bh, sq, sk)


def nvfp4_attention_ds_grads(ds_ptr, ds_dtype, q_seq, k_seq, dq_ptr, dk_ptr, out_dtype, bh, sq, sk, d, alpha, cfg,
                             workspace, workspace_bytes, stream) -> int:
    ref = lambda o: ctypes.byref(o) if o is not None else None
    return lib().nvfp4_attention_ds_grads(ds_ptr, ds_dtype, ref(q_seq), ref(k_seq), dq_ptr, dk_ptr, out_dtype, bh, sq,
                                          sk, d, ctypes.c_float(alpha), ref(cfg), workspace, workspace_bytes, stream)


def nvfp4_quantize_group(jobs, njobs, x_dtype, opts, workspace, workspace_bytes, stream) -> int:
    return lib().nvfp4_quantize_group(jobs, njobs, x_dtype, ctypes.byref(opts) if opts is not None else None,
                                      workspace, workspace_bytes, stream)


def nvfp4_gemm(a, b, c_ptr, c_dtype, ldc, batch_stride_c, alpha, stream) -> int:
    return lib().nvfp4_gemm(ctypes.byref(a) if a is not None else None,
                            ctypes.byref(b) if b is not None else None,
                            c_ptr, c_dtype, ldc, batch_stride_c, ctypes.c_float(alpha), stream)


def nvfp4_gemm_ex(a, b, c_ptr, c_dtype, ldc, batch_stride_c, alpha, tile_m, tile_n, stream) -> int:
    return lib().nvfp4_gemm_ex(ctypes.byref(a) if a is not None else None,
                               ctypes.byref(b) if b is not None else None,
                               c_ptr, c_dtype, ldc, batch_stride_c, ctypes.c_float(alpha), tile_m, tile_n, stream)


def nvfp4_quantize_workspace_check(workspace, workspace_bytes, stream) -> int:
    return lib().nvfp4_quantize_workspace_check(workspace, workspace_bytes, stream)


def nvfp4_linear_view(workspace, workspace_bytes, M, N, K, which, out) -> int:
    return lib().nvfp4_linear_view(workspace, workspace_bytes, M, N, K, which,
                                   ctypes.byref(out) if out is not None else None)


def nvfp4_linear_fwd_bwd(x_ptr, w_ptr, dy_ptr, y_ptr, dx_ptr, dw_ptr, M, N, K, cfg, workspace,
                         workspace_bytes, stream) -> int:
    return lib().nvfp4_linear_fwd_bwd(x_ptr, w_ptr, dy_ptr, y_ptr, dx_ptr, dw_ptr, M, N, K,
                                      ctypes.byref(cfg) if cfg is not None else None,
                                      workspace, workspace_bytes, stream)


# --- torch wrappers ----------------------------------------------------------

def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, what: str) -> None:
    if status != OK:
        raise NVFP4Error(status, what)


@dataclass
class QTensor:
    """A quantized view on the GPU: codes [batch][rows][cols/2] (uint8),
    scales [batch][rows][cols/16] (uint8, E4M3FN), tensor_scale [1] (float32)."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    batch: int
    rows: int
    cols: int

    def c_struct(self) -> QTensorC:
        return QTensorC(self.codes.data_ptr(), self.scales.data_ptr(), self.tensor_scale.data_ptr(),
                        self.batch, self.rows, self.cols)

    @staticmethod
    def empty(batch: int, rows: int, cols: int, device) -> "QTensor":
        n = batch * rows * cols
        return QTensor(torch.empty(max(n // 2, 1), dtype=torch.uint8, device=device)[: n // 2]
                       .view(batch, rows, cols // 2),
                       torch.empty(max(n // 16, 1), dtype=torch.uint8, device=device)[: n // 16]
                       .view(batch, rows, cols // 16),
                       torch.empty(1, dtype=torch.float32, device=device), batch, rows, cols)


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled device workspace (the C ABI requires zeros before first use)."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def _quantize_args(x: torch.Tensor, axis: int, rounding: int, sr_seed: int, sr_stream: int, rht: bool,
                   rht_seed: int, out: QTensor | None, workspace: torch.Tensor | None):
    """Validated ctypes arguments of one nvfp4_quantize call (and its output)."""
    if x.dim() == 2:
        x3 = x.unsqueeze(0)
    elif x.dim() == 3:
        x3 = x
    else:
        raise ValueError("x must be 2-D or 3-D")
    if x3.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be bfloat16 or float32")
    if x3.size(2) > 1 and x3.stride(2) != 1:
        raise ValueError("the last dimension of x must be contiguous")
    b, r, c = x3.shape
    qr, qc = (r, c) if axis == ALONG_COLS else (c, r)
    if out is None:
        out = QTensor.empty(b, qr, qc, x.device)
    if workspace is None:
        workspace = new_workspace(nvfp4_quantize_workspace_size(), x.device)
    opts = QuantOptsC(rounding, int(bool(rht)), sr_seed, rht_seed, sr_stream, 0)
    q = out.c_struct()
    args = (x3.data_ptr(), BF16 if x3.dtype == torch.bfloat16 else F32, b, r, c,
            x3.stride(1) if r > 1 else c, x3.stride(0) if b > 1 else r * c, axis, ctypes.byref(opts),
            ctypes.byref(q), workspace.data_ptr(), workspace.numel(), _stream(x.device))
    return args, (opts, q, x3, workspace), out


def quantize(x: torch.Tensor, axis: int = ALONG_COLS, rounding: int = RNE, sr_seed: int = 0,
             sr_stream: int = 0, rht: bool = False, rht_seed: int = 0, out: QTensor | None = None,
             workspace: torch.Tensor | None = None) -> QTensor:
    """Quantize a 2-D [rows][cols] or 3-D [batch][rows][cols] CUDA tensor
    (bfloat16 or float32, last dimension contiguous)."""
    args, _keep, out = _quantize_args(x, axis, rounding, sr_seed, sr_stream, rht, rht_seed, out, workspace)
    _check(lib().nvfp4_quantize(*args), "nvfp4_quantize")
    return out


def quantize_noalloc(x: torch.Tensor, axis: int = ALONG_COLS, rounding: int = RNE, sr_seed: int = 0,
                     sr_stream: int = 0, rht: bool = False, rht_seed: int = 0,
                     out: QTensor | None = None) -> QTensor:
    """quantize() through nvfp4_quantize_noalloc: no workspace (the library's
    per-GPU static control block); `out` must be given to allocate nothing."""
    args, _keep, out = _quantize_args(x, axis, rounding, sr_seed, sr_stream, rht, rht_seed, out,
                                      torch.empty(0, dtype=torch.uint8, device=x.device))
    # nvfp4_quantize's arguments without the workspace pointer and size
    _check(lib().nvfp4_quantize_noalloc(*args[:10], args[12]), "nvfp4_quantize_noalloc")
    return out


def _dual_args(x: torch.Tensor, row_rounding: int, col_rounding: int, sr_seed: int, row_stream: int,
               col_stream: int, outs, workspace: torch.Tensor | None):
    x3 = x.unsqueeze(0) if x.dim() == 2 else x
    if x3.dim() != 3 or x3.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be a 2-D or 3-D bfloat16 or float32 tensor")
    if x3.size(2) > 1 and x3.stride(2) != 1:
        raise ValueError("the last dimension of x must be contiguous")
    b, r, c = x3.shape
    if outs is None:
        outs = (QTensor.empty(b, r, c, x.device), QTensor.empty(b, c, r, x.device))
    if workspace is None:
        workspace = new_workspace(nvfp4_quantize_workspace_size(), x.device)
    ro = QuantOptsC(row_rounding, 0, sr_seed, 0, row_stream, 0)
    co = QuantOptsC(col_rounding, 0, sr_seed, 0, col_stream, 0)
    rq, cq = outs[0].c_struct(), outs[1].c_struct()
    args = (x3.data_ptr(), BF16 if x3.dtype == torch.bfloat16 else F32, b, r, c, x3.stride(1) if r > 1 else c,
            x3.stride(0) if b > 1 else r * c, ctypes.byref(ro), ctypes.byref(rq), ctypes.byref(co), ctypes.byref(cq),
            workspace.data_ptr(), workspace.numel(), _stream(x.device))
    return args, (ro, co, rq, cq, x3, workspace), outs


def quantize_dual(x: torch.Tensor, row_rounding: int = RNE, col_rounding: int = RNE, sr_seed: int = 0,
                  row_stream: int = 0, col_stream: int = 0, outs=None, workspace: torch.Tensor | None = None):
    """Both orientations of x from one read: (view along the last dimension,
    transposed view along the rows), one tensor scale (nvfp4_quantize_dual)."""
    args, _keep, outs = _dual_args(x, row_rounding, col_rounding, sr_seed, row_stream, col_stream, outs, workspace)
    _check(lib().nvfp4_quantize_dual(*args), "nvfp4_quantize_dual")
    return outs


def bind_quantize_dual(x: torch.Tensor, outs, workspace: torch.Tensor, row_rounding: int = RNE,
                       col_rounding: int = RNE, sr_seed: int = 0, row_stream: int = 0, col_stream: int = 0):
    args, keep, outs = _dual_args(x, row_rounding, col_rounding, sr_seed, row_stream, col_stream, outs, workspace)
    return BoundCall(lib().nvfp4_quantize_dual, args, keep, "nvfp4_quantize_dual", outs)


def _attn_args(ds, q_seq: QTensor, k_seq: QTensor, dq, dk, alpha, sr_seed, ds_rounding, workspace):
    bh, sq, sk = ds.shape
    d = q_seq.rows
    if not ds.is_contiguous() or ds.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("ds must be a contiguous [bh][sq][sk] bfloat16 or float32 tensor")
    cfg = AttnCfgC(sr_seed, ds_rounding, 0)
    qs, ks = q_seq.c_struct(), k_seq.c_struct()
    args = (ds.data_ptr(), BF16 if ds.dtype == torch.bfloat16 else F32, ctypes.byref(qs), ctypes.byref(ks),
            dq.data_ptr(), dk.data_ptr(), BF16 if dq.dtype == torch.bfloat16 else F32, bh, sq, sk, d,
            ctypes.c_float(alpha), ctypes.byref(cfg), workspace.data_ptr(), workspace.numel(), _stream(ds.device))
    return args, (cfg, qs, ks, ds, dq, dk, workspace)


def attention_ds_grads(ds: torch.Tensor, q_seq: QTensor, k_seq: QTensor, alpha: float, sr_seed: int,
                       ds_rounding: int = SR, out_dtype: torch.dtype = torch.bfloat16,
                       workspace: torch.Tensor | None = None):
    """(dQ, dK) = (alpha dS K, alpha dS^T Q) with dS quantized in both
    orientations (nvfp4_attention_ds_grads); q_seq / k_seq are the
    sequence-major views [bh][d][s] of Q and K."""
    bh, sq, sk = ds.shape
    d = q_seq.rows
    dq = torch.empty(bh, sq, d, dtype=out_dtype, device=ds.device)
    dk = torch.empty(bh, sk, d, dtype=out_dtype, device=ds.device)
    if workspace is None:
        workspace = new_workspace(nvfp4_attention_ds_workspace_size(bh, sq, sk), ds.device)
    args, _keep = _attn_args(ds, q_seq, k_seq, dq, dk, alpha, sr_seed, ds_rounding, workspace)
    _check(lib().nvfp4_attention_ds_grads(*args), "nvfp4_attention_ds_grads")
    return dq, dk


def bind_attention_ds_grads(ds, q_seq: QTensor, k_seq: QTensor, dq, dk, workspace: torch.Tensor, alpha: float,
                            sr_seed: int, ds_rounding: int = SR) -> "BoundCall":
    args, keep = _attn_args(ds, q_seq, k_seq, dq, dk, alpha, sr_seed, ds_rounding, workspace)
    return BoundCall(lib().nvfp4_attention_ds_grads, args, keep, "nvfp4_attention_ds_grads", (dq, dk))


def attention_ds_view(workspace: torch.Tensor, bh: int, sq: int, sk: int, which: int) -> QTensor:
    """The quantized dS view nvfp4_attention_ds_grads left in `workspace`:
    0 = along the keys [bh][sq][sk], 1 = along the queries [bh][sk][sq]
    (the layout the header states: each view's codes, scales and tensor-scale
    slot, 256-byte aligned, in that order)."""
    n = bh * sq * sk

    def up(v):
        return (v + 255) // 256 * 256

    off = 0
    views = []
    for i in range(2):
        r, c = (sq, sk) if i == 0 else (sk, sq)
        codes = workspace[off:off + n // 2].view(bh, r, c // 2)
        off = up(off + n // 2)
        scales = workspace[off:off + n // 16].view(bh, r, c // 16)
        off = up(off + n // 16)
        ts = workspace[off:off + 4].view(torch.float32)
        off += 256
        views.append(QTensor(codes, scales, ts, bh, r, c))
    return views[which]


@dataclass
class QAdamWState:
    """AdamW moments in NVFP4: m (transformed, stochastic rounding), v (the
    transformed residual of sqrt(v) after its 16-element block means, RNE)
    and the BF16 block means [rows][cols/16] (uint16 bits)."""
    m: QTensor
    v: QTensor
    v_means: torch.Tensor

    @staticmethod
    def empty(rows: int, cols: int, device) -> "QAdamWState":
        n = rows * cols // 16
        return QAdamWState(QTensor.empty(1, rows, cols, device), QTensor.empty(1, rows, cols, device),
                           torch.empty(max(n, 1), dtype=torch.int16, device=device)[:n].view(rows, cols // 16))

    def c_struct(self) -> QAdamWStateC:
        return QAdamWStateC(self.m.c_struct(), self.v.c_struct(), self.v_means.data_ptr())


def _moment(t: torch.Tensor, what: str) -> torch.Tensor:
    if t.dim() != 2 or t.dtype != torch.float32:
        raise ValueError(f"{what} must be a 2-D float32 tensor")
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"the last dimension of {what} must be contiguous")
    return t


def _qadamw_encode_args(m, v, rht_seed, sr_seed, sr_stream, state, workspace):
    m, v = _moment(m, "m"), _moment(v, "v")
    if m.shape != v.shape or (m.size(0) > 1 and m.stride(0) != v.stride(0)):
        raise ValueError("m and v must have one shape and one row stride")
    rows, cols = m.shape
    if state is None:
        state = QAdamWState.empty(rows, cols, m.device)
    if workspace is None:
        workspace = new_workspace(nvfp4_qadamw_workspace_size(), m.device)
    st = state.c_struct()
    args = (m.data_ptr(), v.data_ptr(), rows, cols, m.stride(0) if rows > 1 else cols, rht_seed, sr_seed, sr_stream,
            ctypes.byref(st), workspace.data_ptr(), workspace.numel(), _stream(m.device))
    return args, (st, m, v, workspace), state


def qadamw_encode(m: torch.Tensor, v: torch.Tensor, rht_seed: int, sr_seed: int, sr_stream: int = 0,
                  state: QAdamWState | None = None, workspace: torch.Tensor | None = None) -> QAdamWState:
    """Encode FP32 moments m, v ([rows][cols], v >= 0) into NVFP4 state."""
    args, _keep, state = _qadamw_encode_args(m, v, rht_seed, sr_seed, sr_stream, state, workspace)
    _check(lib().nvfp4_qadamw_encode(*args), "nvfp4_qadamw_encode")
    return state


def _qadamw_decode_args(state: QAdamWState, rht_seed: int, m_out, v_out):
    rows, cols = state.m.rows, state.m.cols
    dev = state.m.codes.device
    m_out = torch.empty(rows, cols, dtype=torch.float32, device=dev) if m_out is None else _moment(m_out, "m")
    v_out = torch.empty(rows, cols, dtype=torch.float32, device=dev) if v_out is None else _moment(v_out, "v")
    if tuple(m_out.shape) != (rows, cols) or tuple(v_out.shape) != (rows, cols) or (
            rows > 1 and m_out.stride(0) != v_out.stride(0)):
        raise ValueError("outputs must be [rows][cols] with one row stride")
    st = state.c_struct()
    args = (ctypes.byref(st), rht_seed, m_out.data_ptr(), v_out.data_ptr(), m_out.stride(0) if rows > 1 else cols,
            _stream(dev))
    return args, (st, m_out, v_out), (m_out, v_out)


def qadamw_decode(state: QAdamWState, rht_seed: int, m_out: torch.Tensor | None = None,
                  v_out: torch.Tensor | None = None):
    """Reconstruct the FP32 moments (m, v) from NVFP4 state."""
    args, _keep, outs = _qadamw_decode_args(state, rht_seed, m_out, v_out)
    _check(lib().nvfp4_qadamw_decode(*args), "nvfp4_qadamw_decode")
    return outs


def bind_qadamw_encode(m, v, state: QAdamWState, workspace: torch.Tensor, rht_seed: int, sr_seed: int,
                       sr_stream: int = 0) -> "BoundCall":
    args, keep, state = _qadamw_encode_args(m, v, rht_seed, sr_seed, sr_stream, state, workspace)
    return BoundCall(lib().nvfp4_qadamw_encode, args, keep, "nvfp4_qadamw_encode", state)


def bind_qadamw_decode(state: QAdamWState, rht_seed: int, m_out, v_out) -> "BoundCall":
    args, keep, outs = _qadamw_decode_args(state, rht_seed, m_out, v_out)
    return BoundCall(lib().nvfp4_qadamw_decode, args, keep, "nvfp4_qadamw_decode", outs)


class BoundCall:
    """One C-ABI call with its arguments marshalled once (pointers, sizes,
    option structs and the current stream at bind time).  Calling it only
    enqueues the kernels again; for loops that repeat the same call on the
    same buffers, where per-call argument conversion would otherwise
    dominate the host time."""

    def __init__(self, fn, args, keep, what: str, result=None):
        self._fn, self._args, self._keep, self._what, self.result = fn, args, keep, what, result

    def __call__(self):
        st = self._fn(*self._args)
        if st != OK:
            raise NVFP4Error(st, self._what)
        return self.result


def bind_quantize(x: torch.Tensor, out: QTensor, workspace: torch.Tensor, axis: int = ALONG_COLS,
                  rounding: int = RNE, sr_seed: int = 0, sr_stream: int = 0, rht: bool = False,
                  rht_seed: int = 0) -> BoundCall:
    """quantize() bound to fixed buffers and the current stream."""
    args, keep, out = _quantize_args(x, axis, rounding, sr_seed, sr_stream, rht, rht_seed, out, workspace)
    return BoundCall(lib().nvfp4_quantize, args, keep, "nvfp4_quantize", out)


def _quantize_group_args(xs, rounding: int, sr_seed: int, sr_stream: int, rht: bool, rht_seed: int,
                         outs, workspace: torch.Tensor | None):
    """Validated ctypes arguments of one nvfp4_quantize_group call (and its outputs)."""
    if not 1 <= len(xs) <= 4:
        raise ValueError("a group holds 1 to 4 tensors")
    if len({x.dtype for x in xs}) != 1:
        raise TypeError("all tensors of a group must have one dtype")
    outs = list(outs) if outs is not None else [None] * len(xs)
    jobs = (QuantJobC * len(xs))()
    x3s = []
    for i, x in enumerate(xs):
        x3 = x.unsqueeze(0) if x.dim() == 2 else x
        if x3.dim() != 3:
            raise ValueError("x must be 2-D or 3-D")
        if x3.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("x must be bfloat16 or float32")
        if x3.size(2) > 1 and x3.stride(2) != 1:
            raise ValueError("the last dimension of x must be contiguous")
        b, r, c = x3.shape
        if outs[i] is None:
            outs[i] = QTensor.empty(b, r, c, x.device)
        jobs[i] = QuantJobC(x3.data_ptr(), b, r, c, x3.stride(1) if r > 1 else c,
                            x3.stride(0) if b > 1 else r * c, outs[i].c_struct())
        x3s.append(x3)
    if workspace is None:
        workspace = new_workspace(nvfp4_quantize_group_workspace_size(), xs[0].device)
    opts = QuantOptsC(rounding, int(bool(rht)), sr_seed, rht_seed, sr_stream, 0)
    args = (jobs, len(xs), BF16 if xs[0].dtype == torch.bfloat16 else F32, ctypes.byref(opts),
            workspace.data_ptr(), workspace.numel(), _stream(xs[0].device))
    return args, (jobs, opts, x3s, workspace), outs


def quantize_group(xs, rounding: int = RNE, sr_seed: int = 0, sr_stream: int = 0, rht: bool = False,
                   rht_seed: int = 0, outs=None, workspace: torch.Tensor | None = None) -> list:
    """Quantize 1-4 tensors along their last dimension with shared options,
    each with its own tensor scale (same results as quantize() on each)."""
    args, _keep, outs = _quantize_group_args(xs, rounding, sr_seed, sr_stream, rht, rht_seed, outs, workspace)
    _check(lib().nvfp4_quantize_group(*args), "nvfp4_quantize_group")
    return outs


def bind_quantize_group(xs, outs, workspace: torch.Tensor, rounding: int = RNE, sr_seed: int = 0,
                        sr_stream: int = 0, rht: bool = False, rht_seed: int = 0) -> BoundCall:
    """quantize_group() bound to fixed buffers and the current stream."""
    args, keep, outs = _quantize_group_args(xs, rounding, sr_seed, sr_stream, rht, rht_seed, outs, workspace)
    return BoundCall(lib().nvfp4_quantize_group, args, keep, "nvfp4_quantize_group", outs)


def gemm(a: QTensor, b: QTensor, out_dtype: torch.dtype = torch.bfloat16, alpha: float = 1.0,
         out: torch.Tensor | None = None, tile: tuple[int, int] | None = None) -> torch.Tensor:
    """C[b] = alpha * A^[b] . B^[b]^T -> [batch][M][N] (squeezed to 2-D when batch == 1).
    ``tile`` = (tile_m, tile_n) requests a workgroup tile (nvfp4_gemm_ex)."""
    created = out is None
    if created:
        out = torch.empty(a.batch, a.rows, b.rows, dtype=out_dtype, device=a.codes.device)
    args, _keep = _gemm_args(a, b, out, alpha)
    if tile is None:
        _check(lib().nvfp4_gemm(*args), "nvfp4_gemm")
    else:
        _check(lib().nvfp4_gemm_ex(*args[:-1], int(tile[0]), int(tile[1]), args[-1]), "nvfp4_gemm_ex")
    return out[0] if created and a.batch == 1 else out


def _gemm_args(a: QTensor, b: QTensor, out: torch.Tensor, alpha: float):
    o3 = out if out.dim() == 3 else out.unsqueeze(0)
    ca, cb = a.c_struct(), b.c_struct()
    args = (ctypes.byref(ca), ctypes.byref(cb), o3.data_ptr(), BF16 if o3.dtype == torch.bfloat16 else F32,
            o3.stride(1) if o3.size(1) > 1 else o3.size(2),
            o3.stride(0) if o3.size(0) > 1 else o3.size(1) * o3.size(2), ctypes.c_float(alpha),
            _stream(a.codes.device))
    return args, (ca, cb, o3)


def quantize_workspace_check(workspace: torch.Tensor) -> int:
    """Status of a quantize workspace (waits for the current stream):
    OK, or ETIMEOUT once a single-pass barrier wait on it has expired."""
    return lib().nvfp4_quantize_workspace_check(workspace.data_ptr(), workspace.numel(),
                                                _stream(workspace.device))


def bind_gemm(a: QTensor, b: QTensor, out: torch.Tensor, alpha: float = 1.0) -> BoundCall:
    """gemm() bound to fixed operands, output and the current stream."""
    args, keep = _gemm_args(a, b, out, alpha)
    return BoundCall(lib().nvfp4_gemm, args, keep, "nvfp4_gemm", out)


def _linear_args(x, w, dy, y, dx, dw, sr_seed, rht_seed, wgrad_sr_x, workspace):
    M, K = x.shape
    N = w.shape[0]
    for t in (x, w, dy):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("x, w, dy must be contiguous bfloat16")
    cfg = LinearCfgC(sr_seed, rht_seed, int(bool(wgrad_sr_x)), F32 if dw.dtype == torch.float32 else BF16)
    args = (x.data_ptr(), w.data_ptr(), dy.data_ptr(), y.data_ptr(), dx.data_ptr(), dw.data_ptr(), M, N, K,
            ctypes.byref(cfg), workspace.data_ptr(), workspace.numel(), _stream(x.device))
    return args, (cfg, x, w, dy, y, dx, dw, workspace)


def _linear_outputs(x, w, dw_dtype):
    M, K = x.shape
    N = w.shape[0]
    return (torch.empty(M, N, dtype=torch.bfloat16, device=x.device),
            torch.empty(M, K, dtype=torch.bfloat16, device=x.device),
            torch.empty(N, K, dtype=dw_dtype, device=x.device))


def linear_fwd_bwd(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, sr_seed: int, rht_seed: int,
                   wgrad_sr_x: bool = True, dw_dtype: torch.dtype = torch.bfloat16,
                   workspace: torch.Tensor | None = None):
    """Fprop, Dgrad and Wgrad of Y = X W^T in NVFP4; returns (Y, dX, dW)."""
    y, dx, dw = _linear_outputs(x, w, dw_dtype)
    if workspace is None:
        workspace = new_workspace(nvfp4_linear_workspace_size(x.shape[0], w.shape[0], x.shape[1]), x.device)
    args, _keep = _linear_args(x, w, dy, y, dx, dw, sr_seed, rht_seed, wgrad_sr_x, workspace)
    _check(lib().nvfp4_linear_fwd_bwd(*args), "nvfp4_linear_fwd_bwd")
    return y, dx, dw


LINEAR_VIEWS = ("X", "W", "dY", "W^T", "dY^T", "X^T")


def linear_view(workspace: torch.Tensor, M: int, N: int, K: int, which: int) -> QTensor:
    """Quantized view `which` (index into LINEAR_VIEWS) that nvfp4_linear_fwd_bwd
    left in `workspace`, as tensors aliasing the workspace memory."""
    q = QTensorC()
    _check(lib().nvfp4_linear_view(workspace.data_ptr(), workspace.numel(), M, N, K, which, ctypes.byref(q)),
           "nvfp4_linear_view")
    base = workspace.data_ptr()
    rows, cols = q.rows, q.cols

    def sub(ptr, n):
        off = ptr - base
        return workspace[off:off + n]

    return QTensor(sub(q.codes, rows * cols // 2).view(1, rows, cols // 2),
                   sub(q.scales, rows * cols // 16).view(1, rows, cols // 16),
                   sub(q.tensor_scale, 4).view(torch.float32), 1, rows, cols)


def bind_linear_fwd_bwd(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, y: torch.Tensor, dx: torch.Tensor,
                        dw: torch.Tensor, workspace: torch.Tensor, sr_seed: int, rht_seed: int,
                        wgrad_sr_x: bool = True) -> BoundCall:
    """linear_fwd_bwd() bound to fixed inputs, outputs, workspace and the current stream."""
    args, keep = _linear_args(x, w, dy, y, dx, dw, sr_seed, rht_seed, wgrad_sr_x, workspace)
    return BoundCall(lib().nvfp4_linear_fwd_bwd, args, keep, "nvfp4_linear_fwd_bwd", (y, dx, dw))


# --- GEMM with an FP32 addend, Newton-Schulz in NVFP4 ---------------------

def gemm_axpby(a: QTensor, b: QTensor, c_in: torch.Tensor, beta: float, alpha: float = 1.0,
               out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """out = alpha sA sB A^ B^^T + beta c_in (c_in FP32 [batch][M][N] or [M][N],
    last dimension contiguous); `out` may be c_in itself (FP32)."""
    M, N = a.rows, b.rows
    if c_in.dtype != torch.float32 or c_in.stride(-1) != 1:
        raise ValueError("c_in must be float32 with a contiguous last dimension")
    c3 = c_in.view(1, M, N) if c_in.dim() == 2 else c_in
    if tuple(c3.shape) != (a.batch, M, N):
        raise ValueError("c_in must be [batch][M][N]")
    if out is None:
        out = torch.empty((a.batch, M, N), dtype=out_dtype, device=a.codes.device)
    o3 = out.view(1, M, N) if out.dim() == 2 else out
    if o3.stride(-1) != 1:
        raise ValueError("out must have a contiguous last dimension")
    qa, qb = a.c_struct(), b.c_struct()
    _check(lib().nvfp4_gemm_axpby(ctypes.byref(qa), ctypes.byref(qb), o3.data_ptr(),
                                  BF16 if o3.dtype == torch.bfloat16 else F32, o3.stride(1),
                                  o3.stride(0), alpha, c3.data_ptr(), c3.stride(1), c3.stride(0), beta,
                                  _stream(o3.device)), "nvfp4_gemm_axpby")
    return out


NS_VIEWS = ("X", "X^T", "A", "B")


def _ns_args(g, coeffs, clip_quantile, clip_mask, out, workspace, product=0):
    if g.dim() != 2 or g.dtype not in (torch.float32, torch.bfloat16) or (g.size(1) > 1 and g.stride(1) != 1):
        raise ValueError("g must be a 2-D float32 or bfloat16 tensor with contiguous rows")
    m, n = g.shape
    co = np.ascontiguousarray(np.asarray(coeffs, dtype=np.float32).reshape(-1, 3))
    if out is None:
        out = torch.empty(m, n, dtype=torch.float32, device=g.device)
    if workspace is None:
        workspace = new_workspace(nvfp4_ns_workspace_size(m, n), g.device)
    cfg = NsCfgC(clip_quantile, clip_mask, product)
    args = (g.data_ptr(), BF16 if g.dtype == torch.bfloat16 else F32, m, n, g.stride(0) if m > 1 else n,
            co.ctypes.data, co.shape[0], ctypes.byref(cfg), out.data_ptr(), out.stride(0) if m > 1 else n,
            workspace.data_ptr(), workspace.numel(), _stream(g.device))
    return args, (co, cfg, g, out, workspace), out


def ns_orthogonalize(g: torch.Tensor, coeffs, clip_quantile: float = 0.99, clip_mask: int = 1,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     product: int = 0) -> torch.Tensor:
    """Newton-Schulz orthogonalization of g [m][n] with every product in NVFP4;
    coeffs is a sequence of (a, b, c) per step.  product: how B^ X^ is
    launched (0 automatic, 1 as [m][n], 2 as its transpose)."""
    args, _keep, out = _ns_args(g, coeffs, clip_quantile, clip_mask, out, workspace, product)
    _check(lib().nvfp4_ns_orthogonalize(*args), "nvfp4_ns_orthogonalize")
    return out


def bind_ns_orthogonalize(g, coeffs, out, workspace, clip_quantile: float = 0.99, clip_mask: int = 1) -> BoundCall:
    args, keep, out = _ns_args(g, coeffs, clip_quantile, clip_mask, out, workspace)
    return BoundCall(lib().nvfp4_ns_orthogonalize, args, keep, "nvfp4_ns_orthogonalize", out)


def ns_internals(workspace: torch.Tensor, m: int, n: int) -> dict:
    """The last step's intermediates in a Newton-Schulz workspace, as tensors
    aliasing it: x_prev [m][n], a, b [m][m] (FP32), clip [3] values (float32
    scalars), inv_norm, and the views X, X^T, A, B (QTensor)."""
    st = NsStateC()
    _check(lib().nvfp4_ns_internals(workspace.data_ptr(), workspace.numel(), m, n, ctypes.byref(st)),
           "nvfp4_ns_internals")
    base = workspace.data_ptr()

    def sub(ptr, nbytes):
        off = ptr - base
        return workspace[off:off + nbytes]

    views = {}
    for i, name in enumerate(NS_VIEWS):
        q = st.view[i]
        views[name] = QTensor(sub(q.codes, q.rows * q.cols // 2).view(1, q.rows, q.cols // 2),
                              sub(q.scales, q.rows * q.cols // 16).view(1, q.rows, q.cols // 16),
                              sub(q.tensor_scale, 4).view(torch.float32), 1, q.rows, q.cols)
    return {"x_prev": sub(st.x_prev, 4 * m * n).view(torch.float32).view(m, n),
            "a": sub(st.a, 4 * m * m).view(torch.float32).view(m, m),
            "b": sub(st.b, 4 * m * m).view(torch.float32).view(m, m),
            "clip": [sub(st.clip[i], 4).view(torch.float32) for i in range(3)],
            "inv_norm": sub(st.inv_norm, 4).view(torch.float32),
            "views": views}


# --- LoRA-style forward: residual in NVFP4, subspace in BF16 ---------------

def nvfp4_lora_workspace_size(M: int, K: int, r: int) -> int:
    return int(lib().nvfp4_lora_workspace_size(M, K, r))


def _lora_args(x, w_res: QTensor, l1, l2, beta, out_dtype, out, workspace):
    for t, name in ((x, "x"), (l1, "l1"), (l2, "l2")):
        if t.dim() != 2 or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D bfloat16 tensor")
    M, K = x.shape
    r = l1.size(0)
    N = w_res.rows
    if l1.size(1) != K or tuple(l2.shape) != (N, r) or w_res.cols != K:
        raise ValueError("shapes: x [M][K], w_res [N][K], l1 [r][K], l2 [N][r]")
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = new_workspace(nvfp4_lora_workspace_size(M, K, r), x.device)
    qw = w_res.c_struct()
    args = (x.data_ptr(), ctypes.byref(qw), l1.data_ptr(), l2.data_ptr(), M, N, K, r, beta, out.data_ptr(),
            BF16 if out.dtype == torch.bfloat16 else F32, out.stride(0) if M > 1 else N, workspace.data_ptr(),
            workspace.numel(), _stream(x.device))
    return args, (qw, x, l1, l2, out, workspace), out


def lora_forward(x: torch.Tensor, w_res: QTensor, l1: torch.Tensor, l2: torch.Tensor, beta: float,
                 out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W_res^T (NVFP4) + beta (X L1^T) L2^T (BF16) for x [M][K] BF16."""
    args, _keep, out = _lora_args(x, w_res, l1, l2, beta, out_dtype, out, workspace)
    _check(lib().nvfp4_lora_forward(*args), "nvfp4_lora_forward")
    return out


def bind_lora_forward(x, w_res: QTensor, l1, l2, beta: float, out: torch.Tensor, workspace: torch.Tensor) -> BoundCall:
    args, keep, out = _lora_args(x, w_res, l1, l2, beta, out.dtype, out, workspace)
    return BoundCall(lib().nvfp4_lora_forward, args, keep, "nvfp4_lora_forward", out)


def lora_internals(workspace: torch.Tensor, M: int, K: int, r: int):
    """(X view, T [M][r] bfloat16) held by a LoRA workspace, aliasing it."""
    q = QTensorC()
    t = ctypes.c_void_p()
    _check(lib().nvfp4_lora_internals(workspace.data_ptr(), workspace.numel(), M, K, r, ctypes.byref(q),
                                      ctypes.byref(t)), "nvfp4_lora_internals")
    base = workspace.data_ptr()

    def sub(ptr, nbytes):
        off = ptr - base
        return workspace[off:off + nbytes]

    xv = QTensor(sub(q.codes, M * K // 2).view(1, M, K // 2), sub(q.scales, M * K // 16).view(1, M, K // 16),
                 sub(q.tensor_scale, 4).view(torch.float32), 1, M, K)
    return xv, sub(t.value, 2 * M * r).view(torch.bfloat16).view(M, r)
