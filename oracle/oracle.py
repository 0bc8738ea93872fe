"""ctypes front end of the plain-C NVFP4 oracle (oracle/nvfp4_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The HIP library and its Python
binding never import this module.

Arrays are numpy.  BF16 tensors are passed as their raw bit patterns in
``numpy.uint16`` arrays (numpy has no bfloat16); FP32 as ``numpy.float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
ALONG_COLS, ALONG_ROWS = 0, 1
RNE, SR = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no FMA contraction, no fast-math."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
             "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=not os.path.exists(_LIB))
        L = ctypes.CDLL(_LIB)
        i64, u32, u64, vp = ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p
        L.oracle_e2m1_decode.argtypes = [ctypes.c_int]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_encode_rne.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_rne.restype = ctypes.c_int
        L.oracle_e2m1_encode_sr.argtypes = [ctypes.c_float, u32]
        L.oracle_e2m1_encode_sr.restype = ctypes.c_int
        L.oracle_e4m3_decode.argtypes = [ctypes.c_int]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode_rne_sat.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_rne_sat.restype = ctypes.c_int
        L.oracle_e2m1_encode_rne_array.argtypes = [vp, i64, vp]
        L.oracle_e4m3_encode_rne_sat_array.argtypes = [vp, i64, vp]
        L.oracle_e2m1_encode_sr_all_words.argtypes = [vp, i64, vp]
        L.oracle_e2m1_encode_sr_pairs.argtypes = [vp, vp, i64, vp]
        L.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        L.oracle_sr_word.argtypes = [u64, u32, u64]
        L.oracle_sr_word.restype = u32
        L.oracle_rht_signs.argtypes = [u64, vp]
        L.oracle_rht16.argtypes = [vp, vp]
        L.oracle_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_int,
                                      ctypes.c_int, u64, u32, ctypes.c_int, u64, vp, vp, vp]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_dequantize.argtypes = [vp, vp, ctypes.c_float, i64, i64, vp]
        L.oracle_gemm_ref.argtypes = [vp, vp, ctypes.c_float, vp, vp, ctypes.c_float, i64, i64,
                                      i64, i64, ctypes.c_double, vp, i64, vp, vp]
        L.oracle_gemm_ref.restype = ctypes.c_int
        L.oracle_sqrt_demean16.argtypes = [vp]
        L.oracle_sqrt_demean16.restype = ctypes.c_uint16
        L.oracle_qadamw_encode.argtypes = [vp, vp, i64, i64, i64, u64, u64, u32, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_qadamw_encode.restype = ctypes.c_int
        L.oracle_qadamw_decode.argtypes = [vp, vp, ctypes.c_float, vp, vp, ctypes.c_float, vp, i64, i64, i64,
                                           u64, vp, vp]
        L.oracle_qadamw_decode.restype = ctypes.c_int
        L.oracle_abs_quantile.argtypes = [vp, i64, ctypes.c_double, vp]
        L.oracle_abs_quantile.restype = ctypes.c_int
        L.oracle_clip.argtypes = [vp, i64, ctypes.c_float, vp]
        L.oracle_frobenius_normalize.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp]
        L.oracle_frobenius_normalize.restype = ctypes.c_float
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return ctypes.c_void_p(a.ctypes.data)


# --- element codecs --------------------------------------------------------

def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(int(code))


def e2m1_encode_rne(q: float) -> int:
    return lib().oracle_e2m1_encode_rne(float(q))


def e2m1_encode_sr(q: float, u: int) -> int:
    return lib().oracle_e2m1_encode_sr(float(q), int(u))


def e4m3_decode(byte: int) -> float:
    return lib().oracle_e4m3_decode(int(byte))


def e4m3_encode(y: float) -> int:
    return lib().oracle_e4m3_encode_rne_sat(float(y))


def e2m1_encode_rne_array(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.shape, dtype=np.uint8)
    lib().oracle_e2m1_encode_rne_array(_ptr(q), q.size, _ptr(out))
    return out


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_rne_sat_array(_ptr(y), y.size, _ptr(out))
    return out


def e2m1_encode_sr_pairs(q: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Code of q[i] under the 16-bit word u[i]."""
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(-1)
    u = np.ascontiguousarray(u, dtype=np.uint32).reshape(-1)
    assert q.size == u.size
    out = np.empty(q.size, dtype=np.uint8)
    lib().oracle_e2m1_encode_sr_pairs(_ptr(q), _ptr(u), q.size, _ptr(out))
    return out


def e2m1_encode_sr_all_words(q: np.ndarray) -> np.ndarray:
    """[len(q)][65536] codes: every value of q under every 16-bit word."""
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(-1)
    out = np.empty((q.size, 65536), dtype=np.uint8)
    lib().oracle_e2m1_encode_sr_all_words(_ptr(q), q.size, _ptr(out))
    return out


# --- random numbers and the Hadamard transform -----------------------------

def philox4x32_10(counter, key) -> np.ndarray:
    c = np.asarray(counter, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_word(seed: int, stream: int, n: int) -> int:
    return int(lib().oracle_sr_word(seed, stream, n))


def rht_signs(seed: int) -> np.ndarray:
    s = np.zeros(16, dtype=np.float32)
    lib().oracle_rht_signs(seed, _ptr(s))
    return s


def rht16(v: np.ndarray, signs: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(v, dtype=np.float32).copy()
    s = np.ascontiguousarray(signs, dtype=np.float32)
    assert w.shape == (16,) and s.shape == (16,)
    lib().oracle_rht16(_ptr(w), _ptr(s))
    return w


# --- quantize / dequantize / GEMM -----------------------------------------

@dataclass
class QTensor:
    """One quantized view: codes [batch][rows][cols/2], scales [batch][rows][cols/16]."""
    codes: np.ndarray
    scales: np.ndarray
    tensor_scale: np.float32
    batch: int
    rows: int
    cols: int


def quantize(x: np.ndarray, dtype: int, axis: int = ALONG_COLS, rounding: int = RNE,
             sr_seed: int = 0, sr_stream: int = 0, rht: bool = False, rht_seed: int = 0,
             batch: int | None = None) -> QTensor:
    """Quantize a 2-D [rows][cols] or 3-D [batch][rows][cols] array.

    ``dtype`` is F32 (x float32) or BF16 (x uint16 bit patterns).  For
    ALONG_ROWS the quantized view is the per-batch transpose of x."""
    x = np.ascontiguousarray(x)
    if dtype == BF16:
        assert x.dtype == np.uint16
    else:
        assert x.dtype == np.float32
    if x.ndim == 2:
        x3 = x.reshape(1, *x.shape)
    else:
        x3 = x
    b, r, c = x3.shape
    qr, qc = (r, c) if axis == ALONG_COLS else (c, r)
    codes = np.zeros((b, qr, qc // 2), dtype=np.uint8)
    scales = np.zeros((b, qr, qc // 16), dtype=np.uint8)
    st = np.zeros(1, dtype=np.float32)
    rc = lib().oracle_quantize(_ptr(x3), dtype, b, r, c, c, r * c, axis, rounding, sr_seed,
                               sr_stream, int(bool(rht)), rht_seed, _ptr(codes), _ptr(scales),
                               _ptr(st))
    if rc != 0:
        raise ValueError(f"oracle_quantize rejected the arguments (rc={rc})")
    return QTensor(codes, scales, np.float32(st[0]), b, qr, qc)


def dequantize(q: QTensor) -> np.ndarray:
    out = np.empty((q.batch, q.rows, q.cols), dtype=np.float64)
    lib().oracle_dequantize(_ptr(q.codes), _ptr(q.scales), float(q.tensor_scale),
                            q.batch * q.rows, q.cols, _ptr(out))
    return out


def gemm_ref(a: QTensor, b: QTensor, alpha: float = 1.0, batch_index: int = 0,
             rows: np.ndarray | None = None):
    """Reference y = alpha * sA * sB * A^ . B^T and its bound sum |.| for one batch
    index and the selected rows of A (all rows when ``rows`` is None)."""
    assert a.cols == b.cols
    M, N, K = a.rows, b.rows, a.cols
    if rows is None:
        sel = None
        nsel = M
        rp = ctypes.c_void_p(0)
    else:
        sel = np.ascontiguousarray(rows, dtype=np.int64)
        nsel = sel.size
        rp = _ptr(sel)
    y = np.empty((nsel, N), dtype=np.float64)
    s = np.empty((nsel, N), dtype=np.float64)
    rc = lib().oracle_gemm_ref(_ptr(a.codes), _ptr(a.scales), float(a.tensor_scale),
                               _ptr(b.codes), _ptr(b.scales), float(b.tensor_scale), M, N, K,
                               batch_index, float(alpha), rp, nsel, _ptr(y), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_gemm_ref failed (rc={rc})")
    return y, s


# --- G3: acceptance of a GEMM output against the reference ---------------

FP32_TOL = 1e-5


def bf16_rne_bits(y: np.ndarray) -> np.ndarray:
    """Exact round-to-nearest-even of float64 values to BF16 bit patterns."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.shape, dtype=np.int64)
    nz = y != 0
    # BF16 shares FP32's exponent range: below 2^-126 the spacing stays 2^-133
    e = np.maximum(np.floor(np.log2(np.abs(y[nz]))), -126.0)
    scale = np.exp2(e - 7)
    r = np.round(y[nz] / scale) * scale  # half-to-even on an exact quotient
    out[nz] = (np.float32(r).view(np.uint32) >> 16).astype(np.int64)
    out[~nz] = (np.signbit(y[~nz]).astype(np.int64) << 15)
    return out


def gemm_accept(y: np.ndarray, y_ref: np.ndarray, sabs: np.ndarray, bf16: bool) -> dict:
    """Counts of the G3 rule over the elements of y (FP32 values, or BF16
    values widened to FP32):
      FP32 out: |y - y_ref| <= 1e-5 * sabs                      -> "ok";
      BF16 out: y is RNE_bf16(y_ref) or one of its two BF16 neighbours
                (1 ulp)                                         -> "ok";
                otherwise |y - y_ref| <= 1e-5 * sabs + ulp_bf16(y) / 2 (FP32
                accumulation error near cancellation)           -> "cancel_only";
      anything else                                             -> "fail"."""
    y = np.asarray(y)
    if not bf16:
        err = np.abs(y.astype(np.float64) - y_ref)
        ok = err <= FP32_TOL * sabs
        return {"n": int(y.size), "ok": int(ok.sum()), "cancel_only": 0, "fail": int((~ok).sum())}
    ybits = (np.asarray(y, dtype=np.float32).view(np.uint32) >> 16).astype(np.int64)
    rbits = bf16_rne_bits(y_ref)

    def mono(b):  # signed magnitude -> a monotone integer, so neighbours differ by 1
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)

    ulp_ok = np.abs(mono(ybits) - mono(rbits)) <= 1
    yv = np.asarray(y, dtype=np.float64)
    ulp_y = np.exp2(np.floor(np.log2(np.maximum(np.abs(yv), 1e-300))) - 7)
    cancel_ok = np.abs(yv - y_ref) <= FP32_TOL * sabs + 0.5 * ulp_y
    return {"n": int(y.size), "ok": int(ulp_ok.sum()), "cancel_only": int((~ulp_ok & cancel_ok).sum()),
            "fail": int((~(ulp_ok | cancel_ok)).sum())}


# --- S1..S4: AdamW moments in NVFP4 ---------------------------------------

@dataclass
class QAdamWState:
    """m and v views [1][rows][cols] and the BF16 block means [rows][cols/16]."""
    m: QTensor
    v: QTensor
    v_means: np.ndarray


def sqrt_demean16(v: np.ndarray):
    """S1 on one block: (residuals, BF16 bits of the mean)."""
    b = np.ascontiguousarray(v, dtype=np.float32).copy()
    assert b.shape == (16,)
    mb = lib().oracle_sqrt_demean16(_ptr(b))
    return b, int(mb)


def qadamw_encode(m: np.ndarray, v: np.ndarray, rht_seed: int, sr_seed: int, sr_stream: int = 0) -> QAdamWState:
    m = np.ascontiguousarray(m, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert m.shape == v.shape and m.ndim == 2
    rows, cols = m.shape

    def view():
        return QTensor(np.zeros((1, rows, cols // 2), np.uint8), np.zeros((1, rows, cols // 16), np.uint8),
                       np.float32(0), 1, rows, cols)
    qm, qv = view(), view()
    means = np.zeros((rows, cols // 16), np.uint16)
    sts = np.zeros(2, np.float32)
    rc = lib().oracle_qadamw_encode(_ptr(m), _ptr(v), rows, cols, cols, rht_seed, sr_seed, sr_stream,
                                    _ptr(qm.codes), _ptr(qm.scales), ctypes.c_void_p(sts.ctypes.data),
                                    _ptr(qv.codes), _ptr(qv.scales), ctypes.c_void_p(sts.ctypes.data + 4),
                                    _ptr(means))
    if rc != 0:
        raise ValueError(f"oracle_qadamw_encode failed (rc={rc})")
    qm.tensor_scale, qv.tensor_scale = np.float32(sts[0]), np.float32(sts[1])
    return QAdamWState(qm, qv, means)


def qadamw_decode(st: QAdamWState, rht_seed: int):
    """(m, v) FP32 [rows][cols] reconstructed from the state."""
    rows, cols = st.m.rows, st.m.cols
    m = np.zeros((rows, cols), np.float32)
    v = np.zeros((rows, cols), np.float32)
    means = np.ascontiguousarray(st.v_means, dtype=np.uint16)
    rc = lib().oracle_qadamw_decode(_ptr(np.ascontiguousarray(st.m.codes)), _ptr(np.ascontiguousarray(st.m.scales)),
                                    float(st.m.tensor_scale), _ptr(np.ascontiguousarray(st.v.codes)),
                                    _ptr(np.ascontiguousarray(st.v.scales)), float(st.v.tensor_scale),
                                    _ptr(means), rows, cols, cols, rht_seed, _ptr(m), _ptr(v))
    if rc != 0:
        raise ValueError(f"oracle_qadamw_decode failed (rc={rc})")
    return m, v


# --- R1..R3 and the Newton-Schulz step in NVFP4 ----------------------------

def abs_quantile(x: np.ndarray, q: float) -> np.float32:
    """R1: the ceil(q N)-th smallest |x|."""
    a = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.zeros(1, np.float32)
    rc = lib().oracle_abs_quantile(_ptr(a), a.size, float(q), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_abs_quantile failed (rc={rc})")
    return out[0]


def clip(x: np.ndarray, p) -> np.ndarray:
    """R2: x clamped to [-p, p]."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(a)
    lib().oracle_clip(_ptr(a), a.size, float(np.float32(p)), _ptr(out))
    return out


def frobenius_normalize(g: np.ndarray, dtype: int):
    """R3: (x = fl(g * f), f = fl32(1 / (||g||_F + 1e-7)))."""
    a = np.ascontiguousarray(g)
    rows, cols = a.shape
    x = np.empty((rows, cols), np.float32)
    f = lib().oracle_frobenius_normalize(_ptr(a), dtype, rows, cols, cols, _ptr(x))
    return x, np.float32(f)


def gemm_axpby_ref(a: QTensor, b: QTensor, alpha: float, c_in: np.ndarray, beta: float, rows=None):
    """y_ref = alpha sA sB A^ B^^T + beta C (float64) and its bound
    sum |alpha sA sB a b| + |beta C| for the selected rows (batch 0)."""
    y, sabs = gemm_ref(a, b, alpha, 0, rows)
    c = np.asarray(c_in, dtype=np.float64)
    if rows is not None:
        c = c[np.asarray(rows)]
    bc = float(np.float32(beta)) * c
    return y + bc, sabs + np.abs(bc)


def ns_quantize(t: np.ndarray, q: float | None, axis: int = ALONG_COLS):
    """The NVFP4 view of a Newton-Schulz operand: clipped at its q order
    statistic of |t| (q None: no clipping), RNE, no transform."""
    t = np.ascontiguousarray(t, dtype=np.float32)
    p = None
    if q is not None:
        p = abs_quantile(t, q)
        t = clip(t, p)
    return quantize(t, F32, axis=axis), p


def ns_chain(g: np.ndarray, dtype: int, coeffs, q: float | None, mask: int, quant: bool = True):
    """The whole iteration on the host: X_0 = R3(g); per step (a, b, c):
    A = X^ X^^T, B = c A^ A^^T + b A, X <- B^ X^T^ + a X, with the NVFP4
    views (clipped where `mask` says) when `quant`, or the FP64 values
    themselves otherwise; A, B and X are rounded to FP32 between steps as the
    products store them.  Returns X as float32."""
    x, _ = frobenius_normalize(g, dtype)
    for a_, b_, c_ in coeffs:
        a_, b_, c_ = float(np.float32(a_)), float(np.float32(b_)), float(np.float32(c_))
        if quant:
            qx, _ = ns_quantize(x, q if mask & 1 else None)
            qxt, _ = ns_quantize(x.T, q if mask & 1 else None)
            A = gemm_ref(qx, qx)[0].astype(np.float32)
            qa, _ = ns_quantize(A, q if mask & 2 else None)
            B = (c_ * gemm_ref(qa, qa)[0] + b_ * A.astype(np.float64)).astype(np.float32)
            qb, _ = ns_quantize(B, q if mask & 4 else None)
            x = (gemm_ref(qb, qxt)[0] + a_ * x.astype(np.float64)).astype(np.float32)
        else:
            xd = x.astype(np.float64)
            A = (xd @ xd.T).astype(np.float32).astype(np.float64)
            B = (c_ * (A @ A.T) + b_ * A).astype(np.float32).astype(np.float64)
            x = (B @ xd + a_ * xd).astype(np.float32)
    return x


# --- L1, L2: the LoRA-style forward (residual NVFP4, subspace BF16) -------

def bf16_values(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64 values (exact)."""
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def lora_down_ref(x_bits: np.ndarray, l1_bits: np.ndarray, rows=None):
    """L1: T = X L1^T in float64 (before its BF16 rounding) and sum |X| |L1|^T
    for the selected rows; X [M][K], L1 [r][K] as BF16 bit patterns."""
    x = bf16_values(x_bits if rows is None else np.asarray(x_bits)[np.asarray(rows)])
    l1 = bf16_values(l1_bits)
    return x @ l1.T, np.abs(x) @ np.abs(l1).T


def lora_forward_ref(qx: QTensor, qw: QTensor, t_bits: np.ndarray, l2_bits: np.ndarray, beta: float, rows=None):
    """L2: y = sX sW X^ W^^T + beta T L2^T in float64 for the selected rows,
    with T the BF16 T (bit patterns [M][r]) and its bound."""
    y, s = gemm_ref(qx, qw, 1.0, 0, rows)
    t = bf16_values(t_bits if rows is None else np.asarray(t_bits)[np.asarray(rows)])
    l2 = bf16_values(l2_bits)
    b = float(np.float32(beta))
    return y + b * (t @ l2.T), s + abs(b) * (np.abs(t) @ np.abs(l2).T)
