"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every entry point include/nvfp4.h declares, and rejects bad arguments with the
documented status codes before making any HIP call."""
import ctypes
import re

import pytest

import bit_block_scaled_nvfp4_amd as nv

FAKE = 0x10000  # aligned, non-null; never dereferenced because validation fails first


def declared_functions():
    text = open(nv.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = nv.lib()
    names = declared_functions()
    assert {"nvfp4_quantize", "nvfp4_gemm", "nvfp4_linear_fwd_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for s in range(8):
        assert nv.status_string(s) and nv.status_string(s) != "unknown status"
    assert nv.status_string(99) == "unknown status"
    assert nv.nvfp4_version() >> 16 == 1
    assert nv.nvfp4_quantize_workspace_size() == 4096
    assert nv.nvfp4_quantize_group_workspace_size() == 16384


def _q(batch, rows, cols, codes=FAKE, scales=FAKE, st=FAKE):
    return nv.QTensorC(codes, scales, st, batch, rows, cols)


def _quant(**kw):
    a = dict(x=FAKE, dt=nv.BF16, b=1, r=32, c=64, ld=64, bs=32 * 64, axis=nv.ALONG_COLS,
             opts=nv.QuantOptsC(0, 0, 0, 0, 0, 0), out=None, ws=FAKE, wsb=4096)
    a.update(kw)
    if a["out"] is None:
        qr, qc = (a["r"], a["c"]) if a["axis"] == nv.ALONG_COLS else (a["c"], a["r"])
        a["out"] = _q(a["b"], qr, qc)
    return nv.nvfp4_quantize(a["x"], a["dt"], a["b"], a["r"], a["c"], a["ld"], a["bs"], a["axis"],
                             a["opts"], a["out"], a["ws"], a["wsb"], None)


def test_quantize_argument_errors():
    assert _quant(dt=7) == nv.EINVAL
    assert _quant(axis=2) == nv.EINVAL
    assert _quant(opts=nv.QuantOptsC(2, 0, 0, 0, 0, 0)) == nv.EINVAL
    assert _quant(opts=nv.QuantOptsC(0, 3, 0, 0, 0, 0)) == nv.EINVAL
    assert _quant(opts=nv.QuantOptsC(0, 0, 0, 0, 0, 1)) == nv.EINVAL
    assert _quant(x=0) == nv.EINVAL
    assert _quant(c=40, ld=40, out=_q(1, 32, 40)) == nv.ESHAPE          # K % 16 != 0
    assert _quant(axis=nv.ALONG_ROWS, r=24, out=_q(1, 64, 24)) == nv.ESHAPE
    assert _quant(r=-1) == nv.ESHAPE
    assert _quant(ld=32) == nv.ESHAPE                                     # ld < cols
    assert _quant(b=2, bs=100) == nv.ESHAPE                               # batch stride too small
    assert _quant(x=FAKE + 2) == nv.EALIGN
    assert _quant(ld=68) == nv.EALIGN                                     # 136-byte rows
    assert _quant(out=_q(1, 32, 48)) == nv.EINVAL                         # view shape mismatch
    assert _quant(out=_q(1, 32, 64, codes=0)) == nv.EINVAL
    assert _quant(out=_q(1, 32, 64, codes=FAKE + 8)) == nv.EALIGN
    assert _quant(out=_q(1, 32, 64, scales=FAKE + 2)) == nv.EALIGN
    assert _quant(ws=0) == nv.EWORKSPACE
    assert _quant(wsb=4095) == nv.EWORKSPACE
    assert _quant(ws=FAKE + 64) == nv.EALIGN
    assert nv.nvfp4_quantize(FAKE, nv.BF16, 1, 32, 64, 64, 0, 0, None, None, FAKE, 4096, None) == nv.EINVAL


def _job(x=FAKE, b=1, r=32, c=64, ld=64, bs=32 * 64, out=None):
    return nv.QuantJobC(x, b, r, c, ld, bs, out if out is not None else _q(b, r, c))


def _group(jobs, dt=nv.BF16, opts=None, ws=FAKE, wsb=16384):
    arr = (nv.QuantJobC * max(len(jobs), 1))(*jobs)
    return nv.nvfp4_quantize_group(arr, len(jobs), dt, opts or nv.QuantOptsC(0, 0, 0, 0, 0, 0), ws, wsb, None)


def test_quantize_group_argument_errors():
    assert _group([]) == nv.EINVAL                                        # no jobs
    assert _group([_job()] * 5) == nv.EINVAL                              # more than 4
    assert nv.nvfp4_quantize_group(None, 1, nv.BF16, nv.QuantOptsC(), FAKE, 16384, None) == nv.EINVAL
    assert _group([_job()], dt=3) == nv.EINVAL
    assert _group([_job()], opts=nv.QuantOptsC(2, 0, 0, 0, 0, 0)) == nv.EINVAL
    assert _group([_job(), _job(c=40, ld=40)]) == nv.ESHAPE               # second job: K % 16 != 0
    assert _group([_job(), _job(x=FAKE + 2)]) == nv.EALIGN
    assert _group([_job(out=_q(1, 32, 48))]) == nv.EINVAL                 # view shape mismatch
    assert _group([_job()], ws=0) == nv.EWORKSPACE
    assert _group([_job()], wsb=16383) == nv.EWORKSPACE                   # one-tensor size is not enough
    assert _group([_job()], ws=FAKE + 64) == nv.EALIGN


def test_gemm_argument_errors():
    a, b = _q(1, 64, 128), _q(1, 32, 128)
    assert nv.nvfp4_gemm(None, b, FAKE, nv.F32, 32, 0, 1.0, None) == nv.EINVAL
    assert nv.nvfp4_gemm(a, b, FAKE, 5, 32, 0, 1.0, None) == nv.EINVAL
    assert nv.nvfp4_gemm(a, _q(1, 32, 112), FAKE, nv.F32, 32, 0, 1.0, None) == nv.EINVAL  # K mismatch
    assert nv.nvfp4_gemm(a, _q(2, 32, 128), FAKE, nv.F32, 32, 0, 1.0, None) == nv.EINVAL  # batch mismatch
    assert nv.nvfp4_gemm(_q(1, 64, 120), _q(1, 32, 120), FAKE, nv.F32, 32, 0, 1.0, None) == nv.ESHAPE
    assert nv.nvfp4_gemm(a, b, 0, nv.F32, 32, 0, 1.0, None) == nv.EINVAL
    assert nv.nvfp4_gemm(a, b, FAKE, nv.F32, 16, 0, 1.0, None) == nv.ESHAPE                # ldc < N
    assert nv.nvfp4_gemm(a, b, FAKE + 2, nv.F32, 32, 0, 1.0, None) == nv.EALIGN
    assert nv.nvfp4_gemm(_q(1, 64, 128, st=0), b, FAKE, nv.F32, 32, 0, 1.0, None) == nv.EINVAL
    assert nv.nvfp4_gemm(_q(2, 64, 128), _q(2, 32, 128), FAKE, nv.F32, 32, 10, 1.0, None) == nv.ESHAPE
    assert nv.nvfp4_gemm(_q(70000, 1, 16), _q(70000, 1, 16), FAKE, nv.F32, 1, 1, 1.0, None) == nv.EUNSUPPORTED


def test_gemm_ex_argument_errors():
    a, b = _q(1, 64, 128), _q(1, 32, 128)
    f = nv.nvfp4_gemm_ex
    assert f(None, b, FAKE, nv.F32, 32, 0, 1.0, 0, 0, None) == nv.EINVAL
    assert f(a, b, FAKE, nv.F32, 32, 0, 1.0, -1, 192, None) == nv.EINVAL     # negative tile
    assert f(a, b, FAKE, nv.F32, 32, 0, 1.0, 0, 192, None) == nv.EINVAL      # half a request
    assert f(a, b, FAKE, nv.F32, 16, 0, 1.0, 0, 0, None) == nv.ESHAPE        # ldc < N (validated first)


def test_quantize_workspace_check_argument_errors():
    f = nv.nvfp4_quantize_workspace_check
    assert f(None, 4096, None) == nv.EWORKSPACE
    assert f(FAKE, 4095, None) == nv.EWORKSPACE
    assert f(FAKE + 64, 4096, None) == nv.EALIGN


def test_linear_view_describes_the_workspace_layout():
    """nvfp4_linear_view is host arithmetic only: the six views' shapes, and
    codes / scales / tensor-scale regions that are 256-byte aligned, in
    order, disjoint and inside the workspace."""
    M, N, K = 8192, 4096, 4096
    need = nv.nvfp4_linear_workspace_size(M, N, K)
    base = 1 << 20
    shapes = [(M, K), (N, K), (M, N), (K, N), (N, M), (K, M)]
    end = base
    for i, (r, c) in enumerate(shapes):
        q = nv.QTensorC()
        assert nv.nvfp4_linear_view(base, need, M, N, K, i, q) == nv.OK
        assert (q.batch, q.rows, q.cols) == (1, r, c)
        regions = [(q.codes, r * c // 2), (q.scales, r * c // 16), (q.tensor_scale, 4)]
        for p, n in regions:
            assert p % 256 == 0 and p >= end
            end = p + n
    assert end <= base + need
    q = nv.QTensorC()
    assert nv.nvfp4_linear_view(base, need, M, N, K, 6, q) == nv.EINVAL
    assert nv.nvfp4_linear_view(base, need - 1, M, N, K, 0, q) == nv.EWORKSPACE
    assert nv.nvfp4_linear_view(base, need, M, N, 40, 0, q) == nv.ESHAPE
    assert nv.nvfp4_linear_view(0, need, M, N, K, 0, q) == nv.EINVAL


def test_linear_argument_errors_and_workspace_size():
    M, N, K = 64, 32, 48
    need = nv.nvfp4_linear_workspace_size(M, N, K)
    views = [(M, K), (N, K), (M, N), (K, N), (N, M), (K, M)]
    assert need >= sum(r * c // 2 + r * c // 16 + 4096 for r, c in views)
    assert nv.nvfp4_linear_workspace_size(0, N, K) == 0
    cfg = nv.LinearCfgC(1, 2, 1, nv.BF16)
    f = nv.nvfp4_linear_fwd_bwd
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, None, FAKE, need, None) == nv.EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, 40, cfg, FAKE, need, None) == nv.ESHAPE
    assert f(FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, M, N, K, cfg, FAKE, need, None) == nv.EALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, cfg, FAKE, need - 1, None) == nv.EWORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, nv.LinearCfgC(1, 2, 1, 9), FAKE, need, None) == nv.EINVAL


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(nv, "_lib", None)
    monkeypatch.setattr(nv, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        nv.lib()


def test_quantize_dual_argument_errors():
    f = nv.nvfp4_quantize_dual
    o = nv.QuantOptsC(0, 0, 0, 0, 0, 0)

    def call(x=FAKE, dt=nv.BF16, b=1, r=32, c=64, ld=64, bs=32 * 64, ro=o, rq=None, co=o, cq=None, ws=FAKE, wsb=4096):
        rq = rq if rq is not None else _q(b, r, c)
        cq = cq if cq is not None else _q(b, c, r)
        return f(x, dt, b, r, c, ld, bs, ro, rq, co, cq, ws, wsb, None)

    assert call(dt=5) == nv.EINVAL
    assert call(x=0) == nv.EINVAL
    assert call(r=24, rq=_q(1, 24, 64), cq=_q(1, 64, 24)) == nv.ESHAPE     # rows % 16
    assert call(c=40, ld=40, rq=_q(1, 32, 40), cq=_q(1, 40, 32)) == nv.ESHAPE  # cols % 16
    assert call(rq=_q(1, 32, 48)) == nv.EINVAL                              # row view shape
    assert call(cq=_q(1, 48, 32)) == nv.EINVAL                              # transposed view shape
    assert call(ro=nv.QuantOptsC(0, 1, 0, 0, 0, 0)) == nv.EUNSUPPORTED     # no transform in the dual quantize
    assert call(ro=nv.QuantOptsC(3, 0, 0, 0, 0, 0)) == nv.EINVAL
    assert call(x=FAKE + 1) == nv.EALIGN                                    # BF16 needs 2-byte alignment
    assert call(ws=0) == nv.EWORKSPACE


def test_attention_ds_argument_errors_and_workspace_size():
    bh, sq, sk, d = 2, 64, 32, 16
    need = nv.nvfp4_attention_ds_workspace_size(bh, sq, sk)
    n = bh * sq * sk
    assert need >= 2 * (n // 2 + n // 16) + 4096
    assert nv.nvfp4_attention_ds_workspace_size(0, sq, sk) == 0
    cfg = nv.AttnCfgC(1, nv.SR, 0)
    qs, ks = _q(bh, d, sq), _q(bh, d, sk)
    f = nv.nvfp4_attention_ds_grads

    def call(ds=FAKE, dt=nv.BF16, q=qs, k=ks, dq=FAKE, dk=FAKE, ot=nv.BF16, b=bh, s1=sq, s2=sk, dd=d, c=cfg,
             ws=FAKE, wsb=need):
        return f(ds, dt, q, k, dq, dk, ot, b, s1, s2, dd, 0.125, c, ws, wsb, None)

    assert call(ds=0) == nv.EINVAL
    assert call(c=None) == nv.EINVAL
    assert call(c=nv.AttnCfgC(1, 7, 0)) == nv.EINVAL
    assert call(c=nv.AttnCfgC(1, nv.SR, 1)) == nv.EINVAL
    assert call(ot=4) == nv.EINVAL
    assert call(dd=24, q=_q(bh, 24, sq), k=_q(bh, 24, sk)) == nv.ESHAPE
    assert call(q=_q(bh, d, sk)) == nv.EINVAL                          # Q view over the wrong length
    assert call(dq=FAKE + 8) == nv.EALIGN
    assert call(wsb=need - 1) == nv.EWORKSPACE
    assert call(ws=FAKE + 64) == nv.EALIGN


def test_qadamw_argument_errors_and_workspace_size():
    assert nv.nvfp4_qadamw_workspace_size() == 8192
    rows, cols = 8, 64

    def state(r=rows, c=cols, means=FAKE, mq=None, vq=None):
        return nv.QAdamWStateC(mq or _q(1, r, c), vq or _q(1, r, c), means)

    L = nv.lib()

    def enc(m=FAKE, v=FAKE, r=rows, c=cols, ld=cols, st=None, ws=FAKE, wsb=8192):
        s = state() if st is None else st
        return L.nvfp4_qadamw_encode(m, v, r, c, ld, 1, 2, 0, ctypes.byref(s), ws, wsb, None)

    assert enc(m=0) == nv.EINVAL
    assert enc(c=40, ld=40, st=state(c=40)) == nv.ESHAPE
    assert enc(ld=cols - 4) == nv.ESHAPE
    assert enc(ld=cols + 2) == nv.EALIGN              # rows of 16-byte multiples
    assert enc(v=FAKE + 4) == nv.EALIGN
    assert enc(st=state(means=0)) == nv.EINVAL
    assert enc(st=state(means=FAKE + 1)) == nv.EALIGN
    assert enc(st=state(vq=_q(1, rows, 2 * cols))) == nv.EINVAL
    assert enc(st=state(mq=_q(2, rows, cols))) == nv.EINVAL
    assert enc(wsb=8191) == nv.EWORKSPACE
    assert enc(ws=FAKE + 128) == nv.EALIGN
    assert L.nvfp4_qadamw_encode(FAKE, FAKE, rows, cols, cols, 1, 2, 0, None, FAKE, 8192, None) == nv.EINVAL

    def dec(st=None, m=FAKE, v=FAKE, ld=cols):
        s = state() if st is None else st
        return L.nvfp4_qadamw_decode(ctypes.byref(s), 1, m, v, ld, None)

    assert dec(m=0) == nv.EINVAL
    assert dec(ld=cols - 16) == nv.ESHAPE
    assert dec(ld=cols + 1) == nv.EALIGN
    assert dec(v=FAKE + 8) == nv.EALIGN
    assert dec(st=state(c=24)) == nv.ESHAPE
    assert dec(st=state(vq=_q(1, rows + 1, cols))) == nv.EINVAL
    assert L.nvfp4_qadamw_decode(None, 1, FAKE, FAKE, cols, None) == nv.EINVAL


def test_gemm_axpby_argument_errors():
    a, b = _q(1, 32, 64), _q(1, 48, 64)
    L = nv.lib()

    def call(cin=FAKE, ldcin=48, bs=32 * 48, c=FAKE + 0x100000, ldc=48, dt=nv.F32):
        return L.nvfp4_gemm_axpby(ctypes.byref(a), ctypes.byref(b), c, dt, ldc, 32 * ldc, 1.0, cin, ldcin, bs,
                                  0.5, None)

    assert call(cin=0) == nv.EINVAL
    assert call(ldcin=47) == nv.ESHAPE
    assert call(cin=FAKE + 2) == nv.EALIGN
    assert call(c=FAKE, ldc=64) == nv.EINVAL            # in place needs the same row stride
    assert call(c=FAKE, dt=nv.BF16) == nv.EINVAL        # and an FP32 output
    assert call(dt=5) == nv.EINVAL


def test_ns_argument_errors_and_layout():
    m, n = 32, 48
    need = nv.nvfp4_ns_workspace_size(m, n)
    assert need > 4 * (m * n + 2 * m * m) + 3 * 4096
    assert nv.nvfp4_ns_workspace_size(24, 48) == 0 and nv.nvfp4_ns_workspace_size(0, 16) == 0
    L = nv.lib()
    co = (ctypes.c_float * 6)(1.5, -0.5, 0.0, 1.5, -0.5, 0.0)
    cfg = nv.NsCfgC(0.99, 1, 0)

    def call(g=FAKE, dt=nv.BF16, mm=m, nn=n, ldg=n, coeffs=co, steps=2, c=cfg, x=FAKE + 0x100000, ldx=n,
             ws=FAKE + 0x200000, wsb=need):
        return L.nvfp4_ns_orthogonalize(g, dt, mm, nn, ldg, coeffs, steps, ctypes.byref(c) if c else None, x, ldx,
                                        ws, wsb, None)

    assert call(g=0) == nv.EINVAL
    assert call(c=None) == nv.EINVAL
    assert call(coeffs=None) == nv.EINVAL
    assert call(steps=-1) == nv.EINVAL
    assert call(c=nv.NsCfgC(0.0, 1, 0)) == nv.EINVAL
    assert call(c=nv.NsCfgC(1.5, 1, 0)) == nv.EINVAL
    assert call(c=nv.NsCfgC(0.99, 8, 0)) == nv.EINVAL
    assert call(c=nv.NsCfgC(0.99, 1, 3)) == nv.EINVAL
    assert call(mm=24) == nv.ESHAPE
    assert call(ldg=n - 4) == nv.ESHAPE
    assert call(ldg=n + 2) == nv.EALIGN
    assert call(x=FAKE + 8) == nv.EALIGN
    assert call(wsb=need - 1) == nv.EWORKSPACE
    assert call(ws=FAKE + 0x200080) == nv.EALIGN
    st = nv.NsStateC()
    assert L.nvfp4_ns_internals(FAKE, need, m, n, ctypes.byref(st)) == nv.OK
    assert st.view[0].rows == m and st.view[0].cols == n and st.view[1].rows == n and st.view[1].cols == m
    assert st.view[2].rows == st.view[2].cols == m
    regions = [st.x_prev, st.a, st.b, st.inv_norm] + list(st.clip) + [v.codes for v in st.view]
    assert all(FAKE <= r < FAKE + need for r in regions) and len(set(regions)) == len(regions)
    assert L.nvfp4_ns_internals(FAKE, need - 1, m, n, ctypes.byref(st)) == nv.EWORKSPACE


def test_lora_argument_errors_and_layout():
    M, N, K, r = 64, 48, 128, 32
    need = nv.nvfp4_lora_workspace_size(M, K, r)
    assert need >= M * K // 2 + M * K // 16 + 2 * M * r + 4096
    assert nv.nvfp4_lora_workspace_size(M, K, 24) == 0 and nv.nvfp4_lora_workspace_size(M, K, 144) == 0
    assert nv.nvfp4_lora_workspace_size(M, 40, r) == 0
    L = nv.lib()
    w = _q(1, N, K)

    def call(x=FAKE, wq=w, l1=FAKE, l2=FAKE, mm=M, nn=N, kk=K, rr=r, beta=0.5, y=FAKE, dt=nv.BF16, ldy=N,
             ws=FAKE + 0x100000, wsb=need):
        return L.nvfp4_lora_forward(x, ctypes.byref(wq), l1, l2, mm, nn, kk, rr, beta, y, dt, ldy, ws, wsb, None)

    assert call(x=0) == nv.EINVAL
    assert call(beta=0.0) == nv.EINVAL
    assert call(beta=float("inf")) == nv.EINVAL
    assert call(dt=3) == nv.EINVAL
    assert call(rr=24) == nv.ESHAPE
    assert call(kk=40, wq=_q(1, N, 40)) == nv.ESHAPE
    assert call(wq=_q(1, N + 1, K)) == nv.EINVAL
    assert call(ldy=N - 1) == nv.ESHAPE
    assert call(l1=FAKE + 8) == nv.EALIGN
    assert call(wsb=need - 1) == nv.EWORKSPACE
    assert call(ws=FAKE + 0x100010) == nv.EALIGN
    q = nv.QTensorC()
    t = ctypes.c_void_p()
    assert L.nvfp4_lora_internals(FAKE, need, M, K, r, ctypes.byref(q), ctypes.byref(t)) == nv.OK
    assert q.rows == M and q.cols == K and FAKE < t.value < FAKE + need
