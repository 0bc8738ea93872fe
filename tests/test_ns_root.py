"""GPU parity of Newton-Schulz with every product in NVFP4 ("Full-Stack FP4
...", section 2.3, Q-Root) and of the GEMM with an FP32 addend, against the
oracle composed step by step on the GPU's own intermediates (each product's
FP32 accumulation order decides the next quantization, so chains of two
implementations are compared one step at a time):

* the normalization factor within one FP32 ulp, X_0 = fl(G f) bit-exact;
* each clip value (the ceil(q N)-th smallest |T|) bit-exact;
* each NVFP4 view (clipped, RNE) bit-exact;
* A, B and X_{k+1} within the FP32 accumulation tolerance of the FP64
  reference plus the addend.
The run with `steps` = k checks step k; the steps are deterministic, so a
run with more steps repeats the earlier ones bit for bit."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, check_gemm, gemm_ref_tasks, to_oracle_view

pytestmark = pytest.mark.gpu


def _f32(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("m,n,k", [(16, 16, 16), (48, 80, 32), (160, 272, 96), (512, 384, 1024)])
@pytest.mark.parametrize("beta", [0.0, -1.25, 2.0])
def test_gemm_axpby_matches_oracle(m, n, k, beta):
    a = torch.from_numpy(_f32((m, k), m + k))
    b = torch.from_numpy(_f32((n, k), n + k, 2.0))
    c = torch.from_numpy(_f32((m, n), m + n, 3.0))
    qa, qb = nv.quantize(a.to(DEV)), nv.quantize(b.to(DEV))
    y = nv.gemm_axpby(qa, qb, c.to(DEV), beta, alpha=0.75)
    torch.cuda.synchronize()
    y_ref, sabs = O.gemm_axpby_ref(to_oracle_view(qa), to_oracle_view(qb), 0.75, c.numpy(), beta)
    check_gemm(y[0].cpu().numpy(), y_ref, sabs, False, f"axpby {m}x{n}x{k} beta {beta}")
    # in place on the addend
    cd = c.to(DEV).clone()
    nv.gemm_axpby(qa, qb, cd, beta, alpha=0.75, out=cd)
    yb = nv.gemm_axpby(qa, qb, c.to(DEV), beta, alpha=0.75, out_dtype=torch.bfloat16)
    # an addend row stride that is not a multiple of 4 (no 16-byte row segments)
    cw = torch.zeros(m, n + 1, device=DEV)
    cw[:, :n] = c.to(DEV)
    yw = nv.gemm_axpby(qa, qb, cw[:, :n], beta, alpha=0.75)
    torch.cuda.synchronize()
    assert torch.equal(cd.cpu(), y[0].cpu())
    assert torch.equal(yw.cpu(), y.cpu())
    check_gemm(yb[0].float().cpu().numpy(), y_ref, sabs, True, "axpby bf16")


@pytest.mark.parametrize("m,n,k", [(1024, 1024, 256), (3072, 3072, 256), (8192, 3072, 128)])
def test_gemm_axpby_every_kernel(m, n, k):
    """The addend epilogue staged through LDS in each kernel the automatic
    choice takes at these shapes (256x256, 256x192, and the 8-wavefront
    512x192): 256 seeded rows against the oracle, in place, and with an
    addend row stride that is not a multiple of 4 (the element-wise epilogue,
    the same bits)."""
    rng = np.random.default_rng(m + n + k)
    a = torch.from_numpy((rng.standard_normal((m, k)) * 2.0).astype(np.float32))
    b = torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32))
    c = torch.from_numpy((rng.standard_normal((m, n)) * 3.0).astype(np.float32))
    qa, qb = nv.quantize(a.to(DEV)), nv.quantize(b.to(DEV))
    cd = c.to(DEV)
    y = nv.gemm_axpby(qa, qb, cd, -1.25, alpha=0.75)
    yi = cd.clone()
    nv.gemm_axpby(qa, qb, yi, -1.25, alpha=0.75, out=yi)
    cw = torch.zeros(m, n + 1, device=DEV)
    cw[:, :n] = cd
    yw = nv.gemm_axpby(qa, qb, cw[:, :n], -1.25, alpha=0.75)
    torch.cuda.synchronize()
    assert torch.equal(yi, y[0]) and torch.equal(yw, y)
    rows = np.sort(rng.choice(m, 256, replace=False))
    y_ref, sabs = O.gemm_axpby_ref(to_oracle_view(qa), to_oracle_view(qb), 0.75, c.numpy(), -1.25, rows=rows)
    check_gemm(y[0].cpu().numpy()[rows], y_ref, sabs, False, f"axpby {m}x{n}x{k}")


def _oracle_rows(qa, qb, alpha, rows):
    (y, s), = gemm_ref_tasks(qa, qb, alpha, [(0, rows)])
    return y, s


def check_last_step(g, m, n, coeffs, q, mask, ws, x_out, rows=None, what=""):
    """Check the last step of a run (len(coeffs) steps) from its intermediates."""
    st = nv.ns_internals(ws, m, n)
    a, b, c = (float(np.float32(t)) for t in coeffs[-1])
    sel = np.arange(m) if rows is None else np.asarray(rows)
    xp = st["x_prev"].cpu().numpy()
    if len(coeffs) == 1:
        gh = g.cpu()
        gv = W.bf16_bits(gh) if gh.dtype == torch.bfloat16 else gh.numpy()
        x0, f = O.frobenius_normalize(gv, O.BF16 if gh.dtype == torch.bfloat16 else O.F32)
        fg = np.float32(st["inv_norm"].item())
        assert abs(int(fg.view(np.int32)) - int(f.view(np.int32))) <= 1, (fg, f)
        gf = (gv.astype(np.uint32) << 16).view(np.float32) if gh.dtype == torch.bfloat16 else gv
        np.testing.assert_array_equal(xp, gf * fg, err_msg=f"{what}: X_0")
    views = {k: to_oracle_view(v) for k, v in st["views"].items()}
    qx = q if mask & 1 else None
    want_x, px = O.ns_quantize(xp, qx)
    want_xt, _ = O.ns_quantize(np.ascontiguousarray(xp.T), qx)
    if px is not None:
        assert st["clip"][0].item() == px, f"{what}: clip X"
    assert_quant_equal(views["X"], want_x, f"{what}: X view")
    assert_quant_equal(views["X^T"], want_xt, f"{what}: X^T view")
    A = st["a"].cpu().numpy()
    y, s = _oracle_rows(views["X"], views["X"], 1.0, sel)
    check_gemm(A[sel], y, s, False, f"{what}: A")
    want_a, pa = O.ns_quantize(A, q if mask & 2 else None)
    if pa is not None:
        assert st["clip"][1].item() == pa, f"{what}: clip A"
    assert_quant_equal(views["A"], want_a, f"{what}: A view")
    B = st["b"].cpu().numpy()
    y, s = _oracle_rows(views["A"], views["A"], c, sel)
    bc = np.float32(b) * A[sel].astype(np.float64)
    check_gemm(B[sel], y + bc, s + np.abs(bc), False, f"{what}: B")
    want_b, pb = O.ns_quantize(B, q if mask & 4 else None)
    if pb is not None:
        assert st["clip"][2].item() == pb, f"{what}: clip B"
    assert_quant_equal(views["B"], want_b, f"{what}: B view")
    X = x_out.cpu().numpy()
    y, s = _oracle_rows(views["B"], views["X^T"], 1.0, sel)
    ax = np.float32(a) * xp[sel].astype(np.float64)
    check_gemm(X[sel], y + ax, s + np.abs(ax), False, f"{what}: X_next")
    return X


@pytest.mark.parametrize("m,n", [(16, 16), (32, 48), (48, 160), (128, 384), (272, 400), (384, 512), (640, 1024),
                                 (400, 272), (1024, 640)])
@pytest.mark.parametrize("mask", [0, 1, 7])
@pytest.mark.parametrize("product", [1, 2])
def test_ns_steps_match_oracle(m, n, mask, product):
    """Both launches of B^ X^ (as [m][n], and as its transpose stored
    transposed, through partial workgroup tiles at these sizes)."""
    g = torch.from_numpy(_f32((m, n), m * n + mask, 1e-2)).to(torch.bfloat16)
    coeffs = [(3.4445, -4.775, 2.0315), (1.875, -1.25, 0.375), (1.5, -0.5, 0.0)]
    ws = nv.new_workspace(nv.nvfp4_ns_workspace_size(m, n), DEV)
    gd = g.to(DEV)
    for k in range(1, 4):
        x = nv.ns_orthogonalize(gd, coeffs[:k], 0.99, mask, workspace=ws, product=product)
        torch.cuda.synchronize()
        check_last_step(g, m, n, coeffs[:k], 0.99, mask, ws, x,
                        what=f"{m}x{n} mask {mask} product {product} step {k}")


def test_ns_fp32_input_strided_output_and_zero_steps():
    m, n = 64, 96
    g = torch.from_numpy(_f32((m, n), 11, 5.0))
    out = torch.full((m, 128), 9.0, device=DEV)
    ws = nv.new_workspace(nv.nvfp4_ns_workspace_size(m, n), DEV)
    x0 = nv.ns_orthogonalize(g.to(DEV), [], out=out[:, :n], workspace=ws)
    torch.cuda.synchronize()
    want, _ = O.frobenius_normalize(g.numpy(), O.F32)
    fg = np.float32(nv.ns_internals(ws, m, n)["inv_norm"].item())
    np.testing.assert_array_equal(x0.cpu().numpy(), g.numpy() * fg)
    assert np.abs(x0.cpu().numpy() - want).max() <= 1e-6 * np.abs(want).max()
    for product in (1, 2):
        x = nv.ns_orthogonalize(g.to(DEV), [(1.5, -0.5, 0.0)], 0.5, 7, out=out[:, :n], workspace=ws, product=product)
        torch.cuda.synchronize()
        check_last_step(g, m, n, [(1.5, -0.5, 0.0)], 0.5, 7, ws, x, what=f"fp32 strided, product {product}")
        assert (out[:, n:] == 9.0).all()


def test_ns_full_size():
    """ns_3b: 3072x8192, five steps; the fifth checked on 1024 rows of every
    product and in full for every view and clip value, and the chain's
    distance from the exact FP64 iteration reported."""
    t = W.ns_3b()
    g, co, q, mask = t["G"], t["coeffs"], t["clip_quantile"], t["clip_mask"]
    m, n = g.shape
    ws = nv.new_workspace(nv.nvfp4_ns_workspace_size(m, n), DEV)
    x = nv.ns_orthogonalize(g.to(DEV), co, q, mask, workspace=ws)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(9).choice(m, 1024, replace=False))
    X = check_last_step(g, m, n, co, q, mask, ws, x, rows=rows, what="ns_3b step 5")
    sv = np.linalg.svd(X[:512].astype(np.float64), compute_uv=False)
    # The other launch of B^ X^ (automatic is the transposed one here): the
    # same products and sums, the same bits.
    x1 = nv.ns_orthogonalize(g.to(DEV), co, q, mask, product=1)
    torch.cuda.synchronize()
    assert torch.equal(x1.view(torch.int32), x.view(torch.int32))
    print(f"\nparity ns_3b: step 5 checked on {rows.size} rows; singular values of 512 rows in "
          f"[{sv.min():.3f}, {sv.max():.3f}]; both launches of B^ X^ bit-identical", flush=True)


def test_ns_ragged_large_both_launches():
    """3008x8192, one step: B^ X^ as the [8192][3008] transposed launch takes
    the 8-wavefront 512x192 tiles with a ragged last tile column, and the
    Gram products the symmetric split-K with a ragged last tile.  The step is
    checked on 256 rows against the oracle, and the direct launch must give
    the same bits."""
    m, n = 3008, 8192
    g = torch.from_numpy(_f32((m, n), 31, 1e-2)).to(torch.bfloat16)
    co = [(1.875, -1.25, 0.375)]
    ws = nv.new_workspace(nv.nvfp4_ns_workspace_size(m, n), DEV)
    x = nv.ns_orthogonalize(g.to(DEV), co, 0.99, 1, workspace=ws, product=2)
    x1 = nv.ns_orthogonalize(g.to(DEV), co, 0.99, 1, product=1)
    torch.cuda.synchronize()
    assert torch.equal(x1.view(torch.int32), x.view(torch.int32))
    rows = np.sort(np.random.default_rng(3).choice(m, 256, replace=False))
    check_last_step(g, m, n, co, 0.99, 1, ws, x, rows=rows, what="3008x8192 step 1")


def _ns_clip_value(g: torch.Tensor, q: float):
    m, n = g.shape
    ws = nv.new_workspace(nv.nvfp4_ns_workspace_size(m, n), DEV)
    nv.ns_orthogonalize(g.to(DEV), [(1.5, -0.5, 0.0)], q, 1, workspace=ws)
    torch.cuda.synchronize()
    st = nv.ns_internals(ws, m, n)
    return st["clip"][0].item(), st["x_prev"].cpu().numpy()


@pytest.mark.parametrize("q", [1e-7, 0.5, 0.99, 0.9999, 1.0])
def test_clip_value_through_the_sampled_bracket(q):
    """384 x 512 (above the size where the select samples a bracket first):
    the clip value equals the oracle's order statistic for quantiles at both
    ends (brackets open below or above) and in between."""
    rng = np.random.default_rng(int(q * 1e6))
    g = torch.from_numpy((rng.standard_t(3, size=(384, 512)) * 1e-2).astype(np.float32))
    got, x0 = _ns_clip_value(g, q)
    assert got == O.abs_quantile(x0, q), q


def test_clip_value_when_the_bracket_misses_or_overflows():
    m, n = 384, 512
    N = m * n
    # every sampled position holds 0, every other element is large: the
    # sample's bracket holds only zeros and misses the rank
    rng = np.random.default_rng(12)
    g = (rng.uniform(1.0, 2.0, size=N)).astype(np.float32)
    g[(np.arange(8192, dtype=np.int64) * N) // 8192] = 0.0
    g = torch.from_numpy(g.reshape(m, n))
    got, x0 = _ns_clip_value(g, 0.99)
    assert got == O.abs_quantile(x0, 0.99)
    # nearly constant: the bracket holds more keys than the compact buffer
    g = np.full((m, n), 0.25, np.float32)
    g[0, :7] = [1, 2, 3, 4, 5, 6, 7]
    got, x0 = _ns_clip_value(torch.from_numpy(g), 0.99)
    assert got == O.abs_quantile(x0, 0.99)


def test_clip_value_when_the_bracket_is_one_key():
    """Ties at the target: every 18th element is 1.0 (5.5%, within the compact
    buffer), the rest uniform in (0, 2), so the median falls among the ties,
    the sample brackets it with lo == hi, and the digit passes have no bits
    left to split (the value is lo itself)."""
    m, n = 384, 512
    rng = np.random.default_rng(13)
    g = rng.uniform(0.0, 2.0, size=m * n).astype(np.float32)
    g[::18] = 1.0
    got, x0 = _ns_clip_value(torch.from_numpy(g.reshape(m, n)), 0.5)
    assert got == O.abs_quantile(x0, 0.5)
    assert (np.abs(x0) == got).sum() >= m * n // 18
