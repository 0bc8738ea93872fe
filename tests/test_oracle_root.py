"""Pins for the oracle's Newton-Schulz pieces (R1-R3 and the step in NVFP4;
"Full-Stack FP4 ...", section 2.3, Q-Root), no GPU.

* R1, the clip value: numpy's percentile with the inverted-CDF method is the
  same nearest-rank order statistic; edge quantiles give the min and max;
  ties, signed zeros, and NaN sorted above every number.
* R2: numpy.clip where no NaN is involved; NaN passes through.
* R3: numpy.linalg.norm in float64.
* The step's composition: without quantization, one step maps the singular
  values s of X to a s + b s^3 + c s^5 with the same singular vectors (a
  closed form of X <- a X + (b A + c A A^T) X with A = X X^T).
* The FP32 addend of the GEMM reference: beta = 0 gives the plain product,
  alpha = 0 gives beta C exactly.
* With quantization, the chain stays near the exact one for a classic
  coefficient choice (the NVFP4 error budget of a few operands)."""
import numpy as np
import pytest

from oracle import oracle as O


@pytest.mark.parametrize("n", [1, 2, 7, 100, 1001, 4096])
@pytest.mark.parametrize("q", [1e-9, 0.25, 0.5, 0.99, 0.999, 1.0])
def test_abs_quantile_is_the_nearest_rank_statistic(n, q):
    rng = np.random.default_rng(n)
    x = (rng.standard_t(2, size=n) * np.exp(rng.uniform(-20, 20, size=n))).astype(np.float32)
    x[rng.random(n) < 0.1] = 0.0
    want = np.percentile(np.abs(x).astype(np.float64), q * 100, method="inverted_cdf")
    got = O.abs_quantile(x, q)
    assert float(got) == float(np.float32(want)), (n, q, got, want)
    if q == 1.0:
        assert got == np.abs(x).max()
    if q == 1e-9:
        assert got == np.abs(x).min()


def test_abs_quantile_ties_zeros_and_nan():
    x = np.array([-0.0, 0.0, 3, -3, 3, 1, -1, 2], np.float32)
    # sorted |x|: 0 0 1 1 2 3 3 3
    assert [float(O.abs_quantile(x, k / 8)) for k in range(1, 9)] == [0, 0, 1, 1, 2, 3, 3, 3]
    assert np.signbit(O.abs_quantile(np.array([-0.0], np.float32), 1.0)) == False  # noqa: E712  |-0| = +0
    y = np.array([1, np.nan, 2, np.inf], np.float32)
    assert O.abs_quantile(y, 0.75) == np.inf and np.isnan(O.abs_quantile(y, 1.0))
    with pytest.raises(ValueError):
        O.abs_quantile(x, 0.0)


def test_clip():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1000).astype(np.float32)
    np.testing.assert_array_equal(O.clip(x, 0.5), np.clip(x, -0.5, 0.5))
    y = O.clip(np.array([np.nan, -np.inf, np.inf, -0.0], np.float32), 1.0)
    assert np.isnan(y[0]) and y[1] == -1 and y[2] == 1 and np.signbit(y[3])


def test_frobenius_normalize():
    rng = np.random.default_rng(4)
    g = (rng.standard_normal((48, 80)) * 1e3).astype(np.float32)
    x, f = O.frobenius_normalize(g, O.F32)
    want = np.float32(1.0 / (np.linalg.norm(g.astype(np.float64)) + 1e-7))
    assert f == want
    np.testing.assert_array_equal(x, g * f)
    bits = (g.view(np.uint32) >> 16).astype(np.uint16)  # BF16 truncation, an input of its own
    xb, fb = O.frobenius_normalize(bits, O.BF16)
    gb = (bits.astype(np.uint32) << 16).view(np.float32)
    assert fb == np.float32(1.0 / (np.linalg.norm(gb.astype(np.float64)) + 1e-7))
    np.testing.assert_array_equal(xb, gb * fb)


def _with_singular_values(rng, m, n, s):
    u, _ = np.linalg.qr(rng.standard_normal((m, m)))
    v, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return u, v, (u * s) @ v.T


@pytest.mark.parametrize("coef", [(3.4445, -4.7750, 2.0315), (1.875, -1.25, 0.375), (1.5, -0.5, 0.0)])
def test_exact_step_maps_singular_values_by_the_polynomial(coef):
    rng = np.random.default_rng(5)
    m, n = 16, 48
    s = np.linspace(0.1, 1.0, m)
    u, v, x = _with_singular_values(rng, m, n, s)
    # one step through the chain (its normalization divides by ||x||_F first)
    got = O.ns_chain(x.astype(np.float32), O.F32, [coef], None, 0, quant=False).astype(np.float64)
    a, b, c = (float(np.float32(t)) for t in coef)
    s0 = s / (np.sqrt((s ** 2).sum()) + 1e-7)
    want = (u * (a * s0 + b * s0 ** 3 + c * s0 ** 5)) @ v.T
    assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max()


def test_gemm_addend_reference():
    rng = np.random.default_rng(6)
    a = O.quantize(rng.standard_normal((32, 64)).astype(np.float32), O.F32)
    b = O.quantize(rng.standard_normal((48, 64)).astype(np.float32), O.F32)
    c = rng.standard_normal((32, 48)).astype(np.float32)
    y0, s0 = O.gemm_ref(a, b, 0.75)
    y1, s1 = O.gemm_axpby_ref(a, b, 0.75, c, 0.0)
    np.testing.assert_array_equal(y0, y1)
    y2, _ = O.gemm_axpby_ref(a, b, 0.0, c, -1.5)
    np.testing.assert_array_equal(y2, -1.5 * c.astype(np.float64))
    y3, s3 = O.gemm_axpby_ref(a, b, 0.75, c, 2.0, rows=[3, 7])
    np.testing.assert_allclose(y3, y0[[3, 7]] + 2.0 * c[[3, 7]], rtol=0, atol=1e-12)


def test_quantized_chain_tracks_the_exact_one():
    rng = np.random.default_rng(7)
    g = rng.standard_normal((64, 192)).astype(np.float32)
    co = [(1.5, -0.5, 0.0)] * 8
    exact = O.ns_chain(g, O.F32, co, None, 0, quant=False)
    quant = O.ns_chain(g, O.F32, co, None, 0, quant=True)
    rel = np.linalg.norm(quant - exact) / np.linalg.norm(exact)
    assert rel < 0.2, rel
    sv = np.linalg.svd(exact.astype(np.float64), compute_uv=False)
    assert sv.min() > 0.9 and sv.max() < 1.01  # the exact chain orthogonalizes
