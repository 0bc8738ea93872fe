"""Pins for the oracle's AdamW state codec (S1-S4; "Full-Stack FP4 ...",
section 2.2, Q-AdamW), no GPU.

* The inverse transform against the 16-point Sylvester matrix of
  scipy.linalg.hadamard in float64: x = (1/4) D H y, rounded once.
* Lossless round trips: states whose dequantized, inverse-transformed values
  are exact in FP32 decode and re-encode to the same codes, scales, tensor
  scales and means, for the first moment under stochastic rounding and for
  the second under RNE (sqrt(fl(s^2)) = s for s >= 0, and blocks built so
  that their residuals sum to zero exactly).
* Blocks of constant sqrt(v) (the residual is zero, the mean is the value,
  the reconstruction is exact) and BF16 ties of the mean.
* The error bound that follows from the orthogonality of (1/4) D H: each
  reconstructed element is within 4 x max |quantization error| of the
  block, which is eb (RNE) or 2 eb (stochastic rounding) with eb the
  block's decode factor."""
import numpy as np
import pytest
import scipy.linalg

from oracle import oracle as O

H16 = scipy.linalg.hadamard(16).astype(np.float64)  # Sylvester order, H H = 16 I
E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
SEED_RHT = 0x4AD40007


def _code_of(q: float) -> int:
    return int(np.where(E2M1 == q)[0][0]) if q != 0 else 0


def _pack(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.uint8).reshape(*codes.shape[:-1], -1, 2)
    return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)


def _state(qvals, sbytes, st, means=None):
    """An oracle state from E2M1 values [rows][cols], scale bytes [rows][cols/16]."""
    rows, cols = qvals.shape
    codes = np.vectorize(_code_of)(qvals)
    q = O.QTensor(_pack(codes)[None], np.asarray(sbytes, np.uint8)[None], np.float32(st), 1, rows, cols)
    if means is None:
        means = np.zeros((rows, cols // 16), np.uint16)
    return q, means


def _e4m3(byte):
    return O.e4m3_decode(int(byte))


def test_inverse_transform_is_quarter_d_h():
    rng = np.random.default_rng(1)
    rows, cols = 3, 64
    qv = rng.choice(E2M1[E2M1 != 0], size=(rows, cols))
    sb = rng.integers(1, 0x7F, size=(rows, cols // 16)).astype(np.uint8)
    st = np.float32(3.7e-5)
    q, means = _state(qv, sb, st)
    st_obj = O.QAdamWState(q, q, means)
    m, v = O.qadamw_decode(st_obj, SEED_RHT)
    d = O.rht_signs(SEED_RHT).astype(np.float64)
    for r in range(rows):
        for g in range(cols // 16):
            y = qv[r, 16 * g:16 * g + 16] * _e4m3(sb[r, g]) * float(st)
            want = (0.25 * d * (H16 @ y)).astype(np.float32)
            np.testing.assert_array_equal(m[r, 16 * g:16 * g + 16], want)
            # v: mean 0 here, so v = fl(x^2)
            np.testing.assert_array_equal(v[r, 16 * g:16 * g + 16], want * want)


def test_zero_results_carry_the_diagonal_sign():
    """A block whose scale is zero (or whose sums cancel) decodes to zeros
    signed by the diagonal alone, whatever the signs of its zero codes."""
    qv = np.zeros((1, 32))
    q, means = _state(qv, [[0, 0x38]], np.float32(1.0))
    q.codes[0, 0, :8] = 0x88  # -0 codes in the first block
    q.codes[0, 0, 8:] = 0x91  # +0.5 and -0.5 in the second: (H y)_j is 0 for j != 1
    m, _ = O.qadamw_decode(O.QAdamWState(q, q, means), SEED_RHT)
    d = O.rht_signs(SEED_RHT)
    np.testing.assert_array_equal(np.signbit(m[0, :16]), d < 0)
    z = np.flatnonzero(m[0, 16:] == 0)
    assert z.size == 15
    np.testing.assert_array_equal(np.signbit(m[0, 16:][z]), d[z] < 0)


def test_inverse_undoes_the_forward_transform():
    """rht16 (the quantizer's forward transform, pinned elsewhere) of the
    decoded block gives the dequantized values back when all is exact."""
    rng = np.random.default_rng(2)
    qv = rng.choice(E2M1[E2M1 != 0], size=(1, 16))
    q, means = _state(qv, [[0x38]], np.float32(2.0 ** -10))  # scale byte 0x38 = 1.0
    m, _ = O.qadamw_decode(O.QAdamWState(q, q, means), SEED_RHT)
    back = O.rht16(m[0], O.rht_signs(SEED_RHT))
    np.testing.assert_array_equal(back, (qv[0] * 2.0 ** -10).astype(np.float32))


def _balanced_block(rng, hs):
    """E2M1 values q (max |q| = 6, no -0) with sum_k q_k (H s)_k = 0, so that
    the block's inverse transform sums to zero."""
    q = np.zeros(16)
    free = [k for k in range(16) if hs[k] == 0]
    by_val = {}
    for k in range(16):
        if hs[k] != 0:
            by_val.setdefault(abs(hs[k]), []).append(k)
    pairs = []
    for ks in by_val.values():
        for i in range(0, len(ks) - 1, 2):
            pairs.append((ks[i], ks[i + 1]))
    assert pairs, "no pair of equal |(H s)_k|"
    mags = [6.0] + list(rng.choice([0.5, 1, 1.5, 2, 3, 4, 6], size=len(pairs) - 1))
    for (k1, k2), a in zip(pairs, mags):
        q[k1] = a
        q[k2] = -a * np.sign(hs[k1]) * np.sign(hs[k2])
    for k in free:
        q[k] = rng.choice([0.5, 1, 1.5, -2, 3, -4])
    assert np.max(np.abs(q)) == 6.0 and abs(np.dot(q, hs)) == 0
    return q


@pytest.mark.parametrize("rows,cols", [(1, 16), (2, 48), (5, 128)])
def test_round_trip_is_lossless(rows, cols):
    rng = np.random.default_rng(rows * cols)
    s = O.rht_signs(SEED_RHT).astype(np.float64)
    hs = H16 @ s
    st = np.float32(2.0 ** -20)
    qm = rng.choice([-6, -4, -3, -2, -1.5, -1, -.5, .5, 1, 1.5, 2, 3, 4, 6], size=(rows, cols)).astype(np.float64)
    qm[:, ::16] = 6.0  # every block holds a 6, so its scale comes back
    qv = np.stack([np.concatenate([_balanced_block(rng, hs) for g in range(cols // 16)])
                   for _ in range(rows)])
    # scale bytes with their lowest significant bit at 1/2 or above; 0x7E = 448 in block (0, 0)
    choices = np.array([0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C, 0x50, 0x58], np.uint8)
    sm = rng.choice(choices, size=(rows, cols // 16))
    sv = rng.choice(choices, size=(rows, cols // 16))
    sm[0, 0] = sv[0, 0] = 0x7E
    mu_bits = np.full((rows, cols // 16), np.float32(2.0 ** -6).view(np.uint32) >> 16, np.uint16)
    q_m, _ = _state(qm, sm, st)
    q_v, _ = _state(qv, sv, st)
    state = O.QAdamWState(q_m, q_v, mu_bits)
    m, v = O.qadamw_decode(state, SEED_RHT)
    assert (v >= 0).all()
    again = O.qadamw_encode(m, v, SEED_RHT, sr_seed=99, sr_stream=3)
    for got, want, what in ((again.m, q_m, "m"), (again.v, q_v, "v")):
        np.testing.assert_array_equal(got.codes, want.codes, err_msg=f"{what} codes")
        np.testing.assert_array_equal(got.scales, want.scales, err_msg=f"{what} scales")
        assert got.tensor_scale == want.tensor_scale, what
    np.testing.assert_array_equal(again.v_means, mu_bits)


def test_constant_sqrt_blocks_and_mean_ties():
    # S1 alone: BF16 ties of the mean go to the even mantissa
    for c, want in ((1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82), (1.5, 0x3FC0)):
        res, mb = O.sqrt_demean16(np.full(16, np.float32(c) * np.float32(c), np.float32))
        assert mb == want, (c, hex(mb))
        mu = np.array([want << 16], np.uint32).view(np.float32)[0]
        np.testing.assert_array_equal(res, np.full(16, np.float32(c) - mu, np.float32))
    # whole codec: constant-sqrt blocks beside random ones decode exactly
    rng = np.random.default_rng(3)
    rows, cols = 4, 64
    v = (rng.standard_normal((rows, cols)).astype(np.float32) * 1e-3) ** 2
    consts = np.float32([0.75, 2.0 ** -10, 1.125, 3.0])
    for r in range(rows):
        v[r, 16:32] = consts[r] * consts[r]
    m = np.zeros((rows, cols), np.float32)
    st = O.qadamw_encode(m, v, SEED_RHT, 1)
    for r in range(rows):
        assert st.v_means[r, 1] == np.array([consts[r]], np.float32).view(np.uint32)[0] >> 16
        assert (st.v.codes[0, r, 8:16] & 0x77 == 0).all()  # +-0 (the transform of zeros keeps signs)
    m2, v2 = O.qadamw_decode(st, SEED_RHT)
    np.testing.assert_array_equal(v2[:, 16:32], v[:, 16:32])
    np.testing.assert_array_equal(m2, np.zeros_like(m2))
    assert st.m.tensor_scale == 0


def _decode_factor(q: O.QTensor):
    return np.vectorize(_e4m3)(q.scales[0]).astype(np.float64) * float(q.tensor_scale)


@pytest.mark.parametrize("seed", [4, 5])
def test_reconstruction_within_the_orthogonal_bound(seed):
    rng = np.random.default_rng(seed)
    rows, cols = 8, 256
    row_scale = np.exp(rng.uniform(-3, 3, size=(rows, 1))).astype(np.float32)
    m = (rng.standard_t(3, size=(rows, cols)) * 1e-3 * row_scale).astype(np.float32)
    v = ((rng.standard_t(3, size=(rows, cols)) * 1e-3 * row_scale) ** 2).astype(np.float32)
    st = O.qadamw_encode(m, v, SEED_RHT, 17, 2)
    m2, v2 = O.qadamw_decode(st, SEED_RHT)
    eb_m = np.repeat(_decode_factor(st.m), 16, axis=1)
    eb_v = np.repeat(_decode_factor(st.v), 16, axis=1)
    # SR: |error| < one gap <= 2 eb per transformed element; RNE: <= half a gap <= eb
    err_m = np.abs(m2.astype(np.float64) - m)
    err_s = np.abs(np.sqrt(v2.astype(np.float64)) - np.sqrt(v.astype(np.float64)))
    slack_m = 1e-6 * np.abs(m) + 1e-30
    slack_s = 1e-6 * np.sqrt(v.astype(np.float64)) + 1e-30
    assert (err_m <= 4 * 2 * eb_m + slack_m).all()
    assert (err_s <= 4 * 1 * eb_v + slack_s).all()
    # the bound is not vacuous: the errors use a fair part of it somewhere
    assert (err_s / (4 * eb_v + slack_s)).max() > 0.2


def test_empty_and_argument_errors():
    st = O.qadamw_encode(np.zeros((0, 32), np.float32), np.zeros((0, 32), np.float32), 1, 2)
    m, v = O.qadamw_decode(st, 1)
    assert m.shape == (0, 32) and v.shape == (0, 32)
    with pytest.raises(ValueError):
        O.qadamw_encode(np.zeros((2, 24), np.float32), np.zeros((2, 24), np.float32), 1, 2)
