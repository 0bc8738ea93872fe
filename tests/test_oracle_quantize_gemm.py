"""Pins for the oracle's quantizer (Q0-Q9) and reference GEMM (G1-G2), no GPU.

The quantizer is compared with a brute-force numpy quantizer written here in
a different way: codes by nearest-value search with an explicit tie rule,
block scales by torch's float8_e4m3fn cast, stochastic rounding by exact
rational arithmetic.  Further pins: lossless round trips, the closed form of
the block that holds the tensor maximum, the all-zero tensor, the exact
expectation of stochastic rounding over all 2^16 random words and its
statistical unbiasedness.  The GEMM reference is compared with numpy.matmul
in float64 over values dequantized here independently."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3_rne(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _e4m3_val(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float32).numpy()


def _nearest_even(a: float) -> int:
    d = [abs(a - g) for g in GRID]
    best = min(d)
    cands = [i for i in range(8) if d[i] == best]
    even = [i for i in cands if i % 2 == 0]
    return 7 if a > 6.0 else (even[0] if even else cands[0])


def _sr_exact(a: float, u: int) -> int:
    a = min(a, 6.0)
    if a == 6.0:
        return 7
    lo = max(i for i in range(8) if GRID[i] <= a)
    fa, flo, fhi = Fraction(a), Fraction(GRID[lo]), Fraction(GRID[lo + 1])
    # the fraction (a - lo) / (hi - lo) carried to 22 bits: round up iff u / 2^16 < floor(f 2^22) / 2^22
    F = ((fa - flo) / (fhi - flo) * 2 ** 22) // 1
    return lo + (1 if 64 * u < F else 0)


def brute_quantize(v: np.ndarray, rounding=O.RNE, sr_seed=0, sr_stream=0):
    """v: float32 logical view [rows][cols] (already transformed if RHT)."""
    R, C = v.shape
    amax = np.float32(np.abs(v).max()) if v.size else np.float32(0)
    st = np.float32(amax / np.float32(2688.0))
    d6 = np.float32(np.float32(6.0) * st)
    blocks = v.reshape(R, C // 16, 16)
    ab = np.abs(blocks).max(axis=2).astype(np.float32)
    if st > 0:
        sb = np.minimum((ab / d6).astype(np.float32), np.float32(448.0))
        S = _e4m3_rne(sb)
    else:
        S = np.zeros_like(ab, dtype=np.uint8)
    eb = (_e4m3_val(S) * st).astype(np.float32)
    with np.errstate(divide="ignore"):
        rb = np.where(eb == 0, np.float32(0), (np.float32(1.0) / eb)).astype(np.float32)
    q = (blocks * rb[:, :, None]).astype(np.float32).reshape(R, C)
    codes = np.zeros((R, C), dtype=np.uint8)
    for r in range(R):
        for c in range(C):
            a = abs(float(q[r, c]))
            if rounding == O.RNE:
                mag = _nearest_even(a)
            else:
                mag = _sr_exact(a, O.sr_word(sr_seed, sr_stream, r * C + c))
            codes[r, c] = mag | (8 if np.signbit(q[r, c]) else 0)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, S, st


def _bf16(a):
    return W.bf16_bits(W.to_bf16(a))


def _adversarial(rng, R, C):
    x = (rng.standard_normal((R, C)) * 2.0 ** rng.integers(-3, 3, (R, 1))).astype(np.float32)
    x[0, :16] = 0.0                     # an all-zero block
    x[1 % R, 16:32] = 3.25              # an all-equal block
    x[R - 1, -16:] = -0.0               # negative zeros
    return x


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("axis", [O.ALONG_COLS, O.ALONG_ROWS])
@pytest.mark.parametrize("rounding", [O.RNE, O.SR])
def test_quantize_vs_brute_force(dtype, axis, rounding):
    rng = np.random.default_rng(100 + 4 * dtype + 2 * axis + rounding)
    R, C = (12, 48) if axis == O.ALONG_COLS else (48, 12)
    x32 = _adversarial(rng, R, C) if axis == O.ALONG_COLS else _adversarial(rng, C, R).T.copy()
    x = _bf16(x32) if dtype == O.BF16 else x32
    q = O.quantize(x, dtype, axis=axis, rounding=rounding, sr_seed=77, sr_stream=5)
    vals = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
            if dtype == O.BF16 else x32)
    logical = vals if axis == O.ALONG_COLS else vals.T.copy()
    codes, S, st = brute_quantize(logical.astype(np.float32), rounding, 77, 5)
    assert q.tensor_scale == st
    np.testing.assert_array_equal(q.scales[0], S)
    np.testing.assert_array_equal(q.codes[0], codes)


@pytest.mark.parametrize("rounding", [O.RNE, O.SR])
def test_quantize_with_rht_vs_brute_force(rounding):
    """The brute force takes the transformed values from the oracle's rht16,
    which the Philox/RHT tests pin separately."""
    rng = np.random.default_rng(7)
    x32 = rng.standard_normal((32, 20)).astype(np.float32)  # ALONG_ROWS: contraction = 32
    x = _bf16(x32)
    vals = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    logical = vals.T.copy()  # [20][32]
    s = O.rht_signs(0x4AD40004)
    t = np.stack([np.concatenate([O.rht16(row[16 * g:16 * g + 16], s) for g in range(2)])
                  for row in logical])
    q = O.quantize(x, O.BF16, axis=O.ALONG_ROWS, rounding=rounding, sr_seed=3, sr_stream=2,
                   rht=True, rht_seed=0x4AD40004)
    codes, S, st = brute_quantize(t.astype(np.float32), rounding, 3, 2)
    assert q.tensor_scale == st
    np.testing.assert_array_equal(q.scales[0], S)
    np.testing.assert_array_equal(q.codes[0], codes)


def test_batched_view_matches_per_batch_layout():
    rng = np.random.default_rng(9)
    x = _bf16(rng.standard_normal((3, 8, 32)).astype(np.float32))
    q = O.quantize(x, O.BF16)
    flat = O.quantize(x.reshape(24, 32), O.BF16)
    assert q.tensor_scale == flat.tensor_scale
    np.testing.assert_array_equal(q.codes.reshape(24, 16), flat.codes[0])
    np.testing.assert_array_equal(q.scales.reshape(24, 2), flat.scales[0])


def test_round_trip_of_representable_tensor():
    """A tensor built as code * dec(S) * s_t, with s_t a power of two, every
    block holding a +-6 element and one block at scale 448, quantizes back to
    exactly the same codes and scales."""
    rng = np.random.default_rng(10)
    R, C = 16, 64
    st = np.float32(2.0 ** -7)
    mags = rng.integers(0, 8, (R, C))
    signs = rng.integers(0, 2, (R, C))
    mags.reshape(R, C // 16, 16)[:, :, 0] = 7
    S = rng.integers(1, 0x7F, (R, C // 16)).astype(np.uint8)
    S[3, 2] = 0x7E
    val = np.array(GRID)[mags] * np.where(signs == 1, -1.0, 1.0)
    x = (val.reshape(R, C // 16, 16) * _e4m3_val(S)[:, :, None].astype(np.float64) * float(st))
    x = x.reshape(R, C).astype(np.float32)
    assert np.all(x.astype(np.float64) == (val.reshape(R, C // 16, 16) *
                  _e4m3_val(S)[:, :, None] * float(st)).reshape(R, C))
    q = O.quantize(x, O.F32)
    assert q.tensor_scale == st
    np.testing.assert_array_equal(q.scales[0], S)
    codes = (mags | (signs << 3)).astype(np.uint8)
    np.testing.assert_array_equal(q.codes[0], (codes[:, 0::2] | (codes[:, 1::2] << 4)))


def test_amax_block_closed_form_and_error_bound():
    x = W.fprop_3b(m=64, k=256, n=16)["X"]
    bits = W.bf16_bits(x)
    q = O.quantize(bits, O.BF16)
    v = x.float().numpy()
    r, c = np.unravel_index(np.abs(v).argmax(), v.shape)
    assert q.tensor_scale == np.float32(np.float32(np.abs(v).max()) / np.float32(2688))
    assert q.scales[0, r, c // 16] == 0x7E
    byte = q.codes[0, r, c // 2]
    assert ((byte >> (4 * (c % 2))) & 7) == 7
    # |v - dec| <= delta/2 * e_b for every unsaturated element
    deq = O.dequantize(q)[0]
    eb = (_e4m3_val(q.scales[0]) * q.tensor_scale).astype(np.float64)
    err = np.abs(deq - v).reshape(64, 16, 16)
    a = np.abs(v).reshape(64, 16, 16) / eb[:, :, None]
    half_step = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * eb[:, :, None]
    ok = (a <= 6.0 * (1 + 2.0 ** -20))
    assert np.all(err[ok] <= half_step[ok] * (1 + 2.0 ** -20))


def test_zero_tensor():
    x = np.zeros((4, 32), np.float32)
    x[1, 3] = -0.0
    q = O.quantize(x, O.F32)
    assert q.tensor_scale == 0.0
    assert not q.scales.any()
    assert q.codes[0, 1, 1] == 0x80 and q.codes.sum() == 0x80


def test_sr_exact_expectation_all_words():
    """Averaging the decoded SR result over all 65536 words gives exactly
    lo + delta * ceil(F / 64) / 2^16 with F = floor(f * 2^22), which is
    lo + delta * ceil(f * 2^16) / 2^16 wherever f has at most 22 bits (all
    a >= 1; tiny a: f * 2^22 < 1 never rounds up)."""
    for a in [0.1, 0.3, 0.74, 1.2, 1.9999, 2.3, 3.7, 4.5, 5.99, 6.0, 7.3, 1e-7, 3e-7, 0.5 + 2 ** -24]:
        a32 = float(np.float32(a))
        total = sum(Fraction(O.e2m1_decode(O.e2m1_encode_sr(a32, u))) for u in range(65536))
        am = min(Fraction(a32), Fraction(6))
        if am == 6:
            want = Fraction(6)
        else:
            lo = max(g for g in GRID if g <= am)
            hi = GRID[GRID.index(lo) + 1]
            f = (am - Fraction(lo)) / (Fraction(hi) - Fraction(lo))
            F = (f * 2 ** 22) // 1
            want = Fraction(lo) + (Fraction(hi) - Fraction(lo)) * Fraction(-(-F // 64), 65536)
            if a32 >= 1.0:
                assert want == Fraction(lo) + (Fraction(hi) - Fraction(lo)) * Fraction(-(-f * 65536 // 1), 65536)
        assert total / 65536 == want, a


def test_sr_unbiased_statistically():
    rng = np.random.default_rng(12)
    n = 200_000
    x = rng.uniform(-5.9, 5.9, (n // 16, 16)).astype(np.float32)
    x[0, 0] = 6.0 * 448 / 448  # pin the scale so q == v * (1 / e_b) stays close to v
    q = O.quantize(x, O.F32, rounding=O.SR, sr_seed=1234, sr_stream=9)
    deq = O.dequantize(q)[0]
    err = deq - x.astype(np.float64)
    # per-element variance <= (delta/2)^2 * e_b^2; mean error must vanish
    sigma = np.sqrt(np.mean((np.abs(err) + 1e-30) ** 2) / n)
    assert abs(err.mean()) < 4.0 * sigma


def _deq_independent(q: O.QTensor) -> np.ndarray:
    codes = np.empty((q.batch, q.rows, q.cols), np.uint8)
    codes[..., 0::2] = q.codes & 0xF
    codes[..., 1::2] = q.codes >> 4
    vals = np.array(GRID)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    sc = np.repeat(_e4m3_val(q.scales).astype(np.float64), 16, axis=-1)
    return vals * sc * float(q.tensor_scale)


def test_dequantize_independent():
    rng = np.random.default_rng(13)
    q = O.quantize(_bf16(rng.standard_normal((2, 5, 48)).astype(np.float32)), O.BF16)
    np.testing.assert_array_equal(O.dequantize(q), _deq_independent(q))


@pytest.mark.parametrize("M,N,K,batch", [(7, 9, 48, 1), (33, 17, 128, 2), (64, 64, 256, 1)])
def test_gemm_ref_vs_numpy(M, N, K, batch):
    rng = np.random.default_rng(M * N + K)
    a = O.quantize(_bf16(rng.standard_normal((batch, M, K)).astype(np.float32)), O.BF16)
    b = O.quantize(_bf16(rng.standard_normal((batch, N, K)).astype(np.float32) * 0.1), O.BF16)
    A, B = _deq_independent(a), _deq_independent(b)
    alpha = 0.375
    for bi in range(batch):
        y, s = O.gemm_ref(a, b, alpha, bi)
        np.testing.assert_allclose(y, alpha * (A[bi] @ B[bi].T), rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(s, alpha * (np.abs(A[bi]) @ np.abs(B[bi]).T), rtol=1e-12)
    rows = np.array([M - 1, 0, M // 2])
    y2, _ = O.gemm_ref(a, b, alpha, batch - 1, rows)
    y_all, _ = O.gemm_ref(a, b, alpha, batch - 1)
    np.testing.assert_array_equal(y2, y_all[rows])


def test_gemm_ref_identity_and_single_nonzero():
    K = 32
    eye = np.eye(K, dtype=np.float32) * 6.0
    b = O.quantize(eye, O.F32)   # every row: one element 6 -> code 7, scale 448
    rng = np.random.default_rng(14)
    a = O.quantize(rng.standard_normal((5, K)).astype(np.float32), O.F32)
    y, _ = O.gemm_ref(a, b)
    A = _deq_independent(a)[0]
    Bd = _deq_independent(b)[0]
    np.testing.assert_array_equal(np.count_nonzero(Bd, axis=1), np.ones(K))
    np.testing.assert_allclose(y, A @ Bd.T, rtol=1e-14, atol=0)
    np.testing.assert_allclose(y, A * 6.0, rtol=1e-6, atol=0)  # s_t = fl(6/2688)
    single = np.zeros((3, K), np.float32)
    single[1, 17] = -2.5
    s = O.quantize(single, O.F32)
    y, sabs = O.gemm_ref(s, s)
    d = _deq_independent(s)[0]
    assert np.count_nonzero(d) == 1 and abs(d[1, 17] + 2.5) < 2.5e-6
    want = np.zeros((3, 3))
    want[1, 1] = d[1, 17] ** 2
    np.testing.assert_allclose(y, want, rtol=1e-15)
    np.testing.assert_allclose(sabs, want, rtol=1e-15)


def test_bf16_rne_bits_vs_torch_cast():
    """The acceptance rule's BF16 rounding equals torch's round-to-nearest-even
    cast on random FP32 patterns, FP32 subnormals and values near the top."""
    import torch
    rng = np.random.default_rng(12)
    p = np.concatenate([rng.integers(0, 2 ** 32, 1 << 18, dtype=np.uint64).astype(np.uint32),
                        np.arange(1, 1 << 16, dtype=np.uint32), np.arange(0x7F7F0000, 0x7F7FFFFF, 7, dtype=np.uint32)])
    f = p.view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) < np.float32(3.38e38))
    f = f[keep]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = (O.bf16_rne_bits(f.astype(np.float64)) & 0xFFFF).astype(np.uint16)
    assert np.array_equal(got, want)


def test_gemm_accept_counts():
    y_ref = np.array([1.0, 1.0, 1.0, 1e-3], np.float64)
    sabs = np.array([1.0, 1.0, 1.0, 1e3], np.float64)
    one = np.float32(1.0)
    up1 = np.float32(1.0078125)   # one BF16 ulp above 1
    up2 = np.float32(1.015625)    # two BF16 ulps above 1
    # exact, 1 ulp, 2 ulps (fails), and a small value far off but inside 1e-5 * sabs (cancellation)
    y = np.array([one, up1, up2, np.float32(1e-3 + 9e-3)], np.float32)
    c = O.gemm_accept(y, y_ref, sabs, bf16=True)
    assert c == {"n": 4, "ok": 2, "cancel_only": 1, "fail": 1}
    c = O.gemm_accept(np.float32([1.0, 1.0 + 2e-5]), np.array([1.0, 1.0]), np.array([1.0, 1.0]), bf16=False)
    assert c == {"n": 2, "ok": 1, "cancel_only": 0, "fail": 1}
