"""Pins for the oracle's element and scale codecs (no GPU).

Each check compares the oracle with something other than itself: the value
set the OCP MX specification lists for E2M1, torch's float8_e4m3fn casts, a
nearest-value search written here, or torch's bfloat16/float16 casts."""
import numpy as np
import pytest
import torch

from oracle import oracle as O

# OCP MX v1.0, FP4 E2M1: magnitudes of the 8 positive codes.
E2M1_OCP_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_all_16_codes():
    for code in range(16):
        want = E2M1_OCP_VALUES[code & 7] * (-1.0 if code & 8 else 1.0)
        got = O.e2m1_decode(code)
        assert got == want and np.signbit(got) == bool(code & 8), code


def _nearest_even_e2m1(q: np.ndarray) -> np.ndarray:
    """Brute force: nearest grid value in float64; on an exact tie take the
    code with mantissa bit 0.  Magnitudes above 6 saturate."""
    grid = np.array(E2M1_OCP_VALUES)
    a = np.abs(q.astype(np.float64))
    d = np.abs(a[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer an even code index
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a > 6.0, 7, pick)
    return (pick | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_rne_tie_points():
    # midpoint -> (lower code, upper code); a tie picks the even one
    ties = {0.25: (0, 1), 0.75: (1, 2), 1.25: (2, 3), 1.75: (3, 4), 2.5: (4, 5),
            3.5: (5, 6), 5.0: (6, 7)}
    for t, (lo, hi) in ties.items():
        even = lo if lo % 2 == 0 else hi
        t32 = np.float32(t)
        assert O.e2m1_encode_rne(t) == even, t
        assert O.e2m1_encode_rne(-t) == even | 8, t
        assert O.e2m1_encode_rne(float(np.nextafter(t32, np.float32(10)))) == hi
        assert O.e2m1_encode_rne(float(np.nextafter(t32, np.float32(0)))) == lo
    assert O.e2m1_encode_rne(7.0) == 7 and O.e2m1_encode_rne(1e30) == 7
    assert O.e2m1_encode_rne(-0.0) == 8 and O.e2m1_encode_rne(0.0) == 0


def test_e2m1_rne_sweep_vs_nearest_search():
    # every float32 in [0, 8) whose low 16 mantissa bits are zero (all bf16
    # patterns there), plus every tie point and its two float32 neighbours,
    # plus 200k random float32 in [-8, 8], against the brute-force search
    hi = np.arange(0, 0x4100, dtype=np.uint32) << 16
    vals = [hi.view(np.float32)]
    for t in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]:
        t32 = np.float32(t)
        vals.append(np.array([np.nextafter(t32, np.float32(0)), t32,
                              np.nextafter(t32, np.float32(10))], dtype=np.float32))
    rng = np.random.default_rng(11)
    vals.append(rng.uniform(-8, 8, 200_000).astype(np.float32))
    q = np.concatenate(vals)
    q = np.concatenate([q, -q])
    np.testing.assert_array_equal(O.e2m1_encode_rne_array(q), _nearest_even_e2m1(q))


def test_e4m3_decode_all_256_vs_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3_decode(i) for i in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert O.e4m3_decode(0x7E) == 448.0 and O.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_special_values():
    assert O.e4m3_encode(0.0) == 0
    assert O.e4m3_encode(448.0) == 0x7E
    assert O.e4m3_encode(449.0) == 0x7E and O.e4m3_encode(1e30) == 0x7E  # saturation
    assert O.e4m3_encode(2.0 ** -9) == 0x01
    assert O.e4m3_encode(2.0 ** -10) == 0x00  # tie to even (0)
    assert O.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie 1.5 -> 2
    assert O.e4m3_encode(7.5 * 2.0 ** -9) == 0x08  # largest subnormal rounds into 2^-6
    assert O.e4m3_encode(1.0625) == 0x38  # tie between 1 and 1.125 -> even (1.0)


@pytest.mark.slow
def test_e4m3_encode_exhaustive_vs_torch():
    """Every float32 bit pattern in (0, 448] encoded by the oracle equals
    torch's float8_e4m3fn round-to-nearest-even cast."""
    top = int(np.float32(448.0).view(np.uint32))
    step = 1 << 24
    for start in range(1, top + 1, step):
        u = np.arange(start, min(start + step, top + 1), dtype=np.uint32)
        y = u.view(np.float32)
        got = O.e4m3_encode_array(y)
        ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (hex(int(u[bad[0]])), got[bad[0]], ref[bad[0]])


def test_decoded_products_exact_in_bf16_and_fp16():
    """E2M1 x E4M3 (all 7 nonzero magnitudes x 126 positive finite scales) is
    exactly representable in both BF16 and FP16."""
    for s in range(1, 0x7F):
        for m in range(1, 8):
            v = O.e2m1_decode(m) * O.e4m3_decode(s)
            t = torch.tensor([v], dtype=torch.float64)
            assert t.to(torch.bfloat16).to(torch.float64).item() == v
            assert t.to(torch.float16).to(torch.float64).item() == v
