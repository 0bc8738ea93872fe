"""Pins for the oracle's Philox4x32-10, its stochastic-rounding word mapping
and the 16-point random Hadamard transform (no GPU).

Philox is checked against rocRAND's block function (a library implementation
of the same published generator, compiled from its public header).  The
Hadamard transform is checked against scipy's Sylvester matrix in float64."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.linalg

from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not os.path.exists(hdr) or shutil.which("g++") is None:
        pytest.skip("rocRAND header or g++ not available")
    exe = str(tmp_path_factory.mktemp("philox") / "rocrand_philox_pin")
    subprocess.check_call(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           os.path.join(HERE, "rocrand_philox_pin.cpp"), "-o", exe])

    def run(tuples):
        inp = "".join(" ".join(f"{w:08x}" for w in t) + "\n" for t in tuples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [[int(w, 16) for w in line.split()] for line in out.strip().splitlines()]
    return run


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(5)
    tuples = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6, (1, 0, 0, 0, 0, 0), (0, 0, 0, 0, 1, 0),
              (0, 0, 0xFFFFFFFF, 0, 0x4AD40004, 0), (7, 0, 1, 0, 0x5EED0004, 0)]
    tuples += [tuple(int(v) for v in rng.integers(0, 2**32, 6, dtype=np.uint64)) for _ in range(200)]
    ref = rocrand_philox(tuples)
    for t, r in zip(tuples, ref):
        got = O.philox4x32_10(t[:4], t[4:])
        assert [int(v) for v in got] == r, t


def test_sr_word_uses_all_halves_of_one_block():
    """Eight consecutive elements share one Philox block; element n takes
    half (n & 1) of word (n mod 8) / 2.  The words must also be distinct across
    blocks, streams and seeds (counter injectivity)."""
    seed, stream = 0x5EED0004, 1
    for g in (0, 1, 12345, 2**33 + 7):
        blk = O.philox4x32_10([g & 0xFFFFFFFF, g >> 32, stream, 0], [seed & 0xFFFFFFFF, seed >> 32])
        halves = []
        for w in blk:
            halves += [int(w) & 0xFFFF, int(w) >> 16]
        assert [O.sr_word(seed, stream, 8 * g + j) for j in range(8)] == halves
    a = [O.sr_word(seed, 1, n) for n in range(0, 4096, 8)]
    b = [O.sr_word(seed, 2, n) for n in range(0, 4096, 8)]
    c = [O.sr_word(seed + 1, 1, n) for n in range(0, 4096, 8)]
    assert a != b and a != c


def test_sr_words_uniform_chi2():
    words = np.array([O.sr_word(99, 3, n) for n in range(1 << 16)], dtype=np.int64)
    counts = np.bincount(words >> 12, minlength=16)  # 16 bins of the top nibble
    exp = words.size / 16
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 45.0  # 15 dof; p ~ 1e-4


def test_hadamard_sylvester_orthogonality():
    H = scipy.linalg.hadamard(16)
    np.testing.assert_array_equal(H @ H.T, 16 * np.eye(16, dtype=H.dtype))


def test_rht_signs_from_philox_word0():
    for seed in (0, 0x4AD40004, 2**40 + 3):
        s = O.rht_signs(seed)
        w = int(O.philox4x32_10([0, 0, 0xFFFFFFFF, 0], [seed & 0xFFFFFFFF, seed >> 32])[0])
        want = np.array([-1.0 if (w >> j) & 1 else 1.0 for j in range(16)], dtype=np.float32)
        np.testing.assert_array_equal(s, want)


def test_rht_equals_matrix_on_exact_inputs():
    """On small integers every butterfly sum is exact in FP32, so the FWHT must
    equal (1/4) H16 diag(s) v computed in float64 bit for bit."""
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(3)
    for seed in (1, 2, 0x4AD40004):
        s = O.rht_signs(seed)
        for _ in range(50):
            v = rng.integers(-1000, 1000, 16).astype(np.float32)
            want = 0.25 * (H @ (s.astype(np.float64) * v))
            np.testing.assert_array_equal(O.rht16(v, s).astype(np.float64), want)
        for j in range(16):  # unit vectors give the columns of (1/4) H diag(s)
            e = np.zeros(16, np.float32)
            e[j] = 1.0
            np.testing.assert_array_equal(O.rht16(e, s), (0.25 * H[:, j] * s[j]).astype(np.float32))


def test_rht_random_within_fp32_bound_and_orthonormal():
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(4)
    s = O.rht_signs(0x4AD40004)
    M = 0.25 * H * s[None, :].astype(np.float64)
    np.testing.assert_allclose(M.T @ M, np.eye(16), atol=0, rtol=0)
    for _ in range(200):
        v = (rng.standard_normal(16) * 10.0 ** rng.integers(-6, 6)).astype(np.float32)
        got = O.rht16(v, s).astype(np.float64)
        want = M @ v.astype(np.float64)
        # 4 rounded butterfly stages: |err| <= 4 * 2^-24 * (1/4) * sum|v| * 4 (growth)
        bound = 4 * 2.0 ** -24 * np.abs(v.astype(np.float64)).sum()
        assert np.all(np.abs(got - want) <= bound)
        # Parseval in float64 on the exact transform
        assert np.isclose((want ** 2).sum(), (v.astype(np.float64) ** 2).sum(), rtol=1e-12)


def test_rht_cancels_in_wgrad_product():
    """Both Wgrad operands take the same transform along the contraction
    dimension, so dY^T X is unchanged: (T dY)^T (T X) = dY^T X with T
    orthonormal and block diagonal over 16-chunks of M."""
    H = scipy.linalg.hadamard(16).astype(np.float64)
    s = O.rht_signs(0x4AD40004).astype(np.float64)
    T1 = 0.25 * H * s[None, :]
    rng = np.random.default_rng(8)
    M, N, K = 64, 5, 7
    dy = rng.standard_normal((M, N))
    x = rng.standard_normal((M, K))
    T = np.kron(np.eye(M // 16), T1)
    np.testing.assert_allclose((T @ dy).T @ (T @ x), dy.T @ x, rtol=1e-12, atol=1e-12)
