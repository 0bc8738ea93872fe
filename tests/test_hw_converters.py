"""Exhaustive checks of the gfx950 conversions the library's kernels rely on,
run through the library's own device functions (tests/hw_probe.hip includes
bit_block_scaled_nvfp4_amd/csrc/device_codec.hpp) and compared with the CPU
oracle or a library routine on the host:

* E2M1 round-to-nearest-even through v_cvt_scalef32_pk_fp4_f32 at scale 1
  (every RNE code the quantizer writes): all 2^32 FP32 patterns minus NaNs,
  against the oracle's encoder (Q8a), nibble order included;
* the E4M3 block-scale encode: every non-negative FP32 pattern up to +inf,
  against the oracle's encoder (Q5);
* stochastic rounding through v_cvt_scalef32_sr_pk_fp4_f32, both of its
  lanes: every FP32 value at the two words around its rounding threshold
  (the rule is monotone in the word, so this covers every word), and 4096
  values (grid points, midpoints, saturation, signed zeros, subnormals,
  random) under all 65536 words, against the oracle (Q8b);
* the GEMM operand decode (v_cvt_scalef32_pk_f16_fp4 at scale 2^8 times the
  E4M3 byte shifted into FP16), run through nvfp4_gemm_ex itself on every
  kernel and tile: every code against every scale byte the quantizer
  produces, in every K-block position of a K step, on either operand, each
  output exactly E2M1 * E4M3 (G1);
* the GEMM epilogue's BF16 convert (v_cvt_pk_bf16_f32): all 2^32 FP32
  patterns minus NaNs, against torch's CPU round-to-nearest-even cast and,
  on a sample, the exact float64 rounding of tests/parity.py.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import oracle as O

from .parity import bf16_rne_bits

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhwprobe.so")
CHUNK = 1 << 28


def probe():
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is missing: run __graft_entry__.build()")
    L = ctypes.CDLL(PROBE)
    u32, i64, vp = ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p
    for name, args in [("hwprobe_e2m1_rne8", [u32, i64, vp, vp]), ("hwprobe_e4m3", [u32, i64, vp, vp]),
                       ("hwprobe_e2m1_sr", [vp, i64, vp, vp, vp]), ("hwprobe_sr_threshold", [u32, i64, vp, vp, vp]),
                       ("hwprobe_bf16", [u32, i64, vp, vp])]:
        getattr(L, name).argtypes = args
        getattr(L, name).restype = ctypes.c_int
    return L


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _parallel(fn, x: np.ndarray) -> np.ndarray:
    """fn over equal slices of x in threads (ctypes releases the GIL)."""
    parts = np.array_split(x, _threads())
    with ThreadPoolExecutor(len(parts)) as ex:
        return np.concatenate(list(ex.map(fn, parts)))


def _patterns(first: int, n: int) -> np.ndarray:
    return np.arange(n, dtype=np.uint32) + np.uint32(first)


def _not_nan(p: np.ndarray) -> np.ndarray:
    return (p & np.uint32(0x7FFFFFFF)) <= np.uint32(0x7F800000)


def test_e2m1_rne_converter_all_fp32_patterns():
    L = probe()
    dev = torch.empty(CHUNK // 2, dtype=torch.uint8, device="cuda:0")
    checked = 0
    for c in range((1 << 32) // CHUNK):
        first = c * CHUNK
        assert L.hwprobe_e2m1_rne8(first, CHUNK, dev.data_ptr(), _stream()) == 0
        packed = dev.cpu().numpy()
        got = np.empty(CHUNK, dtype=np.uint8)
        got[0::2] = packed & 0xF
        got[1::2] = packed >> 4
        pats = _patterns(first, CHUNK)
        want = _parallel(O.e2m1_encode_rne_array, pats.view(np.float32))
        ok = _not_nan(pats)
        bad = np.nonzero((got != want) & ok)[0]
        assert bad.size == 0, f"{bad.size} codes differ, first pattern {int(pats[bad[0]]):#010x}: " \
            f"{int(got[bad[0]]):#x} vs {int(want[bad[0]]):#x}"
        checked += int(ok.sum())
    assert checked == (1 << 32) - 2 * ((1 << 23) - 1)


def test_e4m3_block_scale_encode_all_nonnegative_patterns():
    L = probe()
    end = 0x7F800001  # every non-negative pattern up to and including +inf
    dev = torch.empty(CHUNK, dtype=torch.uint8, device="cuda:0")
    for first in range(0, end, CHUNK):
        n = min(CHUNK, end - first)
        assert L.hwprobe_e4m3(first, n, dev.data_ptr(), _stream()) == 0
        got = dev[:n].cpu().numpy()
        pats = _patterns(first, n)
        want = _parallel(O.e4m3_encode_array, pats.view(np.float32))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{bad.size} scale codes differ, first pattern {int(pats[bad[0]]):#010x}: " \
            f"{int(got[bad[0]]):#x} vs {int(want[bad[0]]):#x}"


def _sr_values() -> np.ndarray:
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    mids = (grid[:-1] + grid[1:]) / 2
    special = np.concatenate([grid, mids, np.nextafter(grid, np.float32(7)), np.nextafter(grid, np.float32(-1)),
                              np.array([6.5, 7.0, 12.0, 1e30, 1e-40, 1e-45, 2.0 ** -126, 0.25, 0.75, 5.0],
                                       np.float32)]).astype(np.float32)
    special = np.concatenate([special, -special])
    rng = np.random.default_rng(9)
    rand = (rng.uniform(0, 7, 4096 - special.size) * rng.choice([-1, 1], 4096 - special.size)).astype(np.float32)
    return np.concatenate([special, rand]).astype(np.float32)


def test_stochastic_rounding_every_word():
    L = probe()
    q = _sr_values()
    dq = torch.from_numpy(q).to("cuda:0")
    dev = torch.empty(q.size * 65536, dtype=torch.uint8, device="cuda:0")
    bad = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    assert L.hwprobe_e2m1_sr(dq.data_ptr(), q.size, dev.data_ptr(), bad.data_ptr(), _stream()) == 0
    got = dev.cpu().numpy().reshape(q.size, 65536)
    assert int(bad.item()) == 0, "the four bytes of one conversion disagree"
    want = _parallel(O.e2m1_encode_sr_all_words, q)
    for lane, g in (("low", got & 0xF), ("high", got >> 4)):
        bad_i = np.argwhere(g != want)
        assert bad_i.size == 0, f"{lane} lane: {len(bad_i)} SR codes differ, first q={q[bad_i[0][0]]!r} u={bad_i[0][1]}"


def _sr_thresholds(f: np.ndarray) -> np.ndarray:
    """U per value: the words u < U round up under the oracle's rule."""
    a = np.minimum(np.abs(f), np.float32(6.0))
    eb = (a.view(np.uint32) >> np.uint32(23)).astype(np.int32)
    e = np.maximum(eb, 127) - 127
    t = np.ldexp(a, (1 - e).astype(np.int32)).astype(np.float32)
    F = np.floor((t - np.floor(t)) * np.float32(4194304.0)).astype(np.uint32)
    return (F + np.uint32(63)) // np.uint32(64)


def _oracle_pairs(f: np.ndarray, u: np.ndarray) -> np.ndarray:
    parts = np.array_split(np.arange(f.size), _threads())
    with ThreadPoolExecutor(len(parts)) as ex:
        return np.concatenate(list(ex.map(lambda p: O.e2m1_encode_sr_pairs(f[p], u[p]), parts)))


def test_stochastic_rounding_every_fp32_value_at_its_threshold():
    L = probe()
    dev = torch.empty(CHUNK, dtype=torch.int16, device="cuda:0")
    nbad = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    for c in range((1 << 32) // CHUNK):
        first = c * CHUNK
        assert L.hwprobe_sr_threshold(first, CHUNK, dev.data_ptr(), nbad.data_ptr(), _stream()) == 0
        got = dev.cpu().numpy().view(np.uint16)
        pats = _patterns(first, CHUNK)
        ok = _not_nan(pats)
        f = pats.view(np.float32)[ok]
        g = got[ok]
        U = _sr_thresholds(f)
        u_lo = np.where(U == 0, 0, U - 1).astype(np.uint32)
        u_hi = np.minimum(U, 65535).astype(np.uint32)
        w_lo, w_hi = _oracle_pairs(f, u_lo), _oracle_pairs(f, u_hi)
        # U is the oracle's own threshold: the codes on its two sides differ wherever it is inside 1..65535
        inner = (U > 0) & (U < 65536)
        assert np.all(w_lo[inner] != w_hi[inner])
        assert np.all(w_lo[U == 0] == w_hi[U == 0])
        for k, want in ((0, w_lo), (1, w_hi)):
            byte = (g >> np.uint16(8 * k)) & np.uint16(0xFF)
            for lane, code in (("low", byte & 0xF), ("high", byte >> 4)):
                bad = np.nonzero(code != want)[0]
                assert bad.size == 0, f"{lane} lane, word {'U-1' if k == 0 else 'U'}: {bad.size} codes differ, " \
                    f"first value {f[bad[0]]!r}"
    assert int(nbad.item()) == 0, "the four bytes of one conversion disagree"


def _decode_operands(K: int):
    """A: 127 rows, row m holds codes 0..15 in K block (m % (K/16)) with E4M3
    scale byte m and zero codes elsewhere; B: 16 rows, row j holds code 2
    (the value 1.0) at offset j of every block, scale byte 0x38 (1.0).  With
    unit tensor scales, C[m][j] = E2M1(j) * E4M3(m) exactly."""
    nb = K // 16
    a_codes = np.zeros((127, K // 2), np.uint8)
    a_scales = np.zeros((127, nb), np.uint8)
    block = np.array([c | ((c + 1) << 4) for c in range(0, 16, 2)], np.uint8)  # codes 0..15, even in the low nibble
    for m in range(127):
        t = m % nb
        a_codes[m, 8 * t:8 * t + 8] = block
        a_scales[m, :] = m
    b_codes = np.zeros((16, K // 2), np.uint8)
    for j in range(16):
        for t in range(nb):
            b_codes[j, 8 * t + j // 2] = 2 << (4 * (j % 2))
    b_scales = np.full((16, nb), 0x38, np.uint8)
    return a_codes, a_scales, b_codes, b_scales


def _qtensor(codes, scales, K):
    import bit_block_scaled_nvfp4_amd as nv
    q = nv.QTensor.empty(1, codes.shape[0], K, "cuda:0")
    q.codes.copy_(torch.from_numpy(codes).view(1, codes.shape[0], K // 2))
    q.scales.copy_(torch.from_numpy(scales).view(1, codes.shape[0], K // 16))
    q.tensor_scale.fill_(1.0)
    return q


@pytest.mark.parametrize("tile,K", [((0, 0), 16), ((256, 128), 144), ((256, 128), 128), ((256, 192), 128),
                                    ((256, 256), 128), ((512, 192), 128), ((256, 384), 128),
                                    ((512, 192), 384), ((256, 256), 256)])
def test_gemm_decode_every_code_and_scale(tile, K):
    import bit_block_scaled_nvfp4_amd as nv
    ac, as_, bc, bs = _decode_operands(K)
    want = np.array([[O.e2m1_decode(j) * O.e4m3_decode(m) for j in range(16)] for m in range(127)])
    qa, qb = _qtensor(ac, as_, K), _qtensor(bc, bs, K)
    for a, b, ref in ((qa, qb, want), (qb, qa, want.T)):  # the decode of either operand
        y = nv.gemm(a, b, out_dtype=torch.float32, tile=tile)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"tile {tile} K {K}: {len(bad)} outputs differ, first {tuple(bad[0])}: " \
            f"{got[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}"


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_epilogue_convert_all_fp32_patterns():
    L = probe()
    dev = torch.empty(CHUNK, dtype=torch.int16, device="cuda:0")
    rng = np.random.default_rng(3)
    for c in range((1 << 32) // CHUNK):
        first = c * CHUNK
        assert L.hwprobe_bf16(first, CHUNK, dev.data_ptr(), _stream()) == 0
        got = dev.cpu().numpy().view(np.uint16)
        pats = _patterns(first, CHUNK)
        f = pats.view(np.float32)
        want = _torch_bf16_bits(f)
        ok = _not_nan(pats)
        bad = np.nonzero((got != want) & ok)[0]
        assert bad.size == 0, f"{bad.size} BF16 values differ, first pattern {int(pats[bad[0]]):#010x}: " \
            f"{int(got[bad[0]]):#06x} vs {int(want[bad[0]]):#06x}"
        # the float64 rounding used by the parity tests agrees on a sample of finite, in-range values
        # (FP32 subnormals included)
        idx = rng.integers(0, CHUNK, 4096)
        fin = np.isfinite(f[idx]) & (np.abs(f[idx]) < np.float32(3.38e38))
        ref = bf16_rne_bits(f[idx][fin].astype(np.float64)) & 0xFFFF
        assert np.array_equal(ref.astype(np.uint16), got[idx][fin])
