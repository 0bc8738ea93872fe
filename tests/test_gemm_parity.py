"""GPU parity of the block-scaled GEMM with the FP64 oracle reference over
the same quantized operands: FP32 outputs within 1e-5 * sum|a^ b^|, BF16
outputs within one BF16 ulp of the exact result (cancellation rule in
tests/parity.py).  Ragged M/N tails, K tails that are not a multiple of the
128-element K step, batching, alpha, strided output."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, gemm_vs_oracle, gpu_quant, oracle_quant, to_oracle_view

pytestmark = pytest.mark.gpu


def _pair(M, N, K, batch, seed, wide=False):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((batch, M, K)).astype(np.float32)
    b = rng.standard_normal((batch, N, K)).astype(np.float32) * np.float32(0.05)
    if wide:
        a *= (2.0 ** rng.integers(-12, 6, (batch, M, 1))).astype(np.float32)
    return torch.from_numpy(a).to(torch.bfloat16), torch.from_numpy(b).to(torch.bfloat16)


SHAPES = [(1, 1, 16, 1), (7, 9, 48, 1), (33, 17, 128, 2), (129, 130, 144, 1), (300, 257, 400, 1),
          (256, 128, 1024, 3), (64, 512, 2048, 1)]


@pytest.mark.parametrize("M,N,K,batch", SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_shapes(M, N, K, batch, out_dtype):
    a, b = _pair(M, N, K, batch, M * 1000 + N + K)
    qa, qb = gpu_quant(a), gpu_quant(b)
    assert_quant_equal(to_oracle_view(qa), oracle_quant(a), "A")
    stats = gemm_vs_oracle(qa, qb, out_dtype=out_dtype, alpha=0.75, what=f"{M}x{N}x{K}x{batch}")
    assert stats["n"] == M * N * batch


def test_gemm_wide_dynamic_range_and_zero_blocks():
    a, b = _pair(96, 80, 256, 1, 5, wide=True)
    a[0, 3, :64] = 0
    b[0, 7, 32:] = 0
    qa, qb = gpu_quant(a), gpu_quant(b)
    for dt in (torch.float32, torch.bfloat16):
        gemm_vs_oracle(qa, qb, out_dtype=dt, what="wide")


def test_gemm_k_zero_gives_zeros():
    qa = nv.QTensor.empty(1, 5, 0, DEV)
    qb = nv.QTensor.empty(1, 3, 0, DEV)
    qa.tensor_scale.fill_(1.0)
    qb.tensor_scale.fill_(1.0)
    y = nv.gemm(qa, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y.shape == (5, 3) and not y.any()


def test_gemm_strided_output():
    a, b = _pair(40, 24, 96, 2, 17)
    qa, qb = gpu_quant(a), gpu_quant(b)
    big = torch.full((2, 48, 40), 7.0, dtype=torch.float32, device=DEV)
    view = big[:, :40, :24]
    nv.gemm(qa, qb, out=view, alpha=2.0)
    want = nv.gemm(qa, qb, out_dtype=torch.float32, alpha=2.0)
    torch.cuda.synchronize()
    assert torch.equal(view, want)
    assert torch.all(big[:, :40, 24:] == 7.0) and torch.all(big[:, 40:, :] == 7.0)


def test_gemm_tiny_fp32_workload_full():
    """The 256x256 FP32 workload: A along K, B (K x N) along K via the
    transposing quantizer, every output element checked."""
    t = W.tiny()
    qa = gpu_quant(t["A"])
    qb = gpu_quant(t["B"], axis=O.ALONG_ROWS)
    assert_quant_equal(to_oracle_view(qa), oracle_quant(t["A"]), "A")
    assert_quant_equal(to_oracle_view(qb), oracle_quant(t["B"], axis=O.ALONG_ROWS), "B")
    stats = gemm_vs_oracle(qa, qb, out_dtype=torch.float32, what="tiny")
    assert stats["n"] == 256 * 256


# Shapes that send the launcher down each main loop: the tile width follows
# from filling 256 CUs in whole rounds (256 x 256 for 4000 x 4001, 256 x 192
# for 4096 x 3072, 256 x 128 for small problems), and K % 128 selects the
# global->LDS path or the register-staged one with a K tail.
LOOP_SHAPES = [(4000, 4001, 256), (4096, 3072, 384), (448, 384, 384),
               (4000, 4001, 272), (4096, 3072, 144), (448, 384, 400)]


@pytest.mark.parametrize("M,N,K", LOOP_SHAPES)
def test_gemm_every_main_loop(M, N, K):
    a, b = _pair(M, N, K, 1, 7 * M + N + K)
    qa, qb = gpu_quant(a), gpu_quant(b)
    rng = np.random.default_rng(K)
    edges = [r for t in range(0, M, 256) for r in (t, t + 127, t + 128, t + 255) if r < M]
    rows = np.unique(np.concatenate([edges, [M - 1], rng.integers(0, M, 32)]))
    for dt in (torch.float32, torch.bfloat16):
        stats = gemm_vs_oracle(qa, qb, out_dtype=dt, rows=rows, what=f"{M}x{N}x{K}")
        assert stats["n"] == rows.size * N


def test_bound_calls_repeat_the_unbound_results():
    """bind_quantize / bind_gemm marshal arguments once; repeated calls on the
    same buffers give the same bytes as the plain wrappers."""
    a, b = _pair(300, 200, 256, 1, 23)
    da, db = a.to(DEV), b.to(DEV)
    qa_ref, qb_ref = nv.quantize(da), nv.quantize(db)
    y_ref = nv.gemm(qa_ref, qb_ref, out_dtype=torch.bfloat16)
    qa, qb = nv.QTensor.empty(1, 300, 256, DEV), nv.QTensor.empty(1, 200, 256, DEV)
    wa = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), DEV)
    wb = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), DEV)
    y = torch.empty(300, 200, dtype=torch.bfloat16, device=DEV)
    calls = (nv.bind_quantize(da, qa, wa), nv.bind_quantize(db, qb, wb), nv.bind_gemm(qa, qb, y))
    for _ in range(3):
        for c in calls:
            c()
        torch.cuda.synchronize()
        assert torch.equal(qa.codes, qa_ref.codes) and torch.equal(qa.scales, qa_ref.scales)
        assert torch.equal(qb.codes, qb_ref.codes) and torch.equal(qa.tensor_scale, qa_ref.tensor_scale)
        assert torch.equal(y, y_ref)


# Forced tiles (nvfp4_gemm_ex): every kernel and tile shape on ragged
# problems.  The eight-wavefront kernel (512 x 192 and 256 x 384) keeps three
# LDS stages in flight and unrolls the K loop by three, so K steps of 1..5
# cover every remainder and the refills issued past the last step.
FORCED = [((512, 192), 520, 200, 128, 1), ((512, 192), 1000, 700, 256, 1), ((512, 192), 1030, 390, 384, 1),
          ((512, 192), 600, 800, 512, 2), ((512, 192), 700, 500, 640, 1), ((256, 384), 300, 770, 384, 1),
          ((256, 384), 520, 400, 640, 2), ((256, 256), 300, 300, 384, 1), ((256, 192), 300, 200, 256, 1),
          ((256, 128), 300, 200, 272, 1), ((256, 256), 300, 300, 272, 1), ((256, 192), 260, 200, 400, 1)]


@pytest.mark.parametrize("tile,M,N,K,batch", FORCED)
def test_gemm_forced_tiles(tile, M, N, K, batch):
    a, b = _pair(M, N, K, batch, 11 * M + N + K)
    qa, qb = gpu_quant(a), gpu_quant(b)
    for dt in (torch.float32, torch.bfloat16):
        stats = gemm_vs_oracle(qa, qb, out_dtype=dt, alpha=0.5, what=f"{tile} {M}x{N}x{K}x{batch}", tile=tile)
        assert stats["n"] == M * N * batch


@pytest.mark.parametrize("tile", [(512, 192), (256, 384)])
def test_gemm_forced_tiles_wide_range(tile):
    """Per-row magnitudes over 2^-12..2^5 give subnormal block scales, whose
    FP16 form (S * 2^-8) is an FP16 subnormal in the eight-wavefront decode."""
    a, b = _pair(640, 420, 512, 1, 29, wide=True)
    qa, qb = gpu_quant(a), gpu_quant(b)
    assert int(to_oracle_view(qa).scales.min()) < 8  # subnormal E4M3 scales present
    for dt in (torch.float32, torch.bfloat16):
        gemm_vs_oracle(qa, qb, out_dtype=dt, what=f"wide {tile}", tile=tile)


def test_gemm_tile_request_refused_where_not_applicable():
    """The eight-wavefront tiles need K % 128 == 0, and only the listed tiles
    exist: other requests are refused before any launch; the automatic
    choice (0, 0) still runs."""
    a, b = _pair(200, 100, 272, 1, 31)
    qa, qb = gpu_quant(a), gpu_quant(b)
    for tile in [(512, 192), (256, 384), (128, 128), (0, 64)]:
        with pytest.raises(nv.NVFP4Error) as e:
            nv.gemm(qa, qb, out_dtype=torch.float32, tile=tile)
        assert e.value.status in (nv.EUNSUPPORTED, nv.EINVAL)
    gemm_vs_oracle(qa, qb, out_dtype=torch.float32, what="automatic", tile=(0, 0))
