"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same host bytes, and compare.

Acceptance (the reading used throughout):
  * quantized codes, block scales and tensor scale: bit-exact;
  * FP32 GEMM output: |y - y_ref| <= 1e-5 * sum_k |a^_ik b^_jk| (scaled);
  * BF16 GEMM output: y equals RNE_bf16(y_ref) or one of its two BF16
    neighbours, or, where cancellation makes the FP32 accumulation error
    larger than one BF16 ulp of a small y_ref, |y - y_ref| <= 1e-5 * Sabs +
    ulp_bf16(y) / 2.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

DEV = "cuda:0"
FP32_TOL = O.FP32_TOL


def host_view(x: torch.Tensor):
    """(numpy array, oracle dtype) of a CPU tensor for the oracle."""
    if x.dtype == torch.bfloat16:
        return W.bf16_bits(x), O.BF16
    return x.contiguous().numpy(), O.F32


def oracle_quant(x: torch.Tensor, axis=O.ALONG_COLS, rounding=O.RNE, sr_seed=0, sr_stream=0,
                 rht=False, rht_seed=0) -> O.QTensor:
    a, dt = host_view(x)
    return O.quantize(a, dt, axis=axis, rounding=rounding, sr_seed=sr_seed, sr_stream=sr_stream,
                      rht=rht, rht_seed=rht_seed)


def gpu_quant(x: torch.Tensor, axis=O.ALONG_COLS, rounding=O.RNE, sr_seed=0, sr_stream=0,
              rht=False, rht_seed=0, device=DEV) -> nv.QTensor:
    return nv.quantize(x.to(device), axis=axis, rounding=rounding, sr_seed=sr_seed,
                       sr_stream=sr_stream, rht=rht, rht_seed=rht_seed)


def to_oracle_view(q: nv.QTensor) -> O.QTensor:
    """Copy a device quantized view back into the oracle's container."""
    torch.cuda.synchronize()
    return O.QTensor(q.codes.cpu().numpy().reshape(q.batch, q.rows, q.cols // 2),
                     q.scales.cpu().numpy().reshape(q.batch, q.rows, q.cols // 16),
                     np.float32(q.tensor_scale.cpu().numpy()[0]), q.batch, q.rows, q.cols)


def assert_quant_equal(got: O.QTensor, want: O.QTensor, what: str = "") -> None:
    assert got.tensor_scale.view(np.uint32) == np.float32(want.tensor_scale).view(np.uint32), \
        f"{what}: tensor scale {got.tensor_scale!r} != {want.tensor_scale!r}"
    bad = np.nonzero(got.scales.reshape(-1) != want.scales.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} block scales differ, first at {bad[0]}: " \
        f"{got.scales.reshape(-1)[bad[0]]:#x} vs {want.scales.reshape(-1)[bad[0]]:#x}"
    bad = np.nonzero(got.codes.reshape(-1) != want.codes.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} code bytes differ, first at {bad[0]}: " \
        f"{got.codes.reshape(-1)[bad[0]]:#x} vs {want.codes.reshape(-1)[bad[0]]:#x}"


bf16_rne_bits = O.bf16_rne_bits


def check_gemm(y: np.ndarray, y_ref: np.ndarray, sabs: np.ndarray, bf16: bool, what: str = "") -> dict:
    """Apply the acceptance rule (oracle.gemm_accept); returns the counts,
    raises on any failure.  For BF16 outputs, elements that pass only by the
    cancellation allowance are counted as "cancel_only"."""
    c = O.gemm_accept(y, y_ref, sabs, bf16)
    if not bf16:
        if c["fail"]:
            err = np.abs(np.asarray(y, dtype=np.float64) - y_ref)
            i = int(np.argmax(err - FP32_TOL * sabs))
            raise AssertionError(f"{what}: {c['fail']} FP32 outputs outside 1e-5*sum|ab|; worst at flat index "
                                 f"{i}: err {err.reshape(-1)[i]:.3e}, bound {(FP32_TOL * sabs).reshape(-1)[i]:.3e}")
        return {"n": c["n"], "fp32_ok": c["ok"]}
    assert c["fail"] == 0, f"{what}: {c['fail']} BF16 outputs fail both criteria"
    return {"n": c["n"], "ulp_ok": c["ok"], "cancel_only": c["cancel_only"]}


def host_threads() -> int:
    """CPU threads for the oracle (the box's share: at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gemm_ref_tasks(qa: O.QTensor, qb: O.QTensor, alpha: float, tasks, mem_cap: float = 8e9):
    """O.gemm_ref over a list of (batch index, row array) tasks, each task
    split into row chunks, in threads (ctypes releases the GIL).  The number
    of threads keeps the oracle's per-call decoded copy of B (N*K doubles)
    under mem_cap bytes in total.  Returns [(y_ref, sabs)] in task order."""
    per_call = 8.0 * qb.rows * qb.cols
    nthr = max(1, min(host_threads(), int(mem_cap // max(per_call, 1.0))))
    jobs = []
    for ti, (bi, rows) in enumerate(tasks):
        rows = np.asarray(rows, dtype=np.int64)
        nchunk = max(1, min(nthr, rows.size // 16)) if len(tasks) < nthr else 1
        for part in np.array_split(rows, nchunk):
            if part.size:
                jobs.append((ti, int(bi), part))
    with ThreadPoolExecutor(nthr) as ex:
        res = list(ex.map(lambda j: O.gemm_ref(qa, qb, alpha, j[1], j[2]), jobs))
    out = []
    for ti in range(len(tasks)):
        parts = [r for j, r in zip(jobs, res) if j[0] == ti]
        out.append((np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])))
    return out


def gemm_vs_oracle(qa_gpu: nv.QTensor, qb_gpu: nv.QTensor, out_dtype=torch.bfloat16, alpha=1.0,
                   rows=None, batches=None, what: str = "", tile=None, rows_per_batch=None) -> dict:
    """Run the GPU GEMM on device views, compare selected rows of selected
    batch entries with the oracle reference computed from the same codes.
    ``rows_per_batch`` (dict batch -> rows) overrides ``rows``/``batches``."""
    y = nv.gemm(qa_gpu, qb_gpu, out_dtype=out_dtype, alpha=alpha, tile=tile)
    y3 = y if y.dim() == 3 else y.unsqueeze(0)
    qa, qb = to_oracle_view(qa_gpu), to_oracle_view(qb_gpu)
    return compare_output(y3, qa, qb, alpha, out_dtype == torch.bfloat16, what, rows=rows, batches=batches,
                          rows_per_batch=rows_per_batch)


def compare_output(y3: torch.Tensor, qa: O.QTensor, qb: O.QTensor, alpha: float, bf16: bool, what: str,
                   rows=None, batches=None, rows_per_batch=None) -> dict:
    """Check rows of a [batch][M][N] device output against the oracle."""
    if rows_per_batch is None:
        sel = np.arange(qa.rows) if rows is None else np.asarray(rows)
        rows_per_batch = {int(bi): sel for bi in (range(qa.batch) if batches is None else batches)}
    tasks = [(bi, np.asarray(r, dtype=np.int64)) for bi, r in rows_per_batch.items()]
    refs = gemm_ref_tasks(qa, qb, alpha, tasks)
    stats = {"n": 0, "rows": 0}
    for (bi, sel), (y_ref, sabs) in zip(tasks, refs):
        got = y3[bi][torch.as_tensor(sel, device=y3.device)].float().cpu().numpy()
        s = check_gemm(got, y_ref, sabs, bf16, f"{what} batch {bi}")
        for k, v in s.items():
            stats[k] = stats.get(k, 0) + v
        stats["rows"] += sel.size
    return stats
