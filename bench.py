"""Benchmark of the NVFP4 quantize + block-scaled GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fprop_3b]

One step is one pass of the whole path over one batch of synthetic input:
quantize X and W (RNE, one grouped call: a single launch when both fit the
single-pass kernel), GEMM Y = X^ W^^T (BF16 out), all on one stream with the
inputs already resident in HBM.  Inputs rotate over enough
copies to exceed twice the 256 MB Infinity Cache, so every step reads its
operands from HBM.  The step time comes from the host clock around K timed
steps, bracketed by device synchronisation; per-kernel times from HIP events
recorded on the launch stream around each kernel during K further steps
(kept out of the timed region because each event adds idle time between
kernels).

Prints one JSON line.  `value` is the whole-step NVFP4 GEMM throughput
(2*M*N*K per step time, TFLOP/s); `roofline` describes the dominant kernel
(the GEMM) against the dense FP16/BF16 MFMA peak, with `traffic` the HBM
bytes per launch from the committed counter summary (null once the GEMM
source changed); `mfma_ceiling` is the sustained rate of the MFMA
instruction itself for constant, random and NVFP4-valued operands on this
GPU; `cpu_baseline` times the CPU oracle (test infrastructure) on a bounded
sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W

METRIC = "NVFP4 GEMM TFLOP/s + %MFMA peak; quantize GB/s + %HBM at 8192x3072x3072"
# (other workloads: the same line for that workload's step; `value` is its
# whole-step TFLOP/s and `roofline` its dominant call)
PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense FP16/BF16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
CACHE_BYTES = 256 << 20    # Infinity Cache
QUANT_BYTES_PER_ELEM = 2 + 0.5 + 1.0 / 16  # BF16 in, E2M1 codes + E4M3 scales out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="fprop_3b",
                   choices=["fprop_3b", "mlp_up_12b", "linear_train", "attn_scores"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-mfma-ceiling", action="store_true", help="skip the MFMA ceiling probe")
    p.add_argument("--cpu-rows", type=int, default=2048,
                   help="GEMM rows in the CPU-oracle sample (about 10 s of one core at the fprop_3b shape)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run 5 device-to-device copies of MIB MiB (calibrates HBM byte counters)")
    return p.parse_args()


def mfma_ceiling():
    """Sustained v_mfma_f32_32x32x16_f16 rate for three operand sets, from the
    probe executable built next to the library (run as a child process before
    this process touches the GPU).  The chip lowers its clock with operand
    toggling, so the NVFP4-valued set is the attainable ceiling for the GEMM's
    MFMA work; the datasheet peak assumes the top clock."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(nv.__file__)), "mfma_ceiling")
    if not os.path.exists(exe):
        return None
    try:
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=120).stdout
    except (subprocess.SubprocessError, OSError):
        return None
    res = {}
    for line in out.splitlines():
        if line.startswith("{"):
            r = json.loads(line)
            res[r["operands"]] = {"TFLOP/s": r["TFLOP/s"], "shader_MHz": r["shader_MHz"]}
    return res or None


def source_digest() -> str:
    """First 16 hex digits of the SHA-256 over the library's sources (every
    file under csrc/, in name order): counter summaries record it, and their
    figures are used only while it still matches."""
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "bit_block_scaled_nvfp4_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` (a name of the `kernels` table) from
    the committed rocprofv3 counter summary of this workload (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy of known size), or None when the library
    sources have changed since those counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_bytes = re.search(r"^%s HBM bytes per launch: (\d+)$" % re.escape(kernel), text, re.M)
    m_sha = re.search(r"^source_sha256_16: ([0-9a-f]+)$", text, re.M)
    if not (m_bytes and m_sha):
        return None
    return int(m_bytes.group(1)) if source_digest() == m_sha.group(1) else None


def copy_probe(mib: int) -> None:
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter readings
    convert the counters of the kernels above into HBM bytes."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def cpu_baseline(x_cpu: torch.Tensor, w_cpu: torch.Tensor, rows: int) -> dict:
    """The oracle as it stands, single-threaded: full quantization of X and W
    plus the FP64 reference GEMM on `rows` rows of X, extrapolated linearly in
    rows to the full step."""
    from oracle import oracle as O
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    xb, wb = W.bf16_bits(x_cpu), W.bf16_bits(w_cpu)
    t0 = time.perf_counter()
    qx = O.quantize(xb, O.BF16)
    qw = O.quantize(wb, O.BF16)
    t_quant = time.perf_counter() - t0
    sel = np.linspace(0, M - 1, rows).astype(np.int64)
    t0 = time.perf_counter()
    O.gemm_ref(qx, qw, 1.0, 0, sel)
    t_gemm = time.perf_counter() - t0
    t_step = t_quant + t_gemm * (M / rows)
    return {"value": 2.0 * M * N * K / t_step / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle quantize of all of X ({M}x{K}) and W ({N}x{K}) in {t_quant:.2f} s plus "
                      f"the FP64 reference GEMM on {rows} of {M} rows in {t_gemm:.2f} s, "
                      f"extrapolated linearly to the full step ({t_step:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    ceiling = None if (args.copy_probe or args.no_mfma_ceiling) else mfma_ceiling()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    t = W.WORKLOADS[args.workload]()
    setup = {"fprop_3b": setup_linear_gemm, "mlp_up_12b": setup_linear_gemm,
             "linear_train": setup_linear_train, "attn_scores": setup_attn}[args.workload]
    S = setup(t, dev)
    calls, nbuf, names = S["calls"], S["nbuf"], S["names"]

    def step(i, ev=None):
        for k, c in enumerate(calls[i % nbuf]):
            if ev is not None:
                ev[k].record()
            c()
        if ev is not None:
            ev[len(names)].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: exactly K steps, nothing else on the stream.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-kernel region: the same K steps again with HIP events recorded on the
    # launch stream around each call (events add a few microseconds of idle
    # between kernels, so they stay out of the timed region above).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + args.steps + i, events[i])
    torch.cuda.synchronize()
    call_ms = [float(np.mean([e[k].elapsed_time(e[k + 1]) for e in events])) for k in range(len(names))]
    ms_per_step = wall / args.steps * 1e3

    kernels = {}
    for k, name in enumerate(names):
        us = call_ms[k] * 1e3
        info = {"us": round(us, 2)}
        if name in S["flops"]:
            tf = S["flops"][name] / (us * 1e-6) / 1e12
            info.update({"TFLOP/s": round(tf, 2), "frac_mfma": round(tf / PEAK_MFMA_TFLOPS, 4)})
        if name in S["bytes"]:
            gbps = S["bytes"][name] / (us * 1e-6) / 1e9
            info.update({"GB/s": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)})
        kernels[name] = info
    dom = S["dominant"]
    dom_us = call_ms[names.index(dom)] * 1e3
    if S["bound"] == "mfma":
        achieved = S["flops"][dom] / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_MFMA_TFLOPS, 4), "traffic": measured_traffic(args.workload, dom)}
    else:
        achieved = S["bytes"][dom] / (dom_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(args.workload, dom)}
    roofline["kernel"] = dom

    out = {
        "metric": METRIC,
        "value": round(S["step_flops"] / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": dict(S["config"], workload=args.workload, rotating_buffers=nbuf),
        "roofline": roofline,
        "kernels": kernels,
        "mfma_ceiling": ceiling,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.workload == "fprop_3b":
        out["cpu_baseline"] = cpu_baseline(t["X"], t["W"], args.cpu_rows)
    print(json.dumps(out), flush=True)


def rotation(in_bytes: int) -> int:
    """Buffer sets to rotate over so a step's inputs are not in the 256 MB
    Infinity Cache from an earlier step."""
    return max(2, int(np.ceil(2 * CACHE_BYTES / in_bytes)) + 1)


def setup_linear_gemm(t, dev) -> dict:
    """One linear layer's forward: quantize X and W (RNE), Y = X W^T (BF16)."""
    x_cpu, w_cpu = t["X"], t["W"]
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    nbuf = rotation((M * K + N * K) * 2)
    xs = [x_cpu.to(dev) for _ in range(nbuf)]
    ws = [w_cpu.to(dev) for _ in range(nbuf)]
    qxs = [nv.QTensor.empty(1, M, K, dev) for _ in range(nbuf)]
    qws = [nv.QTensor.empty(1, N, K, dev) for _ in range(nbuf)]
    ys = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(nbuf)]
    wsp = nv.new_workspace(nv.nvfp4_quantize_group_workspace_size(), dev)
    # Each buffer set's calls marshalled once, so the host enqueues a step in
    # a few microseconds and stays ahead of the GPU.  X and W are quantized
    # by one grouped call (one launch when both fit the single-pass kernel).
    calls = [(nv.bind_quantize_group([xs[j], ws[j]], [qxs[j], qws[j]], wsp),
              nv.bind_gemm(qxs[j], qws[j], ys[j])) for j in range(nbuf)]
    flops = 2.0 * M * N * K
    return {"calls": calls, "nbuf": nbuf, "names": ["quantize_xw", "gemm"],
            "flops": {"gemm": flops}, "step_flops": flops,
            "bytes": {"quantize_xw": QUANT_BYTES_PER_ELEM * (M * K + N * K)},
            "dominant": "gemm", "bound": "mfma",
            "config": {"M": M, "N": N, "K": K, "x_dtype": "bf16", "y_dtype": "bf16", "rounding": "rne"}}


def setup_linear_train(t, dev) -> dict:
    """A linear layer's training step through nvfp4_linear_fwd_bwd: six
    quantizations (RNE, SR, RHT+SR) and the Fprop, Dgrad and Wgrad GEMMs."""
    x_cpu, w_cpu, dy_cpu = t["X"], t["W"], t["dY"]
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    nbuf = rotation((M * K + N * K + M * N) * 2)
    wsp = nv.new_workspace(nv.nvfp4_linear_workspace_size(M, N, K), dev)
    calls = []
    for _ in range(nbuf):
        x, w, dy = x_cpu.to(dev), w_cpu.to(dev), dy_cpu.to(dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
        dw = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        calls.append((nv.bind_linear_fwd_bwd(x, w, dy, y, dx, dw, wsp, t["sr_seed"], t["rht_seed"]),))
    flops = 3 * 2.0 * M * N * K
    return {"calls": calls, "nbuf": nbuf, "names": ["linear_fwd_bwd"], "flops": {"linear_fwd_bwd": flops},
            "step_flops": flops, "bytes": {}, "dominant": "linear_fwd_bwd", "bound": "mfma",
            "config": {"M": M, "N": N, "K": K, "x_dtype": "bf16", "y_dtype": "bf16",
                       "rounding": "rne fprop, sr dgrad, rht+sr wgrad"}}


def setup_attn(t, dev) -> dict:
    """Attention scores: quantize Q and K (RNE, one tensor scale each), then
    S = alpha Q K^T for every (batch, head), FP32 out -- bound by writing S."""
    q_cpu, k_cpu = t["Q"], t["K"]
    B, H, S_, D = q_cpu.shape
    nbuf = rotation(2 * q_cpu.numel() * 2)
    qs = [q_cpu.reshape(B * H, S_, D).to(dev) for _ in range(nbuf)]
    ks = [k_cpu.reshape(B * H, S_, D).to(dev) for _ in range(nbuf)]
    qq = [nv.QTensor.empty(B * H, S_, D, dev) for _ in range(nbuf)]
    qk = [nv.QTensor.empty(B * H, S_, D, dev) for _ in range(nbuf)]
    s_out = torch.empty(B * H, S_, S_, dtype=torch.float32, device=dev)  # 8.6 GB, written every step
    wsp_q = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), dev)
    wsp_k = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), dev)
    calls = [(nv.bind_quantize(qs[j], qq[j], wsp_q), nv.bind_quantize(ks[j], qk[j], wsp_k),
              nv.bind_gemm(qq[j], qk[j], s_out, alpha=t["alpha"])) for j in range(nbuf)]
    flops = 2.0 * B * H * S_ * S_ * D
    gemm_bytes = 4.0 * B * H * S_ * S_ + 2 * B * H * S_ * D * (0.5 + 1 / 16)
    return {"calls": calls, "nbuf": nbuf, "names": ["quantize_q", "quantize_k", "gemm"],
            "flops": {"gemm": flops}, "step_flops": flops,
            "bytes": {"quantize_q": QUANT_BYTES_PER_ELEM * q_cpu.numel(),
                      "quantize_k": QUANT_BYTES_PER_ELEM * k_cpu.numel(), "gemm": gemm_bytes},
            "dominant": "gemm", "bound": "hbm",
            "config": {"batch": B, "heads": H, "seq": S_, "head_dim": D, "x_dtype": "bf16", "y_dtype": "fp32",
                       "rounding": "rne", "alpha": t["alpha"]}}


if __name__ == "__main__":
    main()
