"""Benchmark of the NVFP4 quantize + block-scaled GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fprop_3b]

One step is one pass of the whole path over one batch of synthetic input:
quantize X and W (RNE, one grouped call: a single launch when both fit the
single-pass kernel), GEMM Y = X^ W^^T (BF16 out), all on one stream with the
inputs already resident in HBM.  Inputs rotate over enough copies to exceed
twice the 256 MB Infinity Cache, so every step reads its operands from HBM.

Order of work:
  1. --settle-ms of untimed steps (the shader clock ramps over the first
     tens of milliseconds of load);
  2. right after them, W untimed warm-up steps, then exactly K timed steps
     bracketed by device synchronisation, timed by the host clock;
  3. K more steps, untimed, with an event pair around every call, for each
     call's duration inside the step (`us_in_step`); then per-call timing:
     each call of the step launched alone, back to back (`reps` launches
     over the rotating buffers between two HIP events on the launch stream;
     the mean is the kernel duration plus the launch gap), and isolated (one
     launch between events after a device synchronisation), last because
     the isolated launches let the shader clock drop;
  4. the CPU oracle on the same step (the `cpu_baseline` leg), which also
     checks this run's outputs against the oracle.

Prints one JSON line.  `value` is the whole-step NVFP4 GEMM throughput
(2*M*N*K per step time, TFLOP/s; for the HBM-bound AdamW state codec, the
step's algorithmic GB/s).  `roofline` describes the dominant kernel
(the GEMM, or the attention-scores write) from its duration inside the step:
achieved = algorithmic flops (or bytes) per launch / duration, against the
dense FP16 MFMA peak (or HBM), with `traffic` the HBM bytes per launch from
the committed rocprofv3 counter summary (null once the library sources have
changed since).  `kernels` has every call's back-to-back and isolated times
and its rates, also as a fraction of the copy bandwidth measured in the same
run.  `mfma_ceiling` is the sustained rate of the MFMA instruction itself
for constant, random and NVFP4-valued operands on this GPU.  `cpu_baseline`
times the oracle (test infrastructure) on the same step over the host's
cores and reports the parity of this run's outputs against it.
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
MAX_HOST_THREADS = 16      # the CPU share of one GPU on the measurement boxes


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="fprop_3b",
                   choices=["fprop_3b", "mlp_up_12b", "linear_train", "attn_scores", "attn_bwd", "adamw_state",
                            "ns_3b", "lora_3b"])
    p.add_argument("--reps", type=int, default=100, help="back-to-back launches per call in the per-call timing")
    p.add_argument("--settle-ms", type=float, default=300.0,
                   help="wall time of untimed steps before the per-call timing (lets the shader clock settle)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-mfma-ceiling", action="store_true", help="skip the MFMA ceiling probe")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run 5 device-to-device copies of MIB MiB (calibrates HBM byte counters)")
    return p.parse_args()


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_HOST_THREADS, n))


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


def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Device-to-device copy rate in GB/s (bytes read + bytes written per
    second), the practical bandwidth the HBM-bound kernels compare with."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def time_back_to_back(calls, reps: int) -> float:
    """Mean microseconds per call of `reps` launches (cycling over the
    rotating buffer sets' `calls`) between two events on the launch stream."""
    for c in calls[:2]:
        c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        calls[i % len(calls)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def time_isolated(calls, reps: int) -> float:
    """Mean microseconds of one launch between two events, the device idle
    before each (cold clocks and caches aside from what the call reads)."""
    ts = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(ts))


def time_in_step(steps, names, nsteps: int, start: int) -> dict:
    """Mean microseconds of each call as it runs inside the step: `nsteps`
    steps in the timed region's order, an event pair recorded around every
    call on the launch stream (the events only add idle time between
    calls, never inside one)."""
    nbuf = len(steps)
    pairs = []
    for i in range(nsteps):
        row = []
        for c, name in zip(steps[(start + i) % nbuf], names):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            c()
            e1.record()
            row.append((name, e0, e1))
        pairs.append(row)
    torch.cuda.synchronize()
    acc = {}
    for row in pairs:
        for name, e0, e1 in row:
            acc.setdefault(name, []).append(e0.elapsed_time(e1) * 1e3)
    return {k: float(np.mean(v)) for k, v in acc.items()}


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
    copy_gbps = copy_bandwidth()
    t = W.WORKLOADS[args.workload]()
    setup = {"fprop_3b": setup_linear_gemm, "mlp_up_12b": setup_linear_gemm,
             "linear_train": setup_linear_train, "attn_scores": setup_attn, "attn_bwd": setup_attn_bwd,
             "adamw_state": setup_adamw, "ns_3b": setup_ns, "lora_3b": setup_lora}[args.workload]
    S = setup(t, dev)
    steps, nbuf = S["steps"], S["nbuf"]

    # 1. untimed steps until the shader clock has settled (it ramps over the
    #    first ~10-20 ms of load)
    settle_end = time.perf_counter() + args.settle_ms * 1e-3
    i = 0
    while time.perf_counter() < settle_end or i < 2 * nbuf:
        for c in steps[i % nbuf]:
            c()
        i += 1
        if i % nbuf == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    def step(i):
        for c in steps[i % nbuf]:
            c()

    # 2. warm-up and the timed region right after, while the clock is up:
    #    exactly K steps, nothing else on the stream
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # 3. the same steps once more (untimed), each call between two events:
    #     the duration of every call inside the step, the dominant one's
    #     roofline figure (a profiler's per-kernel mean over a run is this)
    names = []
    for c in steps[0]:
        names.append(next(n for n, cs in S["calls"].items() if cs[0] is c))
    in_step = time_in_step(steps, names, args.steps, args.warmup + args.steps)

    # 3b. per-call timing, last (the isolated launches let the clock drop):
    #     each call of the step back to back, and isolated
    kernels = {}
    for name, calls in S["calls"].items():
        b2b = time_back_to_back(calls, args.reps)
        iso = time_isolated(calls, max(5, args.reps // 5))
        info = {"us": round(b2b, 2), "us_isolated": round(iso, 2)}
        if name in S["flops"]:
            tf = S["flops"][name] / (b2b * 1e-6) / 1e12
            info.update({"TFLOP/s": round(tf, 2), "frac_mfma": round(tf / PEAK_MFMA_TFLOPS, 4)})
        if name in S["bytes"]:
            gbps = S["bytes"][name] / (b2b * 1e-6) / 1e9
            info.update({"GB/s": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)})
            if copy_gbps:
                info["frac_copy"] = round(gbps / copy_gbps, 4)
        kernels[name] = info

    for n, us in in_step.items():
        kernels[n]["us_in_step"] = round(us, 2)

    dom = S["dominant"]
    dom_us = in_step.get(dom, kernels[dom]["us"])
    if S["bound"] == "mfma":
        achieved = S["flops"][dom] / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_MFMA_TFLOPS, 4), "traffic": measured_traffic(args.workload, dom)}
    else:
        achieved = S["bytes"][dom] / (dom_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(args.workload, dom)}
    roofline["kernel"] = dom
    roofline["duration_us"] = dom_us

    if "step_bytes" in S:  # an HBM-bound step: its rate in GB/s
        value, unit = round(S["step_bytes"] / (ms_per_step * 1e-3) / 1e9, 1), "GB/s"
    else:
        value, unit = round(S["step_flops"] / (ms_per_step * 1e-3) / 1e12, 2), "TFLOP/s"
    out = {
        "metric": S.get("metric", METRIC),
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": S.get("dtype", "fp16"),
        "data": "synthetic",
        "config": dict(S["config"], workload=args.workload, rotating_buffers=nbuf),
        "roofline": roofline,
        "kernels": kernels,
        "copy_GB/s": round(copy_gbps, 1) if copy_gbps else None,
        "mfma_ceiling": ceiling,
        "cpu_baseline": None,
    }
    # 4. the oracle on the same step, and this run's outputs against it
    if not args.no_cpu_baseline and "baseline" in S:
        out["cpu_baseline"] = S["baseline"]()
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
    wsx = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), dev)
    wsw = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), dev)
    # Each buffer set's calls marshalled once, so the host enqueues a step in
    # a few microseconds and stays ahead of the GPU.  X and W are quantized
    # by one grouped call (one launch when both fit the single-pass kernel).
    qxw = [nv.bind_quantize_group([xs[j], ws[j]], [qxs[j], qws[j]], wsp) for j in range(nbuf)]
    gem = [nv.bind_gemm(qxs[j], qws[j], ys[j]) for j in range(nbuf)]
    calls = {"quantize_xw": qxw,
             "quantize_x": [nv.bind_quantize(xs[j], qxs[j], wsx) for j in range(nbuf)],
             "quantize_w": [nv.bind_quantize(ws[j], qws[j], wsw) for j in range(nbuf)],
             "gemm": gem}
    flops = 2.0 * M * N * K

    def baseline():
        # the step's results on buffer set 0 come from a fresh call, then the oracle
        qxw[0]()
        gem[0]()
        torch.cuda.synchronize()
        return cpu_baseline_linear(x_cpu, w_cpu, qxs[0], qws[0], ys[0])

    return {"steps": list(zip(qxw, gem)), "calls": calls, "nbuf": nbuf,
            "flops": {"gemm": flops}, "step_flops": flops,
            "bytes": {"quantize_xw": QUANT_BYTES_PER_ELEM * (M * K + N * K),
                      "quantize_x": QUANT_BYTES_PER_ELEM * M * K, "quantize_w": QUANT_BYTES_PER_ELEM * N * K},
            "dominant": "gemm", "bound": "mfma", "baseline": baseline,
            "metric": METRIC if (M, N, K) == (8192, 3072, 3072) else
            f"NVFP4 GEMM TFLOP/s + %MFMA peak; quantize GB/s + %HBM at {M}x{N}x{K}",
            "config": {"M": M, "N": N, "K": K, "x_dtype": "bf16", "y_dtype": "bf16", "rounding": "rne"}}


def cpu_baseline_linear(x_cpu, w_cpu, qx, qw, y) -> dict:
    """The oracle as it stands on the whole step: quantize X and W (one host
    thread each, as the oracle quantizes a tensor in one call), then the FP64
    reference GEMM of every output row, split over the host's threads; also
    the one-core time of the two quantizations.  The GPU's quantized views
    and output from this run are checked against it (codes, scales and tensor
    scales bit for bit; Y by the G3 rule)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as O
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    nthr = host_threads()
    xb, wb = W.bf16_bits(x_cpu), W.bf16_bits(w_cpu)
    t0 = time.perf_counter()
    O.quantize(xb, O.BF16)
    O.quantize(wb, O.BF16)
    t_quant_1core = time.perf_counter() - t0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nthr) as ex:
        fx, fw = ex.submit(O.quantize, xb, O.BF16), ex.submit(O.quantize, wb, O.BF16)
        ox, ow = fx.result(), fw.result()
        t_quant = time.perf_counter() - t0
        chunks = np.array_split(np.arange(M, dtype=np.int64), nthr)
        t1 = time.perf_counter()
        parts = list(ex.map(lambda r: O.gemm_ref(ox, ow, 1.0, 0, r), chunks))
        t_gemm = time.perf_counter() - t1
    t_step = time.perf_counter() - t0
    y_ref = np.concatenate([p[0] for p in parts])
    sabs = np.concatenate([p[1] for p in parts])

    def same(q, o):
        return bool(np.array_equal(q.codes.cpu().numpy().reshape(-1), o.codes.reshape(-1)) and
                    np.array_equal(q.scales.cpu().numpy().reshape(-1), o.scales.reshape(-1)) and
                    np.float32(q.tensor_scale.item()).view(np.uint32) == np.float32(o.tensor_scale).view(np.uint32))

    acc = O.gemm_accept(y.float().cpu().numpy(), y_ref, sabs, bf16=True)
    return {"value": 2.0 * M * N * K / t_step / 1e12, "unit": "TFLOP/s", "cores": nthr, "kind": "oracle",
            "sample": f"the whole step on {nthr} host threads: oracle quantize of X ({M}x{K}) and W ({N}x{K}) "
                      f"in {t_quant:.2f} s (one thread per tensor; {t_quant_1core:.2f} s on one core), FP64 "
                      f"reference GEMM of all {M} rows in {t_gemm:.2f} s",
            "seconds": round(t_step, 3), "quantize_seconds_1core": round(t_quant_1core, 3),
            "parity": {"x_view_bit_exact": same(qx, ox), "w_view_bit_exact": same(qw, ow),
                       "y_rows": M, "y_ulp_ok": acc["ok"], "y_cancel_only": acc["cancel_only"],
                       "y_fail": acc["fail"]}}


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
        calls.append(nv.bind_linear_fwd_bwd(x, w, dy, y, dx, dw, wsp, t["sr_seed"], t["rht_seed"]))
    flops = 3 * 2.0 * M * N * K
    return {"steps": [(c,) for c in calls], "calls": {"linear_fwd_bwd": calls}, "nbuf": nbuf,
            "flops": {"linear_fwd_bwd": flops}, "step_flops": flops, "bytes": {},
            "dominant": "linear_fwd_bwd", "bound": "mfma",
            "metric": f"NVFP4 linear training step (Fprop + Dgrad + Wgrad) TFLOP/s at M={M} N={N} K={K}",
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
    cq = [nv.bind_quantize(qs[j], qq[j], wsp_q) for j in range(nbuf)]
    ck = [nv.bind_quantize(ks[j], qk[j], wsp_k) for j in range(nbuf)]
    cg = [nv.bind_gemm(qq[j], qk[j], s_out, alpha=t["alpha"]) for j in range(nbuf)]
    flops = 2.0 * B * H * S_ * S_ * D
    gemm_bytes = 4.0 * B * H * S_ * S_ + 2 * B * H * S_ * D * (0.5 + 1 / 16)
    return {"steps": list(zip(cq, ck, cg)), "calls": {"quantize_q": cq, "quantize_k": ck, "gemm": cg},
            "nbuf": nbuf, "flops": {"gemm": flops}, "step_flops": flops,
            "bytes": {"quantize_q": QUANT_BYTES_PER_ELEM * q_cpu.numel(),
                      "quantize_k": QUANT_BYTES_PER_ELEM * k_cpu.numel(), "gemm": gemm_bytes},
            "dominant": "gemm", "bound": "hbm",
            "metric": f"NVFP4 attention scores QK^T TFLOP/s + %HBM of the FP32 scores at {B}x{H}x{S_}x{S_}x{D}",
            "config": {"batch": B, "heads": H, "seq": S_, "head_dim": D, "x_dtype": "bf16", "y_dtype": "fp32",
                       "rounding": "rne", "alpha": t["alpha"]}}


def setup_attn_bwd(t, dev) -> dict:
    """Attention backward through dS in NVFP4: the forward's dual views of Q
    and K (one read each), then nvfp4_attention_ds_grads (dS quantized in
    both orientations from one read, dQ = alpha dS K, dK = alpha dS^T Q)."""
    q_cpu, k_cpu, ds_cpu = t["Q"], t["K"], t["dS"]
    bh, sq, d = q_cpu.shape
    sk = k_cpu.shape[1]
    q, k, ds = q_cpu.to(dev), k_cpu.to(dev), ds_cpu.to(dev)
    q_hd, q_seq = nv.QTensor.empty(bh, sq, d, dev), nv.QTensor.empty(bh, d, sq, dev)
    k_hd, k_seq = nv.QTensor.empty(bh, sk, d, dev), nv.QTensor.empty(bh, d, sk, dev)
    wq = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), dev)
    wk = nv.new_workspace(nv.nvfp4_quantize_workspace_size(), dev)
    wds = nv.new_workspace(nv.nvfp4_attention_ds_workspace_size(bh, sq, sk), dev)
    dq = torch.empty(bh, sq, d, dtype=torch.bfloat16, device=dev)
    dk = torch.empty(bh, sk, d, dtype=torch.bfloat16, device=dev)
    cq = nv.bind_quantize_dual(q, (q_hd, q_seq), wq)
    ck = nv.bind_quantize_dual(k, (k_hd, k_seq), wk)
    cg = nv.bind_attention_ds_grads(ds, q_seq, k_seq, dq, dk, wds, t["alpha"], t["sr_seed"])
    flops = 2 * 2.0 * bh * sq * sk * d
    ds_bytes = 2.0 * bh * sq * sk + 2 * bh * sq * sk * (0.5 + 1 / 16) + 2 * bh * (sq + sk) * d * (0.5 + 1 / 16)
    return {"steps": [(cq, ck, cg)], "calls": {"quantize_dual_q": [cq], "quantize_dual_k": [ck],
                                               "attention_ds_grads": [cg]}, "nbuf": 1,
            "flops": {"attention_ds_grads": flops}, "step_flops": flops,
            "bytes": {"quantize_dual_q": (2 + 2 * (0.5 + 1 / 16)) * q.numel(),
                      "quantize_dual_k": (2 + 2 * (0.5 + 1 / 16)) * k.numel(), "attention_ds_grads": ds_bytes},
            "dominant": "attention_ds_grads", "bound": "hbm",
            "metric": "attention dS backward (dS dual quantize + dQ, dK GEMMs) TFLOP/s at 128x4096x4096x128",
            "config": {"batch_heads": bh, "seq_q": sq, "seq_k": sk, "head_dim": d, "ds_rounding": "sr",
                       "out_dtype": "bf16"}}


def setup_adamw(t, dev) -> dict:
    """AdamW state codec: encode FP32 m, v into NVFP4 state, then decode."""
    m_cpu, v_cpu = t["m"], t["v"]
    R, C = m_cpu.shape
    nbuf = rotation(8 * m_cpu.numel())
    ms = [m_cpu.to(dev) for _ in range(nbuf)]
    vs = [v_cpu.to(dev) for _ in range(nbuf)]
    sts = [nv.QAdamWState.empty(R, C, dev) for _ in range(nbuf)]
    ws = nv.new_workspace(nv.nvfp4_qadamw_workspace_size(), dev)
    om, ov = torch.empty(R, C, device=dev), torch.empty(R, C, device=dev)
    enc = [nv.bind_qadamw_encode(ms[j], vs[j], sts[j], ws, t["rht_seed"], t["sr_seed"]) for j in range(nbuf)]
    dec = [nv.bind_qadamw_decode(sts[j], t["rht_seed"], om, ov) for j in range(nbuf)]
    n = R * C
    b = n * (8 + 2 * (0.5 + 1 / 16) + 2 / 16)  # FP32 m, v <-> two NVFP4 views and the BF16 means
    return {"steps": list(zip(enc, dec)), "calls": {"qadamw_encode": enc, "qadamw_decode": dec}, "nbuf": nbuf,
            "flops": {}, "step_flops": 0.0, "bytes": {"qadamw_encode": b, "qadamw_decode": b}, "step_bytes": 2 * b,
            "dominant": "qadamw_encode", "bound": "hbm", "dtype": "f32",
            "metric": "AdamW state codec GB/s (encode + decode) at 20480x5120",
            "config": {"rows": R, "cols": C, "m": "rht+sr", "v": "sqrt, bf16 block mean, rht, rne"}}


def setup_ns(t, dev) -> dict:
    """Newton-Schulz orthogonalization with every product in NVFP4."""
    g_cpu = t["G"]
    m, n = g_cpu.shape
    co = t["coeffs"]
    g = g_cpu.to(dev)
    ws = nv.new_workspace(nv.nvfp4_ns_workspace_size(m, n), dev)
    x = torch.empty(m, n, device=dev)
    c = nv.bind_ns_orthogonalize(g, co, x, ws, t["clip_quantile"], t["clip_mask"])
    flops = len(co) * 2.0 * (m * m * n + m * m * m + m * n * m)
    return {"steps": [(c,)], "calls": {"ns_orthogonalize": [c]}, "nbuf": 1, "flops": {"ns_orthogonalize": flops},
            "step_flops": flops, "bytes": {}, "dominant": "ns_orthogonalize", "bound": "mfma",
            "metric": "Newton-Schulz in NVFP4 TFLOP/s (5 steps) at 3072x8192",
            "config": {"m": m, "n": n, "steps": len(co), "coeffs": list(co[0]), "clip_quantile": t["clip_quantile"],
                       "clip_mask": t["clip_mask"]}}


def setup_lora(t, dev) -> dict:
    """LoRA-style forward: quantize X, T = BF16(X L1^T), Y = X^ W_res^^T +
    beta T L2^T with the low-rank term folded into the NVFP4 GEMM."""
    x_cpu, w_cpu, l1_cpu, l2_cpu = t["X"], t["W_res"], t["L1"], t["L2"]
    M, K = x_cpu.shape
    N, r = w_cpu.shape[0], l1_cpu.shape[0]
    nbuf = rotation(x_cpu.numel() * 2)
    xs = [x_cpu.to(dev) for _ in range(nbuf)]
    wv = nv.quantize(w_cpu.to(dev))
    l1, l2 = l1_cpu.to(dev), l2_cpu.to(dev)
    ws = nv.new_workspace(nv.nvfp4_lora_workspace_size(M, K, r), dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    calls = [nv.bind_lora_forward(xs[j], wv, l1, l2, t["beta"], y, ws) for j in range(nbuf)]
    flops = 2.0 * M * N * K + 2.0 * M * K * r + 2.0 * M * N * r
    return {"steps": [(c,) for c in calls], "calls": {"lora_forward": calls}, "nbuf": nbuf,
            "flops": {"lora_forward": flops}, "step_flops": flops, "bytes": {}, "dominant": "lora_forward",
            "bound": "mfma", "metric": "LoRA-style forward TFLOP/s (NVFP4 residual + BF16 rank-64) at 8192x3072x3072",
            "config": {"M": M, "N": N, "K": K, "rank": r, "beta": t["beta"], "y_dtype": "bf16"}}


if __name__ == "__main__":
    main()
