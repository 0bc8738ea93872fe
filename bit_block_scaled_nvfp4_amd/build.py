"""Build libnvfp4.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m bit_block_scaled_nvfp4_amd.build

Compiles every csrc/*.hip to an object under build/ and links the shared
library next to this file; also builds the measurement probe
probes/mfma_ceiling.hip into the executable `mfma_ceiling` (not part of the
library).  Flags that matter for bit-exact results: no FMA
contraction, correctly rounded FP32 divide, no denormal flushing, and packed
FP32 instructions disabled."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "build")
LIB = os.path.join(PKG, "libnvfp4.so")
PROBE_SRC = os.path.join(PKG, "probes", "mfma_ceiling.hip")
PROBE = os.path.join(PKG, "mfma_ceiling")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *COMMON, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stderr=None if verbose else subprocess.PIPE)))
        objs.append(obj)
    for cmd, p in procs:  # the translation units compile side by side
        _, err = p.communicate()
        if p.returncode != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd, stderr=err)
    tmp = LIB + ".tmp"
    subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    subprocess.run([cc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", PROBE + ".tmp"],
                   check=True, stderr=None if verbose else subprocess.PIPE)
    os.replace(PROBE + ".tmp", PROBE)
    return LIB


def build_shared(src: str, out: str, verbose: bool = False) -> str:
    """One HIP source -> a shared library `out`, with the library's flags
    (used for test probes that exercise the library's device functions)."""
    cmd = [hipcc(), *COMMON, "-shared", src, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
