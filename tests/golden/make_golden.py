"""Writes tests/golden/tiny_oracle.txt from the CPU oracle alone.

The pages print no worked NVFP4 example, so this fixture freezes what the
oracle (pinned by tests/test_oracle_*.py) gives on the 256x256 FP32 workload:
A quantized along its rows' contiguous dimension, B (K x N) quantized along
K (transposing), both RNE; digests of codes and scales, the tensor scales as
float32 bit patterns, and a few reference outputs of C = A^ . B^.
Run:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from bit_block_scaled_nvfp4_amd import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")


def compute():
    t = W.tiny()
    a = O.quantize(t["A"].numpy(), O.F32, axis=O.ALONG_COLS)
    b = O.quantize(t["B"].numpy(), O.F32, axis=O.ALONG_ROWS)
    y, _ = O.gemm_ref(a, b, 1.0, 0, np.array([0, 100, 255]))
    lines = {
        "a_codes_sha256": hashlib.sha256(a.codes.tobytes()).hexdigest(),
        "a_scales_sha256": hashlib.sha256(a.scales.tobytes()).hexdigest(),
        "a_tensor_scale_bits": "%08x" % int(np.float32(a.tensor_scale).view(np.uint32)),
        "b_codes_sha256": hashlib.sha256(b.codes.tobytes()).hexdigest(),
        "b_scales_sha256": hashlib.sha256(b.scales.tobytes()).hexdigest(),
        "b_tensor_scale_bits": "%08x" % int(np.float32(b.tensor_scale).view(np.uint32)),
        "c_row0_col0_7": " ".join(repr(float(v)) for v in y[0, :8]),
        "c_row100_col0_7": " ".join(repr(float(v)) for v in y[1, :8]),
        "c_row255_col248_255": " ".join(repr(float(v)) for v in y[2, 248:]),
    }
    return lines


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write("# written by tests/golden/make_golden.py from oracle/ only\n")
        for k, v in compute().items():
            f.write(f"{k} = {v}\n")
    print("wrote", OUT)
