"""The oracle still reproduces the frozen fixture tests/golden/tiny_oracle.txt
(written by tests/golden/make_golden.py, which calls only oracle/)."""
import os

from tests.golden.make_golden import OUT, compute


def test_tiny_oracle_fixture_unchanged():
    want = {}
    with open(OUT) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split(" = ", 1)
            want[k] = v.strip()
    assert compute() == want
