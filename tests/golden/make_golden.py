"""Writes tests/golden/tiny_fp32_oracle.txt from the fp64 oracle alone.

The AnchorFormer pages print no worked numeric example for anchor attention, so
the only stored values here are the oracle's own, frozen so that a later change to
the oracle's arithmetic shows up as a diff.  Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from efficient_vision_transformer_amd.inputs import make_inputs  # noqa: E402

ROWS = (0, 17, 63)


def main():
    x = make_inputs("tiny_fp32")
    A, delta, W, H = oracle.anchor_slice(x.Q[0, 0], x.U[0], x.V[0, 0])
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.txt")
    with open(out, "w") as f:
        f.write("# tiny fp32 workload (B=1 h=1 n=64 m=8 d=32, seed 1001), fp64 oracle output\n")
        f.write("# written by tests/golden/make_golden.py (oracle only)\n")
        f.write("delta " + " ".join(f"{v:.17e}" for v in delta) + "\n")
        for r in ROWS:
            f.write(f"H{r} " + " ".join(f"{v:.17e}" for v in H[r]) + "\n")
        f.write(f"Hsum {H.sum():.17e}\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
