"""Writes tests/golden/tiny_cross_f32.txt from the fp64 oracle (calls only oracle/).

Run from the repository root: python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import ref  # noqa: E402
from ragged_attention_serving_amd import synth  # noqa: E402


def main():
    w = synth.tiny_cross(0)
    out, lse = ref.run_workload(w)
    path = os.path.join(ROOT, "tests", "golden", "tiny_cross_f32.txt")
    with open(path, "w") as f:
        f.write("# oracle output for the tiny fp32 cross-attention workload (seed 0)\n")
        f.write("# row head lse out[0..15]\n")
        for i in range(out.shape[0]):
            for h in range(out.shape[1]):
                vals = " ".join(f"{v:.17g}" for v in out[i, h])
                f.write(f"{i} {h} {lse[i, h]:.17g} {vals}\n")


if __name__ == "__main__":
    main()
