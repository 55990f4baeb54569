"""Writes quant_error_anchor.txt from the CPU oracle alone.

Workload from the page "旋转量化：大模型低比特量化中的离群值克星", section 2.2:
one row of 4096 standard-normal float32 values from numpy's default_rng(42)
with entry 123 replaced by a spike of 30, quantised to symmetric INT4 with a
per-row absmax scale, once as is and once after the normalised 4096-point
Hadamard rotation (all signs +1).  The mean absolute quantisation error is
measured in the domain that was quantised, as the page's snippet does.

Run from the repository root:  python tests/golden/make_quant_error_anchor.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from hadamard_rotation_amd import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402


def mean_abs_error(w, b):
    s = np.ones(4096, dtype=np.int8)
    r = O.rotate_quant(w, O.F32, b, s, 4, O.F32, want_xr=True)
    q = O.unpack_codes(r["codes"], 4, 4096)
    deq = q * r["scales"].astype(np.float64)[:, None]
    return float(np.mean(np.abs(r["xr"] - deq)))


def main():
    w = W.spiked_gaussian_row(42, 4096, 123, 30.0)
    unrot = mean_abs_error(w, 1)      # b = 1: identity rotation
    rot = mean_abs_error(w, 4096)     # full normalised rotation
    path = os.path.join(HERE, "quant_error_anchor.txt")
    with open(path, "w") as f:
        f.write("# Written by tests/golden/make_quant_error_anchor.py from the CPU oracle.\n")
        f.write("# Error-reduction example of \"旋转量化：大模型低比特量化中的离群值克星\"\n")
        f.write("# section 2.2 (seed 42, spike 30 at index 123, INT4).\n")
        f.write("# The page prints about 0.19 unrotated and below 0.02 rotated; those\n")
        f.write("# figures do not follow from its own recipe and are not pinned.\n")
        f.write(f"unrotated {unrot:.12g}\n")
        f.write(f"rotated {rot:.12g}\n")
    print(path, unrot, rot)


if __name__ == "__main__":
    main()
