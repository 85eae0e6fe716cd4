"""Writes gelu_near_ties.txt: the binary32 arguments h in [-10, 10] whose
binary64 GeLU h * Phi(h) lies within 1e-14 (relative) of a midpoint between
two binary32 neighbours, the rounding decisions a binary64 evaluation is
least sure of.  Found by an exhaustive scan through the oracle
(oracle.gelu_tie_scan); the file holds arguments only, no expected values.

    python tests/golden/gen_gelu_near_ties.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402

REL = 1e-14


def main():
    oracle.build(force=False)
    oracle.set_threads(os.cpu_count() or 1)
    ten = int(np.float32(10.0).view(np.uint32))
    pats = []
    for lo, hi in ((1, ten + 1), (0x80000001, 0x80000000 + ten + 1)):
        found, n = oracle.gelu_tie_scan(lo, hi, REL)
        assert n == found.size, (n, found.size)
        pats.extend(int(u) for u in found)
    pats.sort()
    out = os.path.join(HERE, "gelu_near_ties.txt")
    with open(out, "w") as f:
        f.write("# Binary32 arguments h in [-10, 10] (bit patterns, hex) whose binary64\n"
                "# GeLU h*Phi(h) lies within 1e-14 relative of a binary32 rounding\n"
                "# midpoint; written by gen_gelu_near_ties.py (exhaustive oracle scan).\n"
                "# GeLU is named by the Zero book's GPU chapter (element-wise section)\n"
                "# and GPT chapter (FFN); the exact form h*Phi(h) is the reading the\n"
                "# tests use.  Arguments only: expected values come from mpmath.\n")
        for u in pats:
            f.write(f"{u:08x}\n")
    print(f"{len(pats)} arguments -> {out}")


if __name__ == "__main__":
    main()
