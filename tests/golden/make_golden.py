"""Writes tiny_oracle.txt: the oracle's output on the seeded tiny workload (B=1, H=1, T=64,
d=16, fp32, scalar decay and beta).  Calls only the input generator and the CPU oracle.
It is a regression fixture (does the oracle built on this machine, fed by this generator,
still give the same numbers?), not an independent pin.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

ROWS = (0, 1, 31, 63)


def compute():
    x = synth.make_prefill(synth.WORKLOADS["tiny"])
    o, S = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"])
    return o[0, list(ROWS), 0], S[0, 0]


def main():
    o, S = compute()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")
    with open(path, "w") as f:
        f.write("# fp64 oracle on the seeded tiny workload (seed 1000): rows o_t for t in %s, then S_T\n"
                % (ROWS,))
        f.write("# written by tests/golden/make_golden.py\n")
        for r in o:
            f.write(" ".join("%.17g" % x for x in r) + "\n")
        for r in S:
            f.write(" ".join("%.17g" % x for x in r) + "\n")


if __name__ == "__main__":
    main()
