"""Writes config0_oracle_digest.txt: a digest of the fp64 oracle's output on
the page test's case (16 q heads / 1 kv head, seed 0), for the regression pin
in tests/test_golden.py.  It calls only the oracle and the seeded input
generator; nothing here runs the HIP library.

Run from the repository root:  python3 tests/golden/make_oracle_digest.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle      # noqa: E402
import va_inputs   # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config0_oracle_digest.txt")
COLS = (0, 1, 17, 100, 128, 200, 254, 255)        # sampled output dims of every row


def digest_lines():
    p = va_inputs.config(0)
    out, lse = oracle.attn_problem(p)              # [token * 16 + head, 256] and [rows], fp64
    lines = ["# row = token * 16 + head; natural-log LSE, sum, sum of squares, then dims "
             + " ".join(map(str, COLS))]
    for r in range(out.shape[0]):
        x = out[r]
        vals = [float(lse[r]), float(x.sum()), float((x * x).sum())] + [float(x[c]) for c in COLS]
        lines.append(f"{r} " + " ".join(repr(v) for v in vals))
    return lines


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write("\n".join(digest_lines()) + "\n")
    print("wrote", OUT)
