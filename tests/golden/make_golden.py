"""Write tests/golden/oracle_single_rows.txt from the CPU oracle only.

Stored values are a regression guard for the oracle itself: any later change
to its arithmetic must change this file in the same commit, which names the
passage of the pages that justifies it.  Inputs come from the seeded
generators (ternary_weight_i2_amd.synth, which holds no arithmetic of the
method); every number written here comes from ``oracle``.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from ternary_weight_i2_amd import synth  # noqa: E402


def main():
    W, alpha = synth.matrix("single", "w")
    x = synth.activations("single", "w", 1)
    q, s, qs = oracle.quant_act(x)
    P, bad = oracle.pack_i2s(W)
    assert bad == 0
    R, D = oracle.dot_raw(P, q, qs, W.shape[1])
    rows = [0, 1, 2, 63, 64, 127, 128, 200, 255]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_single_rows.txt")
    with open(out, "w") as f:
        f.write("# Oracle regression values for the 256x512 single-matrix workload\n")
        f.write("# (seeded inputs from ternary_weight_i2_amd.synth; written by\n")
        f.write("# tests/golden/make_golden.py, which calls only the CPU oracle).\n")
        f.write("rows: " + " ".join(map(str, rows)) + "\n")
        f.write("dot: " + " ".join(str(int(D[0, r])) for r in rows) + "\n")
        f.write("qsum: %d\n" % int(qs[0]))
        f.write("packed_row0_first16: " + " ".join(str(int(b)) for b in P[0, :16]) + "\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
