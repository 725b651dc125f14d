"""Writes quant_mul_vs_div.txt: token elements on which the two scale forms
of the pages round to different int8 codes.

"BitNet 딥다이브" §4-5 quantises with a multiplier, q = round(x * s) with
s = 127 / absmax; "bitnet.rs" ("8-bit Activation Quantisation") divides,
q = round(x / alpha) with alpha = absmax / 127.  In fp32 the two products
differ in the last bit now and then; where one of them lands exactly on a
half, round-half-even then gives codes one apart.  This script searches
seeded N(0,1) fp32 rows with numpy only (no oracle, no GPU) and records the
first such elements; the test that reads the file recomputes both forms.

    python tests/golden/find_quant_mul_vs_div.py > tests/golden/quant_mul_vs_div.txt
"""
import numpy as np


def main(want: int = 4) -> None:
    rng = np.random.default_rng(2024)
    print("# token elements where fp32 x*s and x/alpha round to different codes")
    print("# columns: absmax_bits x_bits  (fp32 as hex); s = fp32(127/absmax),")
    print("# alpha = fp32(absmax/127); written by find_quant_mul_vs_div.py")
    got = 0
    while got < want:
        x = rng.standard_normal(1 << 16).astype(np.float32)
        amax = np.float32(np.abs(x).max())
        s = np.float32(127.0 / np.float64(amax))
        alpha = np.float32(np.float64(amax) / 127.0)
        qm = np.rint(x * s)
        qd = np.rint(x / alpha)
        for k in np.nonzero(qm != qd)[0][:1]:
            print(f"{np.float32(amax).view(np.uint32):08x} {x[k].view(np.uint32):08x}")
            got += 1


if __name__ == "__main__":
    main()
