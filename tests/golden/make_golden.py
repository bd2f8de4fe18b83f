"""Writes the oracle regression fixture for the tiny workload (hidden 256,
intermediate 768, 8 tokens, seed 0).  Calls only the oracle and the input
generators; rerun it only with a change to the oracle's arithmetic whose
justification is stated in the commit that makes it."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O          # noqa: E402
import q4k_synth as S       # noqa: E402


def main():
    w = S.WORKLOADS["tiny"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    y, _ = O.mlp(S.workload_x(w), wg, wu, wd, w.hidden, w.inter)
    w32 = O.q4k_dequant_f32(wg[0:1, 0:1], 1, 256)[0]
    with open(os.path.join(HERE, "tiny_oracle.txt"), "w") as f:
        f.write("# oracle output of the tiny workload (hidden 256, intermediate 768, 8 tokens, seed 0)\n")
        f.write("# section w32: fp32 dequant of W_gate row 0, block 0 (256 values, exact)\n")
        f.write("# section y0 / y7: float64 y of tokens 0 and 7 (256 values each)\n")
        for name, vals in (("w32", w32.astype(np.float64)), ("y0", y[0]), ("y7", y[7])):
            f.write(f"[{name}]\n")
            for v in vals:
                f.write(float(v).hex() + "\n")


if __name__ == "__main__":
    main()
