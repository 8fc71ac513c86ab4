"""Write tests/golden/tiny_seed0.txt: sampled fp64 oracle outputs of the tiny
fp32 workload (1 x 256, H=2, P=16, N=16, G=1, seed 0).

The pages print no worked numerical example, so this fixture is not a pin of
the oracle; it freezes the seeded generator plus oracle pair so that a later
change to either shows up as a diff.  It calls only the oracle and the seeded
input generator.  Run:  python tests/golden/make_golden.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

SAMPLES_Y = [(0, 0, 0, 0), (0, 1, 1, 3), (0, 63, 0, 15), (0, 64, 1, 7), (0, 127, 0, 9),
             (0, 200, 1, 0), (0, 255, 0, 5), (0, 255, 1, 15)]
SAMPLES_FS = [(0, 0, 0, 0), (0, 1, 15, 15), (0, 0, 7, 3), (0, 1, 2, 11)]


def main():
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"], seed=0)
    y, fs = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_seed0.txt")
    with open(out, "w") as f:
        f.write("# fp64 oracle on the tiny fp32 workload, seed 0; kind index... value\n")
        for s in SAMPLES_Y:
            f.write("y %d %d %d %d %.17g\n" % (*s, y[s]))
        for s in SAMPLES_FS:
            f.write("fs %d %d %d %d %.17g\n" % (*s, fs[s]))
        f.write("ymax %.17g\n" % np.abs(y).max())
    print("wrote", out)


if __name__ == "__main__":
    main()
