"""Write tests/golden/tiny_layer.txt from the CPU oracle (and the seeded input generator) only.

Run from the repository root:  python tests/golden/make_golden.py
The file pins the oracle's own output on the tiny layer (T=16, H=256, E=64, k=4, I=128, 2-bit
experts, seed 0) so that any later change to the oracle's arithmetic shows up as a diff.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402


def main():
    s = mi.TINY
    y, ids, rw, out, a = oracle.layer(mi.make_weights(s), mi.make_x(s), mi.make_logits(s), s.k,
                                      intermediates=True)
    with open(os.path.join(HERE, "tiny_layer.txt"), "w") as f:
        f.write("# Oracle output on the tiny layer (T=16 H=256 E=64 k=4 I=128, 2-bit, seed 0).\n")
        f.write("# Written by tests/golden/make_golden.py, which calls only oracle/ and moe_inputs/.\n")
        f.write("# ids: topk ids row-major; y_head: y[:, :8] row-major (fp64 hex);"
                " y_rowsum: sum of each y row (fp64 hex)\n")
        f.write("ids " + " ".join(str(int(v)) for v in ids.reshape(-1)) + "\n")
        f.write("y_head " + " ".join(float(v).hex() for v in y[:, :8].reshape(-1)) + "\n")
        f.write("y_rowsum " + " ".join(float(v).hex() for v in y.sum(axis=1)) + "\n")


if __name__ == "__main__":
    main()
