"""Write the 'expected' block of each golden fixture by calling the oracle only.

Usage: python tests/golden/make_golden.py
The hand derivation in each fixture's comments must agree with what this
writes; tests/test_oracle_pins.py checks both the stored values and an
independent brute-force enumeration against them.
"""
import glob
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from golden_io import read_fixture  # noqa: E402


def fmt(a):
    return " ".join(repr(float(x)) if not float(x).is_integer() else str(int(x))
                    for x in list(a))


def main():
    for path in sorted(glob.glob(os.path.join(HERE, "*.txt"))):
        fx, _ = read_fixture(path)
        o = oracle.select(fx["logits"], fx["hidden"], fx["A"], fx["Bt"], fx["W"],
                          fx["prev"], fx["K"])
        with open(path) as f:
            lines = f.read().split("\nexpected\n")[0].rstrip("\n").split("\n")
        lines.append("expected")
        lines.append("cand " + fmt(o["cand"].ravel()))
        lines.append("U " + fmt(o["U"].ravel()))
        lines.append("path " + fmt(o["path"].ravel()))
        lines.append("path_rank " + fmt(o["path_rank"].ravel()))
        lines.append("score " + fmt(o["score"].ravel()))
        lines.append("second " + fmt(o["second"].ravel()))
        lines.append("greedy_path " + fmt(o["greedy_path"].ravel()))
        lines.append("greedy_rank " + fmt(o["greedy_rank"].ravel()))
        lines.append("greedy_score " + fmt(o["greedy_score"].ravel()))
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("wrote", os.path.basename(path))


if __name__ == "__main__":
    main()
