"""Reader for the hand-worked golden fixtures in this folder.

A fixture is a text file: '#' comment lines (citation and the derivation by
hand), 'key value' scalar lines, and matrix blocks (a key on its own line
followed by rows of numbers).  An 'expected' block at the end holds the values
written by make_golden.py, which calls only the oracle.
"""
from __future__ import annotations

import numpy as np

SCALARS = ("B", "P", "V", "d", "r", "K", "prev")
MATS = ("logits", "hidden", "W", "A", "Btab")


def read_fixture(path):
    sc, mats, exp = {}, {}, {}
    cur = None
    in_exp = False
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "expected":
                in_exp = True
                cur = None
                continue
            if in_exp:
                exp[parts[0]] = [float(x) for x in parts[1:]]
                continue
            if parts[0] in SCALARS and len(parts) == 2:
                sc[parts[0]] = int(parts[1])
                cur = None
                continue
            if parts[0] in MATS and len(parts) == 1:
                cur = parts[0]
                mats[cur] = []
                continue
            mats[cur].append([float(x) for x in parts])
    B, P, V, d, r = sc["B"], sc["P"], sc["V"], sc["d"], sc["r"]
    fx = dict(
        K=sc["K"],
        prev=np.full(B, sc["prev"], dtype=np.int32),
        logits=np.array(mats["logits"], dtype=np.float64).reshape(B, P, V),
        hidden=np.array(mats["hidden"], dtype=np.float64).reshape(B, P, d),
        W=np.array(mats["W"], dtype=np.float64).reshape(r, d),
        A=np.array(mats["A"], dtype=np.float64).reshape(V, r),
        Bt=np.array(mats["Btab"], dtype=np.float64).reshape(V, r),
    )
    return fx, exp
