"""Writes oracle_tiny_fixture.json: the float64 oracle's outputs on a tiny
seeded workload (16 atoms in an 8 A periodic box, 4 A cutoff, lmax 2, mmax 2,
C 16, 8 radial functions, seed 0), summarised per output tensor by its sum,
sum of squares and a few fixed entries. It calls only oracle/ and the input
generators, so it records what the oracle computes today: a regression
fixture that catches accidental changes to the oracle, not an independent
check of it (the pages print no operator values to compare with).

Run from the repository root:  python tests/golden/make_oracle_fixture.py
"""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import so2_synth  # noqa: E402
from oracle import so2conv_oracle as O  # noqa: E402

WORKLOAD = dict(base="T", n_atoms=16, box=8.0, rc=4.0, lmax=2, mmax=2, channels=16, n_rbf=8, seed=0)
ENTRIES = (0, 7, 101, 333)


def summarise(t):
    a = t.detach().double().reshape(-1)
    return {"shape": list(t.shape), "sum": float(a.sum()), "sumsq": float((a * a).sum()),
            "entries": {str(i): float(a[i % a.numel()]) for i in ENTRIES}}


def compute():
    w = dict(WORKLOAD)
    cfg = so2_synth.make_config(w.pop("base"), **w)
    d = so2_synth.make_inputs(cfg)
    inp = O.to_oracle_inputs(d)
    t = lambda a: torch.tensor(a, dtype=torch.float64)  # noqa: E731
    gy = t(d["gy"])
    y = O.forward(inp)
    b = O.backward(inp, gy, with_edge_grad=True)
    dd = O.double_backward(inp, gy, px=t(d["px"]), ppos=t(d["ppos"]), prbf=t(d["prbf"]))
    out = {"n_edges": int(len(d["src"])), "y": summarise(y)}
    for k in ("gx", "gpos", "grbf", "gw_rad", "gedge"):
        out["bwd_" + k] = summarise(b[k])
    out["bwd_gw1_0"] = summarise(b["gw1"][0])
    for k in ("ggy", "gx", "grbf", "gw_rad"):
        out["dbwd_" + k] = summarise(dd[k])
    out["dbwd_gw2_1"] = summarise(dd["gw2"][1])
    return out


if __name__ == "__main__":
    rec = {"workload": WORKLOAD, "written_by": "tests/golden/make_oracle_fixture.py (oracle/ only)",
           "values": compute()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_fixture.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", path)
