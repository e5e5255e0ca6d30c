"""Write tests/golden/oracle_small.json by calling only the fp64 oracle.

The FiX pages print no worked numeric example, so this fixture is a
regression anchor for the oracle itself, not a page value: any later change
to the oracle's arithmetic that moves these numbers must regenerate it and
say in its commit message which passage (or reading of one) justifies it.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle as O  # noqa: E402


def case():
    rng = np.random.default_rng(2026)
    lengths = [3, 5]
    T, Hq, Hkv, dk, dv = 8, 2, 1, 4, 4
    q = np.round(rng.standard_normal((1, T, Hq, dk)), 3)
    k = np.round(rng.standard_normal((1, T, Hkv, dk)), 3)
    v = np.round(rng.standard_normal((1, T, Hkv, dv)), 3)
    g = np.round(-np.abs(rng.standard_normal((1, T, Hkv, dv))), 3)
    w = np.round(rng.standard_normal(dv), 3)
    z = np.round(rng.standard_normal((1, T, Hq, dv)), 3)
    dO = np.round(rng.standard_normal((1, T, Hq, dv)), 3)
    cu = np.array([0, 3, 8], np.int64)
    return dict(q=q, k=k, v=v, g=g, w=w, z=z, dO=dO, cu=cu, eps=1e-5)


def evaluate(c):
    f = O.oracle_fwd(c["q"], c["k"], c["v"], c["g"], c["cu"], eps=c["eps"], w=c["w"], z=c["z"])
    b = O.oracle_bwd(c["q"], c["k"], c["v"], c["g"], c["dO"], c["cu"], eps=c["eps"], w=c["w"], z=c["z"])
    return {"o": f["o"], "m": f["m"], "rstd": f["rstd"], **{n: b[n] for n in ("dq", "dk", "dv", "dg", "dw", "dz")}}


if __name__ == "__main__":
    c = case()
    out = evaluate(c)
    doc = {"inputs": {n: np.asarray(a).tolist() for n, a in c.items() if n != "eps"},
           "eps": c["eps"],
           "expected": {n: np.asarray(a).tolist() for n, a in out.items()}}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
    print("wrote", path)
