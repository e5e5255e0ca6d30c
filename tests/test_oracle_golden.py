"""The oracle reproduces its stored regression fixture (tests/golden)."""
import json
import os

import numpy as np

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_fixture():
    doc = json.load(open(os.path.join(HERE, "golden", "oracle_small.json")))
    a = {n: np.array(v) for n, v in doc["inputs"].items()}
    f = O.oracle_fwd(a["q"], a["k"], a["v"], a["g"], a["cu"].astype(np.int64), eps=doc["eps"], w=a["w"], z=a["z"])
    b = O.oracle_bwd(a["q"], a["k"], a["v"], a["g"], a["dO"], a["cu"].astype(np.int64), eps=doc["eps"],
                     w=a["w"], z=a["z"])
    got = {"o": f["o"], "m": f["m"], "rstd": f["rstd"], **b}
    for n, v in doc["expected"].items():
        np.testing.assert_allclose(got[n], np.array(v), rtol=1e-12, atol=1e-12, err_msg=n)
