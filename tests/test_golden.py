"""The oracle still reproduces its stored outputs on the seeded fp32 case."""
import json
import os

import numpy as np

from oracle import pisa
from workloads import WORKLOADS, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_stored_tiny_case():
    with open(os.path.join(HERE, "golden", "tiny_fp32_oracle.json")) as f:
        g = json.load(f)
    w = WORKLOADS["tiny_fp32"]
    q, k, v = (t.double().numpy() for t in make_inputs(w))
    res = pisa.pisa_reference(q, k, v, w.block, w.k, w.lam, w.scale)
    for key, ref in g["heads"].items():
        b, h = map(int, key.split(","))
        r = res[(b, h)]
        assert np.allclose(r["stats"]["M"], ref["M"], rtol=1e-12, atol=0)
        assert (r["idx"] == np.array(ref["idx"])).all()
        assert np.allclose(r["O"][g["rows"]], ref["O_rows"], rtol=0, atol=1e-13)
