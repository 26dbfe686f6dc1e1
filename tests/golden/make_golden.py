"""Write tests/golden/tiny_fp32_oracle.json from the fp64 oracle alone.

The summary pages print no worked numeric example of the method, so the only
stored expected values are these oracle outputs on the seeded 1024-token fp32
workload; they guard the oracle against silent changes (its correctness is
pinned by tests/test_oracle_pins.py). Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import pisa  # noqa: E402
from workloads import WORKLOADS, make_inputs  # noqa: E402

ROWS = [0, 1, 63, 64, 500, 777, 1023]


def main():
    w = WORKLOADS["tiny_fp32"]
    q, k, v = (t.double().numpy() for t in make_inputs(w))
    res = pisa.pisa_reference(q, k, v, w.block, w.k, w.lam, w.scale)
    out = {"workload": w.describe(), "rows": ROWS, "heads": {}}
    for (b, h), r in res.items():
        out["heads"][f"{b},{h}"] = {
            "M": r["stats"]["M"].tolist(),
            "Hbar_fro": float((r["stats"]["Hbar"] ** 2).sum() ** 0.5),
            "kbar_row0": r["stats"]["kbar"][0].tolist(),
            "idx": r["idx"].tolist(),
            "O_rows": r["O"][ROWS].tolist(),
        }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
