"""Write ``oracle_tiny.json``: oracle outputs for tiny seeded inputs.

Calls only ``oracle/`` and the seeded generator in ``workloads.py``.  The
stored values guard against silent drift of the oracle or of the input
recipe; they are not an independent pin (the pins live in test_oracle.py).

    python tests/golden/make_oracle_fixture.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402

CASES = [
    {"B": 1, "H": 2, "N": 5, "D": 4, "dtype": "f16", "seed": 7, "causal": True},
    {"B": 1, "H": 1, "N": 6, "D": 8, "dtype": "bf16", "seed": 8, "causal": False},
]


def main():
    out = {"_about": __doc__.strip().splitlines()[0], "attn": [], "softmax": []}
    for c in CASES:
        q, k, v = workloads.attn_inputs(c["B"], c["H"], c["N"], c["D"], c["dtype"], c["seed"])
        o, lse = oracle.attn_fwd(q, k, v, c["causal"], nthreads=1)
        out["attn"].append(dict(c, o=o.reshape(-1).tolist(), lse=lse.reshape(-1).tolist()))
    x = workloads.softmax_inputs(3, 9, seed=9)
    y = oracle.row_softmax(x, nthreads=1)
    out["softmax"].append({"M": 3, "N": 9, "seed": 9, "last": 80.0, "y": y.reshape(-1).tolist()})
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
