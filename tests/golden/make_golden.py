"""Writes ``oracle_small.json``: a frozen oracle result on a tiny seeded case.

It calls only ``oracle/`` (and ``synth`` for the seeded bf16 inputs). The
fixture guards the oracle against accidental changes: any later edit of its
arithmetic must regenerate this file in the same commit and name the passage
of the pages that justifies the change.

    python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from synth import make_inputs  # noqa: E402

CASES = [
    dict(name="causal_n12_d4", seed=0, B=1, H=1, N=12, d=4, causal=True, sparse=False),
    dict(name="dense_n9_d8", seed=1, B=1, H=1, N=9, d=8, causal=False, sparse=False),
]


def main():
    out = []
    for c in CASES:
        inp = make_inputs(c["seed"], c["B"], c["H"], c["N"], c["d"])
        scale = 1.0 / math.sqrt(c["d"])
        r = oracle.attn_bwd_ref(inp["q"], inp["k"], inp["v"], inp["do"], c["causal"], scale)
        rec = dict(c)
        rec["scale"] = scale
        rec["inputs_sha"] = {n: int(np.sum(inp[n].astype(np.int64) * np.arange(1, inp[n].size + 1).reshape(inp[n].shape))) for n in ("q", "k", "v", "do")}
        for n in ("O", "lse", "dQ", "dK", "dV"):
            rec[n] = [float(x).hex() for x in r[n].ravel()]
        out.append(rec)
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
