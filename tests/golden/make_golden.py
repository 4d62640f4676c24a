"""Write tests/golden/oracle_small.json: the oracle's outputs on a tiny seeded
case, kept as a regression fixture (any later change to the oracle's
arithmetic shows up as a diff).  Calls only oracle/ and synth/."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def case():
    R, H = 6, 16
    x = synth.rows(0, "x", 0, R, H)
    r = synth.rows(0, "r", 0, R, H)
    dy = synth.rows(0, "dy", 0, R, H)
    w = synth.weight(0, H, "bf16")
    y, h, rstd = oracle.fwd_bf16(x, w, 1e-6, r)
    rho32 = rstd.astype(np.float32)
    dx, _, dw = oracle.bwd_bf16(h, dy, w, rho32)
    g = synth.rows(0, "g", 0, R, H)
    gy, grstd = oracle.gated_fwd_bf16(x, g, w, 1e-6)
    gdx, gdg, _, _, gdw = oracle.gated_bwd_bf16(x, g, dy, w, grstd.astype(np.float32))
    return {
        "R": R, "H": H, "eps": 1e-6, "seed": 0,
        "y": [int(v) for v in y.ravel()],
        "h": [int(v) for v in h.ravel()],
        "rstd": [float(v).hex() for v in rstd],
        "dx": [int(v) for v in dx.ravel()],
        "dw": [float(v).hex() for v in dw],
        "gated": {
            "y": [int(v) for v in gy.ravel()],
            "rstd": [float(v).hex() for v in grstd],
            "dx": [int(v) for v in gdx.ravel()],
            "dg": [int(v) for v in gdg.ravel()],
            "dw": [float(v).hex() for v in gdw],
        },
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(case(), f, indent=0)
        f.write("\n")
