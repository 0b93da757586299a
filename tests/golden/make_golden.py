"""Write tests/golden/tiny_oracle.json: oracle outputs on the tiny workload.

Calls only `oracle/` and the seeded generators.  The pages print no values of
the operation, so this fixture is a regression guard for the oracle (values it
produced once, after its pins passed), not an external pin.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle import convtp as ct, graph, sh  # noqa: E402
from workloads import gen  # noqa: E402


def compute():
    d = gen.tiny(seed=0)
    L = d["lmax"]
    prob = ct.Problem(L, L, L)
    Y = sh.real_sh(L, d["vec"]).astype(np.float32)
    out = ct.fwd(prob, d["x"], Y, d["w"], d["row_ptr"], d["senders"])
    sp, pe, sr = graph.transpose(d["n_nodes"], d["row_ptr"], d["senders"])
    dx = ct.bwd_dx(prob, Y, d["w"], d["grad_out"], sp, pe, sr)
    dw, dY = ct.bwd_edges(prob, d["x"], Y, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    dvec = sh.vec_grad_from_sh_grad(L, d["vec"], dY)
    pick = dict(out=(out, [(0, 0, 0), (5, 3, 15), (63, 1, 7)]),
                dx=(dx, [(0, 0, 0), (17, 2, 9), (63, 3, 15)]),
                dw=(dw, [(0, 0, 0), (500, 4, 3), (1023, 2, 15)]),
                dY=(dY, [(0, 0), (777, 3), (1023, 1)]),
                dvec=(dvec, [(0, 0), (10, 2), (1023, 1)]))
    return {k: [[list(i), float(a[i])] for i in idx] for k, (a, idx) in pick.items()}


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(dict(workload="tiny, seed 0, Y = real_sh(vec) rounded to fp32",
                       values=compute()), f, indent=1)
