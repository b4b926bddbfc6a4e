"""Write the tiny-step fixtures in this folder from the 50-digit reference.

The pages print no worked example of a Dion step, so these fixtures are not
the pages' numbers: they are the 50-digit modified-Gram-Schmidt step of
oracle/mp_reference.py (steps as on the rivista.ai Dion page, "Dion e la fine
del monopolio di Adam negli optimizer AI distribuiti": error feedback, one
power-iteration step, QR) on small dyadic inputs that are exact in fp32.
They pin the fp64 oracle, which uses a different QR algorithm.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.mp_reference import dion_step_mp  # noqa: E402


def inputs(m, n, r):
    i = np.arange(m)[:, None]
    j = np.arange(n)[None, :]
    X = (((i * 7 + j * 3) % 11) - 5) / 64.0
    G = (((i * 5 + j * 2) % 13) - 6) / 32.0
    M = (((i + 3 * j) % 7) - 3) / 16.0
    k = np.arange(r)[None, :]
    jn = np.arange(n)[:, None]
    Q = (((jn * 3 + k * 5) % 9) - 4) / 8.0 + np.eye(n, r)
    return X, G, M, Q


CASES = [
    dict(name="tall-6x5-r3", m=6, n=5, r=3, mu=0.95, lr=0.01, eps=1e-8),
    dict(name="wide-4x7-fullrank", m=4, n=7, r=4, mu=0.9, lr=0.05, eps=1e-8),
    dict(name="square-5x5-r2-eps", m=5, n=5, r=2, mu=0.5, lr=0.1, eps=0.25),
]


def main():
    out = []
    for c in CASES:
        X, G, M, Q = inputs(c["m"], c["n"], c["r"])
        res = dion_step_mp(X, G, M, Q, c["mu"], c["lr"], c["eps"])
        out.append(dict(case=c, inputs={k: v.tolist() for k, v in dict(X=X, G=G, M=M, Q=Q).items()},
                        expected={k: res[k].tolist() for k in ("X", "M", "Q", "P", "PQ", "R")}))
    with open(os.path.join(HERE, "tiny_steps_mp50.json"), "w") as f:
        json.dump({"source": "oracle/mp_reference.py at 50 digits (modified Gram-Schmidt QR); "
                             "inputs from tests/golden/make_golden.py",
                   "cases": out}, f, indent=1)


if __name__ == "__main__":
    main()
