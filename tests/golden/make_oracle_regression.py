"""Write oracle_regression_small.json: a small fixed problem and the fp64 oracle's
outputs for it.  Calls only the oracle package.  The file guards against unintended
changes to the oracle's arithmetic; any intended change regenerates it and names the
passage that justifies the change in its commit message.

Inputs are a deterministic trigonometric pattern (no random generator), L = 11
tokens, d = 4, band width W = 4, T = 3 base steps, R = 2, epsilon = 0.8.
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def inputs():
    L, d = 11, 4
    i = np.arange(L)[:, None]
    c = np.arange(d)[None, :]
    Q = np.sin(0.7 * i + 1.3 * c + 0.1)
    K = np.cos(0.5 * i - 0.9 * c + 0.3)
    V = np.sin(1.1 * i * (c + 1) + 0.2)
    dO = np.cos(0.3 * i + 2.1 * c - 0.4)
    return Q, K, V, dO


def main():
    Q, K, V, dO = inputs()
    prob = oracle.BandProblem(W=4, T=3, R=2, eps=0.8)
    O, duals = oracle.forward(Q, K, V, prob)
    dQ, dK, dV = oracle.vjp_one_reference(Q, K, V, dO, duals, prob)
    out = dict(problem=dict(W=4, T=3, R=2, eps=0.8), O=O.tolist(), duals=duals.tolist(),
               dQ=dQ.tolist(), dK=dK.tolist(), dV=dV.tolist())
    with open(os.path.join(HERE, "oracle_regression_small.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
