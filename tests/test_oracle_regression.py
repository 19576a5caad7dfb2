"""The oracle still reproduces the regression fixture its committed script wrote."""

import json
import os

import numpy as np

import oracle
from tests.golden.make_oracle_regression import inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_regression_fixture():
    with open(os.path.join(HERE, "golden", "oracle_regression_small.json")) as f:
        ref = json.load(f)
    Q, K, V, dO = inputs()
    prob = oracle.BandProblem(**ref["problem"])
    O, duals = oracle.forward(Q, K, V, prob)
    dQ, dK, dV = oracle.vjp_one_reference(Q, K, V, dO, duals, prob)
    for name, X in (("O", O), ("duals", duals), ("dQ", dQ), ("dK", dK), ("dV", dV)):
        np.testing.assert_allclose(X, np.array(ref[name]), rtol=0, atol=1e-13)
