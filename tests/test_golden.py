"""Regression pin: the oracle still reproduces its stored outputs (see golden/README.md)."""
import json
import os

import numpy as np

import oracle
from linear_attention_looped_amd import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_regression_fixture():
    with open(os.path.join(HERE, "oracle_regression.json")) as f:
        data = json.load(f)
    for name, rec in data.items():
        shape = synth.GDNShape(*rec["shape"])
        x = synth.gdn_inputs(shape, seed=rec["seed"])
        o, S = oracle.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
        np.testing.assert_allclose(o.ravel(), rec["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(S.ravel(), rec["S"], rtol=0, atol=1e-14)
