"""Writes the stored oracle outputs under tests/golden/ (calls only oracle/).

The LT2 pages print no worked numerical example of the gated-delta recurrence,
so the fixtures here are not the pages' numbers: they freeze the oracle's output
on small seeded inputs, so that any later change of the oracle's arithmetic
shows up as a failing regression test and has to name the passage that
justifies it.  Inputs are rebuilt from the seeded generators at test time.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from linear_attention_looped_amd import synth  # noqa: E402

CASES = {
    "gdn_head_f32": synth.GDNShape(1, 37, 2, 8, 6, "head", 0.0, "f32"),
    "gdn_channel_bf16": synth.GDNShape(1, 37, 2, 8, 6, "channel", 2.0, "bf16"),
}


def main():
    out = {}
    for name, shape in CASES.items():
        x = synth.gdn_inputs(shape, seed=0)
        o, S = oracle.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"])
        out[name] = dict(shape=list(shape.__dict__.values()), seed=0,
                         o=np.round(o, 15).ravel().tolist(), S=np.round(S, 15).ravel().tolist())
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f)


if __name__ == "__main__":
    main()
