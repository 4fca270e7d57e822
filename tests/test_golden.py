"""Regression lock: the oracle still reproduces the stored tiny-configuration
samples bit for bit (tests/golden/tiny_oracle_samples.json, written by
tests/golden/make_golden.py, which calls only the oracle and the generator)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_tiny_oracle_samples_unchanged():
    doc = json.load(open(os.path.join(HERE, "golden", "tiny_oracle_samples.json")))
    outs, pos = make_golden.tiny_outputs()
    assert pos[doc["rows"]].tolist() == doc["positions"]
    for name, rows in doc["samples"].items():
        a = outs[name]
        for ri, r in enumerate(doc["rows"]):
            want = np.array([float.fromhex(v) for v in rows[ri]], dtype=np.float64)
            got = a[r, :doc["cols"]].astype(np.float64)
            assert np.array_equal(got, want), (name, r)
