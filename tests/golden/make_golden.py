"""Writes tests/golden/tiny_oracle_samples.json: sampled outputs of the CPU
oracle on the tiny configuration (112 tokens = 2x6x8 video + 16 audio,
hidden 256, 4 heads x 64, RoPE split 16/24/24, SwiGLU inner 512, fp32, seed 0).

It calls only the oracle and the seeded input generator.  The pages print no
worked example for any of the operators, so this file is a regression lock on
the oracle (its correctness is pinned by tests/test_oracle_pins.py); values
are stored as fp32 hex strings so that the comparison is exact.

Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import h3gen  # noqa: E402
import oracle  # noqa: E402

T, H, W, A = 2, 6, 8, 16
N, D, HEADS, DH, F = T * H * W + A, 256, 4, 64, 512
SPLIT = (16, 24, 24)
ROWS = [0, 1, 47, 95, 96, 111]
COLS = 8


def tiny_outputs():
    g = lambda name, rows, cols: h3gen.host_rows(name, rows, cols, "f32", seed=0)  # noqa: E731
    x = g("x", N, D)
    out = {}
    out["adaln_y"] = oracle.adaln_modulate(x, g("shift", 1, D), g("scale", 1, D), eps=1e-6)
    out["gated_x"] = oracle.gated_residual(x, g("h", N, D), g("gate", 1, D))
    out["swiglu_out"] = oracle.swiglu(g("gate_up", N, 2 * F))
    pos = oracle.positions(N, T, H, W, A)
    q = g("q", N, HEADS * DH).reshape(N, HEADS, DH)
    k = g("k", N, HEADS * DH).reshape(N, HEADS, DH)
    qo, ko = oracle.qk_rmsnorm_rope3d(q, k, g("q_weight", 1, DH), g("k_weight", 1, DH), pos,
                                      SPLIT, eps=1e-6)
    out["q_out"] = qo.reshape(N, HEADS * DH)
    out["k_out"] = ko.reshape(N, HEADS * DH)
    return out, pos


def sample(a):
    return [[float(v).hex() for v in a[r, :COLS]] for r in ROWS]


def main():
    outs, pos = tiny_outputs()
    doc = {
        "what": "oracle outputs on the tiny configuration, rows %s, first %d columns" % (ROWS, COLS),
        "written_by": "tests/golden/make_golden.py (calls only oracle/ and h3gen/)",
        "rows": ROWS,
        "cols": COLS,
        "positions": pos[ROWS].tolist(),
        "samples": {k: sample(v) for k, v in outs.items()},
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_samples.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
