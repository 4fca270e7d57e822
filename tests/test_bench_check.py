"""The benchmark's output check (CPU): on the tiny grid, rows produced by the
oracle's own replay of the block step pass with zero error, and a planted
error in any output is reported for the operator that wrote it."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests"))

import h3gen  # noqa: E402
import oracle  # noqa: E402
from bench_check import check_block_step, sample_rows  # noqa: E402

TINY = dict(T=2, H=6, W=8, A=16, D=256, heads=4, Dh=64, split=(16, 24, 24), F=512)


def _replay(idx, steps, fused, chain, seed=0):
    c = TINY
    D, F, H, Dh = c["D"], c["F"], c["heads"], c["Dh"]
    xd = "f32" if chain else "bf16"
    g = lambda n, r, cols, dt="bf16": h3gen.host_rows(n, r, cols, dt, seed=seed)  # noqa: E731
    m = {n: g(n, 1, D, xd) for n in ("shift", "scale", "gate", "shift2", "scale2", "gate2")}
    x = g("x", idx, D, xd)
    h1, h2 = g("h", idx, D), g("h2", idx, D)
    for _ in range(steps):
        if fused:
            x, _ = oracle.gated_residual_adaln(x, h2, m["gate2"], m["shift"], m["scale"],
                                               y_dtype=np.uint16)
            x, y = oracle.gated_residual_adaln(x, h1, m["gate"], m["shift2"], m["scale2"],
                                               y_dtype=np.uint16)
        else:
            x = oracle.gated_residual(x, h1, m["gate"])
            y = oracle.adaln_modulate(x, m["shift2"], m["scale2"], y_dtype=np.uint16)
            x = oracle.gated_residual(x, h2, m["gate2"])
    N = c["T"] * c["H"] * c["W"] + c["A"]
    pos = oracle.positions(N, c["T"], c["H"], c["W"], c["A"])[idx]
    q, k = oracle.qk_rmsnorm_rope3d(g("q", idx, H * Dh).reshape(-1, H, Dh),
                                    g("k", idx, H * Dh).reshape(-1, H, Dh),
                                    g("q_weight", 1, Dh).reshape(Dh),
                                    g("k_weight", 1, Dh).reshape(Dh), pos, c["split"])
    return {"x": x, "y": y, "act": oracle.swiglu(g("gate_up", idx, 2 * F)),
            "q_out": q.reshape(len(idx), -1), "k_out": k.reshape(len(idx), -1)}


@pytest.mark.parametrize("fused,chain", [(False, False), (True, False), (False, True)])
def test_exact_replay_passes(oracle_lib, fused, chain):
    N = 112
    idx = sample_rows(N, N - 16, every=7, head=4, tail=4)
    got = _replay(idx, 3, fused, chain)
    r = check_block_step(got, idx, TINY, 3, 0, fused=fused, chain=chain)
    assert r["rows"] == len(idx) and r["steps_replayed"] == 3
    assert all(v == 0.0 for v in r["per_op"].values()), r


def test_planted_errors_are_attributed(oracle_lib):
    N = 112
    idx = sample_rows(N, N - 16, every=7, head=4, tail=4)
    for name, op in (("y", "adaln"), ("x", "gated"), ("act", "swiglu"), ("k_out", "qk")):
        got = _replay(idx, 2, False, False)
        a = got[name]
        # one element 8 bf16 ulps away: well past the one-ulp tolerance
        a[3, 5] = np.uint16(int(a[3, 5]) + 8)
        r = check_block_step(got, idx, TINY, 2, 0)
        assert r["per_op"][op] > 1.0, (name, r)
        assert all(v == 0.0 for k, v in r["per_op"].items() if k != op), (name, r)
    # replaying a different number of steps than the GPU ran is caught through x and y
    got = _replay(idx, 2, False, False)
    r = check_block_step(got, idx, TINY, 3, 0)
    assert r["per_op"]["gated"] > 1.0 and r["per_op"]["adaln"] > 1.0
