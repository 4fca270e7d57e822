"""Check of a benchmark run's timed outputs against the CPU oracle.

Test infrastructure: bench.py calls it after every timed region (as it runs
its CPU baseline), never inside one.  The timed step is replayed row by row on
the host for a sample of rows: the inputs are regenerated from the seeded
generator, the residual stream is carried through the same number of steps as
the GPU ran (warmup included), rounding to its storage type at every store as
the kernels do, and the last outputs of every operator are compared with what
the GPU left in its buffers.  Every operator is row-local, so a sampled row
depends only on its own inputs.

Result per operator: max over sampled elements of |got - ref| / tol(ref),
tolerances by output type (tolerance.py); <= 1 passes.
"""
from __future__ import annotations

import numpy as np

import h3gen
import oracle
from tolerance import err_over_tol


def sample_rows(n_rows, n_video, every=97, head=64, tail=64):
    """Rows 0..head-1, every `every`-th row, all audio rows, the last `tail` rows."""
    s = set(range(min(head, n_rows)))
    s.update(range(0, n_rows, every))
    s.update(range(n_video, n_rows))
    s.update(range(max(0, n_rows - tail), n_rows))
    return np.array(sorted(s), dtype=np.int64)


def _dev_rows(t, idx):
    """Sampled rows of a GPU tensor -> numpy (bf16 as uint16 bit patterns)."""
    import torch

    it = torch.as_tensor(idx, device=t.device)
    r = t.index_select(0, it).contiguous().cpu()
    if r.dtype == torch.bfloat16:
        return r.view(torch.int16).numpy().view(np.uint16).reshape(len(idx), -1).copy()
    return r.numpy().reshape(len(idx), -1).copy()


OUTPUTS = ("x", "y", "act", "q_out", "k_out")


def fetch_rows(t, idx):
    """Host copies of the sampled rows of a block step's output buffers."""
    return {name: _dev_rows(t[name], idx) for name in OUTPUTS}


def check_block_step(got, idx, c, n_steps, seed, fused=False, chain=False):
    """Compare the sampled rows `got` (fetch_rows) of a block step's buffers after
    n_steps steps with the oracle's replay of the same steps on those rows.

    c: the workload's grid (T, H, W, A, D, heads, Dh, split, F).
    Returns {"per_op": {op: max_err_over_tol}, "rows": n, "steps_replayed": n_steps}."""
    N = c["T"] * c["H"] * c["W"] + c["A"]
    D, F, H, Dh = c["D"], c["F"], c["heads"], c["Dh"]
    xd = "f32" if chain else "bf16"
    g = lambda name, rows, cols, dt="bf16": h3gen.host_rows(name, rows, cols, dt, seed=seed)  # noqa: E731
    mods = {n: g(n, 1, D, xd) for n in ("shift", "scale", "gate", "shift2", "scale2", "gate2")}
    x = g("x", idx, D, xd)
    h1, h2 = g("h", idx, D), g("h2", idx, D)
    y = None
    for _ in range(n_steps):
        if fused:
            x, _ = oracle.gated_residual_adaln(x, h2, mods["gate2"], mods["shift"], mods["scale"],
                                               y_dtype=np.uint16)
            x, y = oracle.gated_residual_adaln(x, h1, mods["gate"], mods["shift2"],
                                               mods["scale2"], y_dtype=np.uint16)
        else:
            oracle.adaln_modulate(x, mods["shift"], mods["scale"], y_dtype=np.uint16)
            x = oracle.gated_residual(x, h1, mods["gate"])
            y = oracle.adaln_modulate(x, mods["shift2"], mods["scale2"], y_dtype=np.uint16)
            x = oracle.gated_residual(x, h2, mods["gate2"])
    act = oracle.swiglu(g("gate_up", idx, 2 * F))
    pos = oracle.positions(N, c["T"], c["H"], c["W"], c["A"])[idx]
    qw, kw = g("q_weight", 1, Dh).reshape(Dh), g("k_weight", 1, Dh).reshape(Dh)
    rq, rk = oracle.qk_rmsnorm_rope3d(g("q", idx, H * Dh).reshape(-1, H, Dh),
                                      g("k", idx, H * Dh).reshape(-1, H, Dh), qw, kw, pos,
                                      c["split"])
    res = {
        "x": err_over_tol(got["x"], x, xd),
        "y": err_over_tol(got["y"], y, "bf16"),
        "act": err_over_tol(got["act"], act, "bf16"),
        "q_out": err_over_tol(got["q_out"], rq.reshape(len(idx), -1), "bf16"),
        "k_out": err_over_tol(got["k_out"], rk.reshape(len(idx), -1), "bf16"),
    }
    per_op = {"qk": max(res["q_out"], res["k_out"]), "swiglu": res["act"]}
    if fused:
        per_op["gated_adaln"] = max(res["x"], res["y"])
    else:
        per_op["adaln"] = res["y"]
        per_op["gated"] = res["x"]
    return {"per_op": {k: round(v, 4) for k, v in per_op.items()}, "rows": int(len(idx)),
            "steps_replayed": int(n_steps)}
