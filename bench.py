"""Benchmark of the fused per-token DiT operators (libh3fused) on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: the six
fused-operator calls of one DiT block at the 5 s 1344x768 token shape
(125,120 tokens = 31x48x84 video + 128 audio, hidden 5120, 40 heads x 128,
SwiGLU inner 13,824, bf16 I/O):

    adaln(x -> y) ; qk_rmsnorm_rope3d(q, k -> q', k') ; gated(x += g1*h1) ;
    adaln(x -> y) ; swiglu(gate_up -> act) ; gated(x += g2*h2)

Inputs are generated on the device before timing.  The reported value is the
step's algorithmic bytes (each input element read once, each output element
written once) divided by the step time: achieved HBM GB/s.  Per-operator
durations come from HIP events recorded around every launch on the stream the
kernels run on.  The CPU oracle is timed on a bounded sample of the same
workload (rank 0) as a baseline.  Outside the step, `extra_ops` times the
step-reuse residual difference and the block-sparse attention router on the
same shape.

On the sweep shapes (tensors of a few hundred MB, comparable to the 256 MB
Infinity Cache) a 1 GiB scratch buffer is written before every timed launch
(--flush-mb), each launch is timed by its own event pair, and the step time is
the sum of the launch times.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5s|10s|chain10s|sweepD]
                       [--fused] [--no-cpu-baseline] [--seed S] [--flush-mb M]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published peak

GRIDS = {
    "5s": dict(T=31, H=48, W=84, A=128, D=5120, heads=40, Dh=128, split=(32, 48, 48), F=13824),
    "10s": dict(T=61, H=48, W=84, A=256, D=5120, heads=40, Dh=128, split=(32, 48, 48), F=13824),
}
for _D, _F in ((3072, 8320), (4096, 11008), (5120, 13824), (6144, 16640)):
    GRIDS[f"sweep{_D}"] = dict(T=8, H=48, W=84, A=512, D=_D, heads=_D // 128, Dh=128,
                               split=(32, 48, 48), F=_F)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="5s", choices=sorted(GRIDS) + ["chain10s"])
    ap.add_argument("--fused", action="store_true",
                    help="fuse each gated residual with the AdaLN that follows it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=32768,
                    help="rows of the workload the oracle is timed on")
    ap.add_argument("--seed", type=int, default=0, help="seed of the synthetic inputs")
    ap.add_argument("--flush-mb", type=int, default=-1,
                    help="MiB written to a scratch buffer before every timed launch, so no "
                         "operand is served from the 256 MB Infinity Cache (default: 1024 for "
                         "the sweep shapes, whose tensors are comparable to the cache; 0 "
                         "otherwise)")
    return ap.parse_args()


def op_bytes(name, N, c, x_bytes=2):
    """Algorithmic bytes of one call (activations bf16, x of x_bytes per element)."""
    D, F, H, Dh = c["D"], c["F"], c["heads"], c["Dh"]
    if name == "adaln":
        return N * D * x_bytes + N * D * 2 + 2 * D * x_bytes
    if name == "gated":
        return 2 * N * D * x_bytes + N * D * 2 + D * x_bytes
    if name == "swiglu":
        return 3 * N * F * 2
    if name == "qk":
        return 4 * N * H * Dh * 2 + 2 * Dh * 2
    if name == "gated_adaln":
        return 2 * N * D * x_bytes + N * D * 2 + N * D * 2 + 3 * D * x_bytes
    raise KeyError(name)


def router_bytes(N, c, nb, keep):
    """Algorithmic bytes of one router call: q and k read once (bf16), the fp32
    block scores and the int32 kept-block lists written once."""
    H, Dh = c["heads"], c["Dh"]
    return 2 * N * H * Dh * 2 + H * nb * nb * 4 + H * nb * keep * 4


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "video_diffusion_transformer_h3f_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/pmc_traffic.json), or None when it is missing or the kernel's
    source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        doc = json.load(open(path))
        ent = doc["kernels"][f"{kernel_key}@{workload}"]
        if ent.get("source_digest") != source_digest(ent["source_files"]):
            return None
    except (KeyError, ValueError, OSError):
        return None
    return ent.get("hbm_bytes_per_launch")


def build_inputs(c, N, torch, h3gen, dev, chain=False, seed=0):
    D, F, H, Dh = c["D"], c["F"], c["heads"], c["Dh"]
    bf = torch.bfloat16
    xdt = torch.float32 if chain else bf
    t = {}

    def mk(name, rows, cols, dt, gen_name=None):
        x = torch.empty(rows, cols, dtype=dt, device=dev)
        h3gen.fill_device(x, gen_name or name, seed=seed)
        return x

    t["x"] = mk("x", N, D, xdt)
    for n in ("shift", "scale", "gate", "shift2", "scale2", "gate2"):
        t[n] = mk(n, 1, D, xdt)
    t["h"] = mk("h", N, D, bf)
    t["h2"] = mk("h2", N, D, bf)
    t["gate_up"] = mk("gate_up", N, 2 * F, bf)
    if chain:
        qkv = torch.empty(N, 3, H, Dh, dtype=bf, device=dev)
        flat = qkv.view(N, 3 * H * Dh)
        for i, n in enumerate(("q", "k", "v")):
            h3gen.fill_device(flat[:, i * H * Dh:(i + 1) * H * Dh], n, seed=seed)
        t["qkv"] = qkv
        t["q"], t["k"] = qkv[:, 0], qkv[:, 1]
    else:
        t["q"] = mk("q", N, H * Dh, bf).view(N, H, Dh)
        t["k"] = mk("k", N, H * Dh, bf).view(N, H, Dh)
    t["q_weight"] = mk("q_weight", 1, Dh, bf).view(Dh)
    t["k_weight"] = mk("k_weight", 1, Dh, bf).view(Dh)
    t["y"] = torch.empty(N, D, dtype=bf, device=dev)
    t["q_out"] = torch.empty(N, H, Dh, dtype=bf, device=dev)
    t["k_out"] = torch.empty(N, H, Dh, dtype=bf, device=dev)
    t["act"] = torch.empty(N, F, dtype=bf, device=dev)
    return t


def make_step(h3, t, rope, fused):
    """The six fused calls of one DiT block, each tagged with its operator name."""
    if not fused:
        return [
            ("adaln", lambda: h3.h3f_adaln_modulate(t["y"], t["x"], t["shift"], t["scale"])),
            ("qk", lambda: h3.h3f_qk_rmsnorm_rope3d(t["q_out"], t["k_out"], t["q"], t["k"],
                                                   t["q_weight"], t["k_weight"], rope)),
            ("gated", lambda: h3.h3f_gated_residual(t["x"], t["h"], t["gate"])),
            ("adaln", lambda: h3.h3f_adaln_modulate(t["y"], t["x"], t["shift2"], t["scale2"])),
            ("swiglu", lambda: h3.h3f_swiglu(t["act"], t["gate_up"])),
            ("gated", lambda: h3.h3f_gated_residual(t["x"], t["h2"], t["gate2"])),
        ]
    # gated residual + the next AdaLN in one pass; the block's first AdaLN is fused
    # with the previous block's last gated residual
    return [
        ("gated_adaln", lambda: h3.h3f_gated_residual_adaln(
            t["x"], t["h2"], t["gate2"], t["shift"], t["scale"], t["y"])),
        ("qk", lambda: h3.h3f_qk_rmsnorm_rope3d(t["q_out"], t["k_out"], t["q"], t["k"],
                                               t["q_weight"], t["k_weight"], rope)),
        ("gated_adaln", lambda: h3.h3f_gated_residual_adaln(
            t["x"], t["h"], t["gate"], t["shift2"], t["scale2"], t["y"])),
        ("swiglu", lambda: h3.h3f_swiglu(t["act"], t["gate_up"])),
    ]


def cpu_baseline(c, rows, x_bytes, min_seconds=10.0, seed=0):
    """Time the oracle on `rows` rows of the same workload (one block's six calls),
    on all the host threads it uses, and again on one thread over a sixteenth of
    the sample."""
    import oracle

    full = _time_oracle(c, rows, x_bytes, min_seconds, seed)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        one = _time_oracle(c, max(1, rows // 16), x_bytes, min_seconds / 2, seed)
    finally:
        oracle.set_num_threads(threads)
    full["single_thread"] = {"value": one["value"], "unit": "GB/s", "cores": 1,
                             "seconds": one["seconds"], "steps": one["steps"],
                             "sample": one["sample"]}
    return full


def _time_oracle(c, rows, x_bytes, min_seconds, seed):
    import numpy as np

    import h3gen
    import oracle

    D, F, H, Dh = c["D"], c["F"], c["heads"], c["Dh"]
    xd = "f32" if x_bytes == 4 else "bf16"
    g = lambda n, r, cols, dt="bf16": h3gen.host_rows(n, r, cols, dt, seed=seed)  # noqa: E731
    x = g("x", rows, D, xd)
    mods = {n: g(n, 1, D, xd) for n in ("shift", "scale", "gate", "shift2", "scale2", "gate2")}
    hh, hh2 = g("h", rows, D), g("h2", rows, D)
    q = g("q", rows, H * Dh).reshape(rows, H, Dh)
    k = g("k", rows, H * Dh).reshape(rows, H, Dh)
    qw, kw = g("q_weight", 1, Dh), g("k_weight", 1, Dh)
    gu = g("gate_up", rows, 2 * F)
    pos = oracle.positions(rows, c["T"], c["H"], c["W"], c["A"])
    # the sample's steps are repeated until at least min_seconds of CPU work
    # have been timed (each step restarts from the same x)
    x0 = x
    reps = 0
    t0 = time.perf_counter()
    while True:
        x = x0
        oracle.adaln_modulate(x, mods["shift"], mods["scale"], y_dtype=np.uint16)
        oracle.qk_rmsnorm_rope3d(q, k, qw, kw, pos, c["split"])
        x = oracle.gated_residual(x, hh, mods["gate"])
        oracle.adaln_modulate(x, mods["shift2"], mods["scale2"], y_dtype=np.uint16)
        oracle.swiglu(gu)
        oracle.gated_residual(x, hh2, mods["gate2"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    nbytes = reps * sum(op_bytes(n, rows, c, x_bytes) for n in
                        ("adaln", "qk", "gated", "adaln", "swiglu", "gated"))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3), "steps": reps,
            "sample": f"{rows} of the workload's rows (tokens 0..{rows - 1}), the six fused "
                      f"calls of one block, {reps} steps, inputs from the same seeded generator"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this benchmark runs on exactly one GPU (the operators are row-local; "
              "a multi-GPU run would shard rows with no exchange); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import h3gen
    import video_diffusion_transformer_h3f_amd as h3

    h3.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    chain = args.workload == "chain10s"
    c = GRIDS["10s" if chain else args.workload]
    N = c["T"] * c["H"] * c["W"] + c["A"]
    x_bytes = 4 if chain else 2
    t = build_inputs(c, N, torch, h3gen, dev, chain=chain, seed=args.seed)
    flush_mb = args.flush_mb if args.flush_mb >= 0 else (
        1024 if args.workload.startswith("sweep") else 0)
    scratch = torch.empty(flush_mb << 20, dtype=torch.uint8, device=dev) if flush_mb else None
    flush = (lambda: scratch.fill_(1)) if flush_mb else None

    def time_calls(fn, reps):
        """Average ms of fn over reps launches: back to back, or each after a flush
        with its own event pair (the flush is outside the timed interval)."""
        if flush is None:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(reps)]
        for a, b in pairs:
            flush()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in pairs) / reps
    rope = h3.make_rope(c["T"], c["H"], c["W"], c["A"], c["split"])
    step = make_step(h3, t, rope, args.fused)
    if chain:
        args.steps = 50 if args.steps == 30 else args.steps

    # copy ceiling (untimed for the metric): 2 GiB -> 2 GiB
    cp_src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    for _ in range(3):
        h3.h3f_stream_copy(cp_dst, cp_src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        h3.h3f_stream_copy(cp_dst, cp_src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * cp_src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del cp_src, cp_dst

    for _ in range(args.warmup):
        for _, fn in step:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    n_ops = len(step)
    # event pairs around every launch; without a flush consecutive launches share
    # their boundary event
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_ops)] for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(K):
        for i, (_, fn) in enumerate(step):
            if flush is not None:
                flush()
            if flush is not None or i == 0:
                ev[s][2 * i].record()
            fn()
            ev[s][2 * i + 1].record()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    def launch_ms(s, i):
        first = ev[s][2 * i] if (flush is not None or i == 0) else ev[s][2 * i - 1]
        return first.elapsed_time(ev[s][2 * i + 1])

    per_op_ms = {}
    per_op_n = {}
    per_op_all = {}
    for s in range(K):
        for i, (name, _) in enumerate(step):
            ms = launch_ms(s, i)
            per_op_ms[name] = per_op_ms.get(name, 0.0) + ms
            per_op_n[name] = per_op_n.get(name, 0) + 1
            per_op_all.setdefault(name, []).append(ms)
    if flush is None:
        ms_per_step = start.elapsed_time(stop) / K
    else:  # the flushes between launches are not part of a step
        ms_per_step = sum(launch_ms(s, i) for s in range(K) for i in range(n_ops)) / K
    step_bytes = sum(op_bytes(name, N, c, x_bytes) for name, _ in step)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    per_op = {}
    for name in per_op_ms:
        avg = per_op_ms[name] / per_op_n[name]
        b = op_bytes(name, N, c, x_bytes)
        ts = sorted(per_op_all[name])
        per_op[name] = {"avg_ms": round(avg, 4), "median_ms": round(ts[len(ts) // 2], 4),
                        "min_ms": round(ts[0], 4), "launches": len(ts),
                        "bytes": b, "GBps": round(b / (avg * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                        "frac_of_copy_ceiling": round(b / (avg * 1e-3) / 1e9 / copy_gbps, 4)}

    # Step-reuse test (residual difference between neighbouring steps): timed on its
    # own, outside the block step, since a block runs it at most once per step.
    extra_ops = {}
    if not chain:
        x_prev = torch.empty_like(t["x"])
        h3gen.fill_device(x_prev, "x_prev")
        l1_out = torch.zeros(3, dtype=torch.float64, device=dev)
        ws = torch.empty(max(16, h3.h3f_residual_l1_workspace_bytes(N, c["D"], t["x"].dtype)),
                         dtype=torch.uint8, device=dev)
        for _ in range(3):
            h3.h3f_residual_l1(l1_out, t["x"], x_prev, ws)
        torch.cuda.synchronize()
        avg = time_calls(lambda: h3.h3f_residual_l1(l1_out, t["x"], x_prev, ws), K)
        b = 2 * N * c["D"] * 2
        extra_ops["residual_l1"] = {"avg_ms": round(avg, 4), "bytes": b,
                                    "GBps": round(b / (avg * 1e-3) / 1e9, 1),
                                    "frac_of_peak": round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        del x_prev, ws

        # Block-sparse attention router on the step's post-RoPE q / k (what attention
        # reads), blocks of 128 tokens, sparsity 0.8, a routed step.
        blk, sp = 128, 0.8
        nb, keep, need = h3.h3f_subblock_plan(N, c["heads"], c["Dh"], blk, sp, 10)
        kv = torch.empty(c["heads"], nb, keep, dtype=torch.int32, device=dev)
        sc = torch.empty(c["heads"], nb, nb, dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
        for _ in range(3):
            h3.h3f_subblock_route(kv, sc, t["q_out"], t["k_out"], blk, sp, 10, ws)
        torch.cuda.synchronize()
        avg = time_calls(lambda: h3.h3f_subblock_route(kv, sc, t["q_out"], t["k_out"], blk, sp,
                                                       10, ws), K)
        b = router_bytes(N, c, nb, keep)
        extra_ops["subblock_route"] = {
            "avg_ms": round(avg, 4), "bytes": b, "GBps": round(b / (avg * 1e-3) / 1e9, 1),
            "frac_of_peak": round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "block": blk, "sparsity": sp, "n_blocks": nb, "keep": keep,
            "score_flops": 2 * c["heads"] * nb * nb * c["Dh"]}

        # A routed step with the router's pooling fused into the QK operator: the
        # QK call that also writes the block means, then the route from them.
        def qk_pool():
            h3.h3f_qk_rmsnorm_rope3d_pool(t["q_out"], t["k_out"], t["q"], t["k"], t["q_weight"],
                                          t["k_weight"], rope, blk, ws)

        def route_pooled():
            h3.h3f_subblock_route_pooled(kv, sc, N, c["heads"], blk, sp, 10, ws)

        for _ in range(3):
            qk_pool()
            route_pooled()
        torch.cuda.synchronize()
        a_qp = time_calls(qk_pool, K)
        a_rp = time_calls(route_pooled, K)
        b_qp = op_bytes("qk", N, c, x_bytes) + 2 * c["heads"] * nb * c["Dh"] * 4
        b_rp = c["heads"] * nb * nb * 4 + c["heads"] * nb * keep * 4 + 2 * c["heads"] * nb * c["Dh"] * 4
        extra_ops["qk_rmsnorm_rope3d_pool"] = {
            "avg_ms": round(a_qp, 4), "bytes": b_qp, "GBps": round(b_qp / (a_qp * 1e-3) / 1e9, 1),
            "frac_of_peak": round(b_qp / (a_qp * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        extra_ops["subblock_route_pooled"] = {
            "avg_ms": round(a_rp, 4), "bytes": b_rp, "GBps": round(b_rp / (a_rp * 1e-3) / 1e9, 1)}
        extra_ops["routed_qk_step_ms"] = {
            "separate": round(per_op["qk"]["avg_ms"] + avg, 4), "fused": round(a_qp + a_rp, 4)}
        del kv, sc, ws

    dom = "swiglu"
    roofline = {"bound": "hbm", "achieved": per_op[dom]["GBps"], "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": per_op[dom]["frac_of_peak"],
                "traffic": traffic_from_profiles(dom, args.workload),
                "kernel": "swiglu_kernel<bf16,8>", "bytes_per_launch": per_op[dom]["bytes"],
                "avg_launch_ms": per_op[dom]["avg_ms"]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(c, min(args.cpu_rows, N), x_bytes, seed=args.seed)

    wl = {"5s": "5 s 1344x768 clip token shape", "10s": "10 s 1344x768 clip token shape",
          "chain10s": "10 s shape, fp32 residual stream, packed qkv, block epilogue chain"}
    config = {
        "workload": (wl.get(args.workload, f"roofline sweep, hidden {c['D']}") +
                     f": {N} tokens ({c['T']}x{c['H']}x{c['W']} video + {c['A']} audio), "
                     f"hidden {c['D']}, {c['heads']}x{c['Dh']} heads, RoPE split "
                     f"{'/'.join(map(str, c['split']))}, SwiGLU inner {c['F']}; one DiT block's "
                     f"{'four fused (gated+AdaLN fused)' if args.fused else 'six'} fused-op calls "
                     f"per step"),
        "tokens": N, "hidden": c["D"], "heads": c["heads"], "head_dim": c["Dh"],
        "swiglu_inner": c["F"], "fused_gated_adaln": bool(args.fused),
    }
    out = {
        "metric": "achieved HBM GB/s (and % of peak) per fused op at 5 s 1344x768 token shape",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # arithmetic; every kernel computes in fp32 on bf16 / fp32 storage
        "storage_dtype": ("fp32 residual stream, bf16 activations" if chain else "bf16"),
        "data": "synthetic (seeded counter-based generator, N(0,1)-like activations)",
        "config": config,
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "per_op": per_op,
        "extra_ops": extra_ops,
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "cache_flush_mb": flush_mb,
        "seed": args.seed,
        "wall_s_timed_region": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
