"""Seeded random shapes for every per-token entry point, against the oracle.

Each case draws its arguments from a generator seeded by the case number, so a
failure names a reproducible case: random row counts (ragged against every
tile size), hidden sizes that are any multiple of the vector width, padded
row strides, modulation groupings, dtype combinations, head counts, head
dimensions and RoPE splits, token offsets that wrap the sequence, both pair
layouts, and packed qkv views.  Tolerances as in every parity test (fp32
|err| <= 1e-6 + 1e-5 |ref|, bf16 |err| <= 2^-7 |ref| + 1e-3)."""
import numpy as np
import pytest
import torch

import h3gen
import oracle
from gpu_util import DEV, dev_tensor, from_np, host, kind, to_np
from tolerance import assert_close

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("video_diffusion_transformer_h3f_amd")

N_CASES = 12
DT_PAIRS = [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h3.lib()
    h3gen.dev_lib()
    yield
    torch.cuda.synchronize()


def tdt(d):
    return torch.bfloat16 if d == "bf16" else torch.float32


def npy(d):
    return np.uint16 if d == "bf16" else np.float32


def width(*dts):
    return 4 if "f32" in dts else 8


def grouping(r, rows):
    """rows_per_group and group count: one group, per token, or a random split."""
    rpg = int(r.choice([rows, 1, int(r.integers(1, rows + 1))]))
    return rpg, -(-rows // rpg)


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_gated_residual(case):
    r = np.random.default_rng(1000 + case)
    xd, hd = DT_PAIRS[int(r.integers(3))]
    V = width(xd, hd)
    rows, D = int(r.integers(1, 700)), V * int(r.integers(1, 800))
    xpad, hpad = V * int(r.integers(0, 4)), V * int(r.integers(0, 4))
    rpg, groups = grouping(r, rows)
    print(f"gated case {case}: rows={rows} D={D} {xd}/{hd} pads={xpad},{hpad} rpg={rpg}", flush=True)
    x = dev_tensor("x", rows, D, xd, row_stride=D + xpad)
    h = dev_tensor("h", rows, D, hd, row_stride=D + hpad)
    gate = dev_tensor("gate", groups, D, xd)
    h3.h3f_gated_residual(x, h, gate, rows_per_group=rpg)
    ref = oracle.gated_residual(host("x", rows, D, xd), host("h", rows, D, hd),
                                host("gate", groups, D, xd), rows_per_group=rpg)
    assert_close(to_np(x), ref, kind(xd), f"gated case {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_swiglu(case):
    r = np.random.default_rng(2000 + case)
    dt = "f32" if r.integers(2) else "bf16"
    V = width(dt)
    rows, F = int(r.integers(1, 600)), V * int(r.integers(1, 1200))
    packed = bool(r.integers(2))
    print(f"swiglu case {case}: rows={rows} F={F} {dt} packed={packed}", flush=True)
    ref = oracle.swiglu(np.concatenate([host("gate_up", rows, F, dt), host("h", rows, F, dt)], 1))
    out = torch.empty(rows, F, dtype=tdt(dt), device=DEV)
    if packed:
        gu = torch.empty(rows, 2 * F, dtype=tdt(dt), device=DEV)
        gu[:, :F] = dev_tensor("gate_up", rows, F, dt)
        gu[:, F:] = dev_tensor("h", rows, F, dt)
        h3.h3f_swiglu(out, gu)
    else:
        a = dev_tensor("gate_up", rows, F, dt, row_stride=F + V * int(r.integers(0, 4)))
        b = dev_tensor("h", rows, F, dt, row_stride=F + V * int(r.integers(0, 4)))
        h3.h3f_swiglu(out, a, b)
    assert_close(to_np(out), ref, kind(dt), f"swiglu case {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_adaln(case):
    r = np.random.default_rng(3000 + case)
    xd, yd = DT_PAIRS[int(r.integers(3))]
    V = width(xd, yd)
    max_d = 8192 if xd == "f32" else 16384
    rows, D = int(r.integers(1, 500)), V * int(r.integers(1, max_d // V + 1))
    xpad = V * int(r.integers(0, 4))
    rpg, groups = grouping(r, rows)
    print(f"adaln case {case}: rows={rows} D={D} {xd}->{yd} pad={xpad} rpg={rpg}", flush=True)
    x = dev_tensor("x", rows, D, xd, row_stride=D + xpad)
    sh, sc = dev_tensor("shift", groups, D, xd), dev_tensor("scale", groups, D, xd)
    y = torch.empty(rows, D, dtype=tdt(yd), device=DEV)
    h3.h3f_adaln_modulate(y, x, sh, sc, eps=1e-6, rows_per_group=rpg)
    ref = oracle.adaln_modulate(host("x", rows, D, xd), host("shift", groups, D, xd),
                                host("scale", groups, D, xd), eps=1e-6, y_dtype=npy(yd),
                                rows_per_group=rpg)
    assert_close(to_np(y), ref, kind(yd), f"adaln case {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_gated_residual_adaln(case):
    r = np.random.default_rng(4000 + case)
    xd, hd = DT_PAIRS[int(r.integers(3))]
    yd = "f32" if (xd == "f32" and r.integers(2)) else "bf16"
    V = width(xd, hd, yd)
    max_d = 8192 if xd == "f32" else 16384
    rows, D = int(r.integers(1, 400)), V * int(r.integers(1, max_d // V + 1))
    rpg, groups = grouping(r, rows)
    print(f"fused case {case}: rows={rows} D={D} x={xd} h={hd} y={yd} rpg={rpg}", flush=True)
    x = dev_tensor("x", rows, D, xd)
    h = dev_tensor("h", rows, D, hd, row_stride=D + V * int(r.integers(0, 4)))
    gate, sh, sc = (dev_tensor(n, groups, D, xd) for n in ("gate", "shift", "scale"))
    y = torch.empty(rows, D, dtype=tdt(yd), device=DEV)
    h3.h3f_gated_residual_adaln(x, h, gate, sh, sc, y, eps=1e-6, rows_per_group=rpg)
    rx, ry = oracle.gated_residual_adaln(host("x", rows, D, xd), host("h", rows, D, hd),
                                         host("gate", groups, D, xd), host("shift", groups, D, xd),
                                         host("scale", groups, D, xd), eps=1e-6, y_dtype=npy(yd),
                                         rows_per_group=rpg)
    assert_close(to_np(x), rx, kind(xd), f"fused x case {case}")
    assert_close(to_np(y), ry, kind(yd), f"fused y case {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_adaln_affine(case):
    r = np.random.default_rng(8000 + case)
    xd, yd = DT_PAIRS[int(r.integers(3))]
    V = width(xd, yd)
    max_d = 8192 if xd == "f32" else 16384
    rows, D = int(r.integers(1, 400)), V * int(r.integers(1, max_d // V + 1))
    rpg, groups = grouping(r, rows)
    print(f"adaln affine case {case}: rows={rows} D={D} {xd}->{yd} rpg={rpg}", flush=True)
    x = dev_tensor("x", rows, D, xd, row_stride=D + V * int(r.integers(0, 4)))
    gm, bt = dev_tensor("ln_gamma", 1, D, xd).view(D), dev_tensor("ln_beta", 1, D, xd).view(D)
    sh, sc = dev_tensor("shift", groups, D, xd), dev_tensor("scale", groups, D, xd)
    y = torch.empty(rows, D, dtype=tdt(yd), device=DEV)
    h3.h3f_adaln_affine_modulate(y, x, gm, bt, sh, sc, eps=1e-6, rows_per_group=rpg)
    ref = oracle.adaln_affine_modulate(host("x", rows, D, xd), host("ln_gamma", 1, D, xd),
                                       host("ln_beta", 1, D, xd), host("shift", groups, D, xd),
                                       host("scale", groups, D, xd), eps=1e-6, y_dtype=npy(yd),
                                       rows_per_group=rpg)
    assert_close(to_np(y), ref, kind(yd), f"adaln affine case {case}")


SPLITS = {32: (8, 8, 16), 64: (16, 24, 24), 128: (32, 48, 48), 256: (64, 96, 96)}


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_qk_rmsnorm_rope3d(case):
    r = np.random.default_rng(5000 + case)
    dt = "f32" if r.integers(2) else "bf16"
    Dh = int(r.choice([32, 64, 128, 256]))
    split = SPLITS[Dh]
    # the rotate-half layout needs every axis chunk to be a multiple of 16
    pairing = (h3.H3F_ROPE_HALF_SPLIT if all(s % 16 == 0 for s in split) and r.integers(2)
               else h3.H3F_ROPE_INTERLEAVED)
    H = int(r.integers(1, 7))
    T, Hg, W, A = int(r.integers(1, 6)), int(r.integers(1, 9)), int(r.integers(1, 11)), int(r.integers(0, 20))
    rows, offset = int(r.integers(1, 400)), int(r.integers(0, 1000))
    packed = bool(r.integers(2))
    print(f"qk case {case}: rows={rows} H={H} Dh={Dh} {dt} grid={T}x{Hg}x{W}+{A} off={offset} "
          f"pairing={pairing} packed={packed}", flush=True)
    if packed:
        qkv = torch.full((rows, 3, H, Dh), float("nan"), dtype=tdt(dt), device=DEV)
        flat = qkv.view(rows, 3 * H * Dh)
        h3gen.fill_device(flat[:, :H * Dh], "q")
        h3gen.fill_device(flat[:, H * Dh:2 * H * Dh], "k")
        q, k = qkv[:, 0], qkv[:, 1]
    else:
        q = dev_tensor("q", rows, H * Dh, dt).view(rows, H, Dh)
        k = dev_tensor("k", rows, H * Dh, dt).view(rows, H, Dh)
    qw = dev_tensor("q_weight", 1, Dh, dt).view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, dt).view(Dh)
    qo = torch.empty(rows, H, Dh, dtype=tdt(dt), device=DEV)
    ko = torch.empty_like(qo)
    rope = h3.make_rope(T, Hg, W, A, split, token_offset=offset, pairing=pairing)
    h3.h3f_qk_rmsnorm_rope3d(qo, ko, q, k, qw, kw, rope, eps=1e-6)
    pos = oracle.positions(rows, T, Hg, W, A, token_offset=offset)
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", rows, H * Dh, dt).reshape(rows, H, Dh),
                                      host("k", rows, H * Dh, dt).reshape(rows, H, Dh),
                                      to_np(qw), to_np(kw), pos, split, eps=1e-6,
                                      pairing=pairing)
    assert_close(to_np(qo), rq, kind(dt), f"q case {case}")
    assert_close(to_np(ko), rk, kind(dt), f"k case {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_positions(case):
    r = np.random.default_rng(6000 + case)
    T, Hg, W, A = int(r.integers(1, 40)), int(r.integers(1, 60)), int(r.integers(1, 90)), int(r.integers(0, 300))
    rows, offset = int(r.integers(1, 20000)), int(r.integers(0, 10 ** 6))
    print(f"positions case {case}: rows={rows} grid={T}x{Hg}x{W}+{A} off={offset}", flush=True)
    pos = torch.empty(rows, 3, dtype=torch.int32, device=DEV)
    h3.h3f_rope3d_positions(pos, h3.make_rope(T, Hg, W, A, (16, 24, 24), token_offset=offset))
    assert np.array_equal(to_np(pos), oracle.positions(rows, T, Hg, W, A, token_offset=offset))


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_residual_l1(case):
    r = np.random.default_rng(7000 + case)
    dt = "f32" if r.integers(2) else "bf16"
    V = width(dt)
    rows, D = int(r.integers(1, 3000)), V * int(r.integers(1, 700))
    pad = V * int(r.integers(0, 4))
    print(f"residual_l1 case {case}: rows={rows} D={D} {dt} pad={pad}", flush=True)
    cur = dev_tensor("x", rows, D, dt, row_stride=D + pad)
    prev = dev_tensor("x_prev", rows, D, dt, row_stride=D + pad)
    out = torch.zeros(3, dtype=torch.float64, device=DEV)
    h3.h3f_residual_l1(out, cur, prev)
    got = out.cpu().numpy()
    num, den = oracle.residual_l1(host("x", rows, D, dt), host("x_prev", rows, D, dt))
    assert abs(got[0] - num) <= 1e-5 * num and abs(got[1] - den) <= 1e-5 * den


def test_fuzz_explicit_positions_match_grid():
    # explicit positions equal to the grid's give the same q/k, bit for bit
    rows, H, Dh = 257, 3, 128
    q = dev_tensor("q", rows, H * Dh, "bf16").view(rows, H, Dh)
    k = dev_tensor("k", rows, H * Dh, "bf16").view(rows, H, Dh)
    qw = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    outs = []
    for explicit in (False, True):
        qo, ko = torch.empty_like(q), torch.empty_like(k)
        pos = from_np(oracle.positions(rows, 3, 5, 7, 9, token_offset=11)) if explicit else None
        rope = h3.make_rope(3, 5, 7, 9, SPLITS[Dh], token_offset=0 if explicit else 11,
                            positions=pos)
        h3.h3f_qk_rmsnorm_rope3d(qo, ko, q, k, qw, kw, rope)
        torch.cuda.synchronize()
        outs.append((to_np(qo), to_np(ko)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
