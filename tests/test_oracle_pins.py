"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, hand-worked values, invariants of the definitions, and special
cases that reduce to library routines (torch / scipy on the CPU, float64).

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a biased/unbiased mix-up, the wrong
half of the gate/up buffer, the wrong pairing or axis) fails it.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tolerance import as_f64, ulp_f32

RNG = np.random.default_rng(1234)


def f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def bf16_bits(a):
    """Round float values to bf16 bit patterns with torch (library RNE)."""
    t = torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ----------------------------------------------------------------------------------
# conversions
# ----------------------------------------------------------------------------------

def test_bf16_narrowing_matches_torch_rne():
    vals = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, -3.5, 3.3895314e38], np.float32),
        # exact ties: 1 + 2^-8 (tie -> even 1.0), 1 + 3*2^-8 (tie -> 1 + 2^-6)
        np.array([1.00390625, 1.01171875, -1.00390625], np.float32),
    ])
    ours = np.array([oracle.f32_to_bf16_scalar(float(v)) for v in vals], np.uint16)
    assert np.array_equal(ours, bf16_bits(vals))
    assert oracle.f32_to_bf16_scalar(1.00390625) == 0x3F80
    assert oracle.f32_to_bf16_scalar(1.01171875) == 0x3F82


def test_bf16_widening_is_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    ours = oracle.bf16_to_f32(bits)
    finite = np.isfinite(t)
    assert np.array_equal(ours[finite], t[finite])
    assert np.all(np.isnan(ours[~np.isfinite(t) & np.isnan(t)]))


# ----------------------------------------------------------------------------------
# positions
# ----------------------------------------------------------------------------------

def brute_positions(T, H, W, A):
    out = []
    for t in range(T):
        for h in range(H):
            for w in range(W):
                out.append((t, h, w))
    for k in range(A):
        out.append((k, 0, 0))
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("grid", [(2, 6, 8, 16), (3, 5, 7, 4), (1, 1, 1, 0), (4, 2, 3, 9)])
def test_positions_brute_force(grid):
    T, H, W, A = grid
    ref = brute_positions(T, H, W, A)
    got = oracle.positions(len(ref), T, H, W, A)
    assert np.array_equal(got, ref)


def test_positions_offset_and_wrap():
    T, H, W, A = 2, 6, 8, 16
    ref = brute_positions(T, H, W, A)
    L = len(ref)
    for off in (0, 5, L - 3, L, 3 * L + 7):
        got = oracle.positions(2 * L, T, H, W, A, token_offset=off)
        idx = (off + np.arange(2 * L)) % L
        assert np.array_equal(got, ref[idx])


def test_positions_5s_grid_counts():
    # 31 x 48 x 84 latent grid + 128 audio tokens: 125,120 rows.
    T, H, W, A = 31, 48, 84, 128
    n = T * H * W + A
    assert n == 125120
    p = oracle.positions(n, T, H, W, A)
    assert p[:, 0].max() == 127 and p[T * H * W - 1].tolist() == [30, 47, 83]
    assert np.all(p[T * H * W:, 1:] == 0)


# ----------------------------------------------------------------------------------
# AdaLN modulate
# ----------------------------------------------------------------------------------

def test_adaln_hand_worked_d8():
    # x = 1..8: mean 4.5, biased variance 42/8 = 5.25 (the unbiased one would be 6).
    x = f32([np.arange(1, 9)])
    zero = f32(np.zeros((1, 8)))
    y = as_f64(oracle.adaln_modulate(x, zero, zero, eps=0.0))
    expect = (np.arange(1, 9) - 4.5) / math.sqrt(5.25)
    assert np.max(np.abs(y[0] - expect)) <= 2 * ulp_f32(expect).max()
    # scale = 1 doubles, shift = 0.25 offsets
    y2 = as_f64(oracle.adaln_modulate(x, f32(np.full((1, 8), 0.25)), f32(np.ones((1, 8))), eps=0.0))
    assert np.max(np.abs(y2[0] - (2 * expect + 0.25))) <= 4 * ulp_f32(2 * expect + 0.25).max()


def test_adaln_zero_modulation_is_layer_norm():
    x = f32(RNG.standard_normal((37, 256)) * 3 + 0.7)
    zero = f32(np.zeros((1, 256)))
    y = as_f64(oracle.adaln_modulate(x, zero, zero, eps=1e-6))
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (256,),
                                         eps=float(np.float32(1e-6))).numpy()
    ref32 = ref.astype(np.float32).astype(np.float64)
    assert np.max(np.abs(y - ref32) / ulp_f32(ref)) <= 1.0


def test_adaln_row_moments():
    x = f32(RNG.standard_normal((16, 512)) * 0.01 + 5.0)
    zero = f32(np.zeros((1, 512)))
    eps = 1e-6
    y = as_f64(oracle.adaln_modulate(x, zero, zero, eps=eps))
    xd = x.astype(np.float64)
    var = xd.var(axis=1)
    assert np.all(np.abs(y.mean(axis=1)) < 1e-6)
    ms = (y ** 2).mean(axis=1)
    assert np.allclose(ms, var / (var + np.float64(np.float32(eps))), rtol=1e-6)


def test_adaln_shift_invariance():
    # values on a 1/64 grid: adding 3.0 is exact in fp32
    x = f32(RNG.integers(-256, 256, (8, 128)) / 64.0)
    sh = f32(RNG.standard_normal((1, 128)) * 0.1)
    sc = f32(RNG.standard_normal((1, 128)) * 0.1)
    y0 = as_f64(oracle.adaln_modulate(x, sh, sc))
    y1 = as_f64(oracle.adaln_modulate(f32(x + 3.0), sh, sc))
    assert np.max(np.abs(y0 - y1) / ulp_f32(y0)) <= 1.0


def test_adaln_scale_minus_one_gives_shift_exactly():
    x = f32(RNG.standard_normal((9, 64)))
    sh = f32(RNG.standard_normal((1, 64)))
    y = oracle.adaln_modulate(x, sh, f32(-np.ones((1, 64))))
    assert np.array_equal(y, np.broadcast_to(sh, y.shape))
    xb = bf16_bits(RNG.standard_normal((9, 64)))
    shb = bf16_bits(RNG.standard_normal((1, 64)))
    yb = oracle.adaln_modulate(xb, shb, bf16_bits(-np.ones((1, 64))))
    assert np.array_equal(yb, np.broadcast_to(shb, yb.shape))


def test_adaln_affine_zero_modulation_is_layer_norm_with_weight_and_bias():
    x = f32(RNG.standard_normal((29, 192)) * 2 + 0.3)
    gamma = f32(1 + RNG.standard_normal(192) * 0.2)
    beta = f32(RNG.standard_normal(192) * 0.3)
    zero = f32(np.zeros((1, 192)))
    y = as_f64(oracle.adaln_affine_modulate(x, gamma, beta, zero, zero, eps=1e-6))
    ref = torch.nn.functional.layer_norm(
        torch.from_numpy(x.astype(np.float64)), (192,),
        weight=torch.from_numpy(gamma.astype(np.float64)),
        bias=torch.from_numpy(beta.astype(np.float64)), eps=float(np.float32(1e-6))).numpy()
    assert np.max(np.abs(y - ref.astype(np.float32).astype(np.float64)) / ulp_f32(ref)) <= 1.0


def test_adaln_affine_order_and_degenerate_parameters():
    x = f32(RNG.standard_normal((7, 64)))
    gamma = f32(1 + RNG.standard_normal(64) * 0.2)
    beta = f32(RNG.standard_normal(64))
    sh = f32(RNG.standard_normal((1, 64)))
    sc = f32(RNG.standard_normal((1, 64)) * 0.3)
    # the modulation acts on the affine LayerNorm output: scale = -1 leaves exactly shift
    y = oracle.adaln_affine_modulate(x, gamma, beta, sh, f32(-np.ones((1, 64))))
    assert np.array_equal(y, np.broadcast_to(sh, y.shape))
    # gamma = 0 leaves beta (1 + scale) + shift, whatever x is
    y0 = as_f64(oracle.adaln_affine_modulate(x, f32(np.zeros(64)), beta, sh, sc))
    want = beta.astype(np.float64) * (1 + sc.astype(np.float64)) + sh.astype(np.float64)
    assert np.max(np.abs(y0 - want) / ulp_f32(want)) <= 1.0
    # gamma = 1, beta = 0 is the plain AdaLN modulate
    y1 = oracle.adaln_affine_modulate(x, f32(np.ones(64)), f32(np.zeros(64)), sh, sc)
    assert np.array_equal(y1, oracle.adaln_modulate(x, sh, sc))


def test_adaln_bf16_output_is_rounded_f32_output():
    x = f32(RNG.standard_normal((11, 96)))
    sh = f32(RNG.standard_normal((1, 96)) * 0.1)
    sc = f32(RNG.standard_normal((1, 96)) * 0.1)
    y32 = oracle.adaln_modulate(x, sh, sc, y_dtype=np.float32)
    yb = oracle.adaln_modulate(x, sh, sc, y_dtype=np.uint16)
    assert np.array_equal(yb, bf16_bits(y32))


def test_adaln_groups_select_modulation_rows():
    x = f32(RNG.standard_normal((12, 32)))
    sh = f32(RNG.standard_normal((3, 32)))
    sc = f32(RNG.standard_normal((3, 32)))
    y = oracle.adaln_modulate(x, sh, sc, rows_per_group=4)
    for g in range(3):
        yg = oracle.adaln_modulate(x[4 * g:4 * g + 4], sh[g:g + 1], sc[g:g + 1])
        assert np.array_equal(y[4 * g:4 * g + 4], yg)
    yl = oracle.adaln_modulate(x, sh, sc, group=np.repeat(np.arange(3), 4))
    assert np.array_equal(y, yl)


def test_adaln_constant_row_gives_shift():
    x = f32(np.full((2, 64), 0.375))
    sh = f32(RNG.standard_normal((1, 64)))
    sc = f32(RNG.standard_normal((1, 64)))
    y = oracle.adaln_modulate(x, sh, sc)
    assert np.array_equal(y, np.broadcast_to(sh, y.shape))


# ----------------------------------------------------------------------------------
# gated residual
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("xd,hd", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_gated_identities(xd, hd):
    conv = {"f32": f32, "bf16": bf16_bits}
    x = conv[xd](RNG.standard_normal((7, 64)))
    h = conv[hd](RNG.standard_normal((7, 64)))
    zero_g = conv[xd](np.zeros((1, 64)))
    assert np.array_equal(oracle.gated_residual(x, h, zero_g), x)
    g = conv[xd](RNG.standard_normal((1, 64)))
    assert np.array_equal(oracle.gated_residual(x, conv[hd](np.zeros((7, 64))), g), x)


def test_gated_unit_gate_is_fp32_add():
    x = f32(RNG.standard_normal((5, 128)))
    h = f32(RNG.standard_normal((5, 128)))
    got = oracle.gated_residual(x, h, f32(np.ones((1, 128))))
    assert np.array_equal(got, x + h)  # numpy's fp32 add rounds once, to nearest even


def test_gated_bf16_unit_gate_is_rounded_sum():
    x = bf16_bits(RNG.standard_normal((5, 128)))
    h = bf16_bits(RNG.standard_normal((5, 128)))
    got = oracle.gated_residual(x, h, bf16_bits(np.ones((1, 128))))
    s = (as_f64(x) + as_f64(h)).astype(np.float32)  # exact sum, then fp32
    assert np.array_equal(got, bf16_bits(s))


def test_gated_fp32_stream_bf16_branch():
    # the chain's mixed form: fp32 stream, bf16 branch output, fp32 gate.  Every
    # bf16 value is exact in fp32, so x = 0 with gate = 1 leaves x = h exactly,
    # and x = -h/2 with gate = 1/2 leaves exactly 0
    hb = bf16_bits(RNG.standard_normal((6, 64)))
    h = as_f64(hb)
    got = oracle.gated_residual(f32(np.zeros((6, 64))), hb, f32(np.ones((1, 64))))
    assert np.array_equal(got, f32(h))
    got = oracle.gated_residual(f32(-h / 2), hb, f32(np.full((1, 64), 0.5)))
    assert np.array_equal(got, f32(np.zeros((6, 64))))


def test_gated_linear_in_gate_and_h():
    x = f32(np.zeros((4, 64)))
    h = f32(RNG.integers(-64, 64, (4, 64)) / 16.0)
    g = f32(RNG.integers(-64, 64, (1, 64)) / 16.0)
    # dyadic values: every product and sum is exact
    got = oracle.gated_residual(x, h, g)
    assert np.array_equal(got, f32(as_f64(g) * as_f64(h)))
    got2 = oracle.gated_residual(x, f32(2 * h), g)
    assert np.array_equal(got2, f32(2 * got))


# ----------------------------------------------------------------------------------
# SwiGLU
# ----------------------------------------------------------------------------------

def test_swiglu_matches_scipy_expit():
    a = RNG.standard_normal((9, 40)) * 3
    b = RNG.standard_normal((9, 40))
    gu = f32(np.concatenate([a, b], axis=1))
    got = as_f64(oracle.swiglu(gu))
    ad, bd = as_f64(gu[:, :40]), as_f64(gu[:, 40:])
    ref = ad * scipy.special.expit(ad) * bd
    assert np.max(np.abs(got - ref.astype(np.float32)) / ulp_f32(ref)) <= 1.0


def test_swiglu_unit_b_is_torch_silu():
    a = RNG.standard_normal((3, 64)) * 4
    gu = f32(np.concatenate([a, np.ones((3, 64))], axis=1))
    got = as_f64(oracle.swiglu(gu))
    ref = torch.nn.functional.silu(torch.from_numpy(as_f64(gu[:, :64]))).numpy()
    assert np.max(np.abs(got - ref.astype(np.float32)) / ulp_f32(ref)) <= 1.0


def test_swiglu_gate_is_first_half():
    gu = f32(np.concatenate([np.full((1, 8), 2.0), np.full((1, 8), 3.0)], axis=1))
    got = as_f64(oracle.swiglu(gu))
    assert np.allclose(got, 3.0 * 2.0 * scipy.special.expit(2.0), rtol=1e-7)
    assert not np.allclose(got, 2.0 * 3.0 * scipy.special.expit(3.0), rtol=1e-3)


def test_swiglu_zero_odd_part_and_limits():
    z = f32(RNG.standard_normal((1, 64)) * 5)
    one = f32(np.ones((1, 64)))
    pos = as_f64(oracle.swiglu(f32(np.concatenate([z, one], 1))))
    neg = as_f64(oracle.swiglu(f32(np.concatenate([-z, one], 1))))
    # silu(-z) = silu(z) - z
    assert np.max(np.abs(neg - (pos - as_f64(z)))) <= 4 * ulp_f32(np.abs(z).max())
    zero = as_f64(oracle.swiglu(f32(np.concatenate([np.zeros((1, 4)), np.ones((1, 4)) * 7], 1))))
    assert np.all(zero == 0)
    big = as_f64(oracle.swiglu(f32([[30.0, -30.0, 1.0, 1.0]])))
    assert big[0, 0] == 30.0
    assert -1e-10 < big[0, 1] < 0


# ----------------------------------------------------------------------------------
# QK RMSNorm + 3D RoPE
# ----------------------------------------------------------------------------------

SPLIT_T = (16, 24, 24)


def qk_inputs(rows=6, heads=4, Dh=64, seed=0):
    r = np.random.default_rng(seed)
    q = f32(r.standard_normal((rows, heads, Dh)))
    k = f32(r.standard_normal((rows, heads, Dh)))
    qw = f32(1 + 0.05 * r.standard_normal(Dh))
    kw = f32(1 + 0.05 * r.standard_normal(Dh))
    return q, k, qw, kw


def test_rope_inv_freq_values():
    f = oracle.rope_inv_freq(4, 4, 8, theta=10000.0)
    # chunk sizes 4/4/8: pairs [t0 t1 | h0 h1 | w0 w1 w2 w3]
    expect = [1.0, 0.01, 1.0, 0.01, 1.0, 0.1, 0.01, 0.001]
    assert np.array_equal(f, np.array(expect, np.float32))


def test_rmsnorm_matches_torch_rms_norm_at_origin():
    q, k, _, _ = qk_inputs()
    ones = f32(np.ones(64))
    pos = np.zeros((6, 3), np.int32)
    qo, ko = oracle.qk_rmsnorm_rope3d(q, k, ones, ones, pos, SPLIT_T, eps=1e-6)
    for inp, out in ((q, qo), (k, ko)):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(as_f64(inp)), (64,),
                                           eps=float(np.float32(1e-6))).numpy()
        assert np.max(np.abs(as_f64(out) - ref.astype(np.float32)) / ulp_f32(ref)) <= 1.0


def test_rmsnorm_unit_rms_and_weights():
    q, k, qw, kw = qk_inputs()
    pos = np.zeros((6, 3), np.int32)
    ones = f32(np.ones(64))
    qo, _ = oracle.qk_rmsnorm_rope3d(q, k, ones, ones, pos, SPLIT_T, eps=1e-6)
    m = (as_f64(q) ** 2).mean(axis=2)
    ms = (as_f64(qo) ** 2).mean(axis=2)
    assert np.allclose(ms, m / (m + np.float64(np.float32(1e-6))), rtol=1e-6)
    # separate q and k weights, shared across heads
    qo2, ko2 = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, pos, SPLIT_T)
    _, ko1 = oracle.qk_rmsnorm_rope3d(q, k, ones, ones, pos, SPLIT_T)
    # one rounding of the weighted value vs a rounded unweighted value times w: <= 2 ulps
    assert np.max(np.abs(as_f64(qo2) - as_f64(qo) * as_f64(qw)) / ulp_f32(as_f64(qo2))) <= 2.0
    assert np.max(np.abs(as_f64(ko2) - as_f64(ko1) * as_f64(kw)) / ulp_f32(as_f64(ko2))) <= 2.0
    # and the weight is not applied to the wrong tensor
    assert np.max(np.abs(as_f64(ko2) - as_f64(ko1) * as_f64(qw)) / ulp_f32(as_f64(ko2))) > 100


def complex_rope_reference(u, pos, split, theta, pairing="interleaved"):
    """RoPE as complex multiplication (RoFormer sec. 3.4.2 complex form), per axis chunk,
    with the frequency table computed here in float64 and rounded to fp32."""
    rows, heads, Dh = u.shape
    out = np.array(u, dtype=np.float64)
    start = 0
    for c, dc in enumerate(split):
        freqs = (theta ** (-np.arange(0, dc, 2, dtype=np.float64) / dc)).astype(np.float32)
        ang = (pos[:, c].astype(np.float32)[:, None] * freqs[None, :]).astype(np.float64)  # [rows, dc/2]
        rot = np.exp(1j * ang)[:, None, :]
        chunk = out[:, :, start:start + dc]
        if pairing == "interleaved":
            z = chunk[..., 0::2] + 1j * chunk[..., 1::2]
            z = z * rot
            chunk[..., 0::2] = z.real
            chunk[..., 1::2] = z.imag
        else:
            z = chunk[..., :dc // 2] + 1j * chunk[..., dc // 2:]
            z = z * rot
            chunk[..., :dc // 2] = z.real
            chunk[..., dc // 2:] = z.imag
        out[:, :, start:start + dc] = chunk
        start += dc
    return out


@pytest.mark.parametrize("pairing", ["interleaved", "half_split"])
def test_rope_matches_complex_form(pairing):
    rows = 40
    q, k, qw, kw = qk_inputs(rows=rows, seed=3)
    pos = oracle.positions(rows, 2, 3, 5, 10)
    pos[:, 0] += 37  # larger angles too
    pr = oracle.PAIR_INTERLEAVED if pairing == "interleaved" else oracle.PAIR_HALF_SPLIT
    ones = f32(np.ones(64))
    zero = np.zeros_like(pos)
    qn, kn = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, zero, SPLIT_T, pairing=pr)
    qo, ko = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, pos, SPLIT_T, pairing=pr)
    # reference rotates the oracle's own normalised values; compare within 2 fp32 ulps
    # of the pair norm (rounding of the normalised input + rounding of the output)
    for nrm, out in ((qn, qo), (kn, ko)):
        ref = complex_rope_reference(as_f64(nrm), pos, SPLIT_T, 10000.0, pairing)
        scale = np.abs(as_f64(nrm)).max()
        assert np.max(np.abs(as_f64(out) - ref)) <= 3 * ulp_f32(scale)
    del ones


def test_rope_position_zero_and_audio_identity():
    q, k, qw, kw = qk_inputs(rows=3)
    zero = np.zeros((3, 3), np.int32)
    base_q, base_k = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, zero, SPLIT_T)
    audio = np.array([[5, 0, 0], [9, 0, 0], [1, 0, 0]], np.int32)
    aq, ak = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, audio, SPLIT_T)
    # h and w chunks (dims 16..63) untouched, t chunk rotated
    assert np.array_equal(aq[..., 16:], base_q[..., 16:])
    assert np.array_equal(ak[..., 16:], base_k[..., 16:])
    assert not np.array_equal(aq[..., :16], base_q[..., :16])


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_axis_drives_only_its_chunk(axis):
    q, k, qw, kw = qk_inputs(rows=2)
    zero = np.zeros((2, 3), np.int32)
    p = zero.copy()
    p[:, axis] = [3, 7]
    bq, _ = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, zero, SPLIT_T)
    oq, _ = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, p, SPLIT_T)
    bounds = [(0, 16), (16, 40), (40, 64)]
    for c, (s, e) in enumerate(bounds):
        same = np.array_equal(oq[..., s:e], bq[..., s:e])
        assert same == (c != axis)


def test_rope_preserves_pair_norms():
    q, k, qw, kw = qk_inputs(rows=20, seed=5)
    pos = oracle.positions(20, 2, 3, 4, 6)
    zero = np.zeros_like(pos)
    bq, _ = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, zero, SPLIT_T)
    oq, _ = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, pos, SPLIT_T)
    nb = np.hypot(as_f64(bq)[..., 0::2], as_f64(bq)[..., 1::2])
    no = np.hypot(as_f64(oq)[..., 0::2], as_f64(oq)[..., 1::2])
    assert np.max(np.abs(nb - no)) <= 2 * ulp_f32(nb.max())


def test_rope_relative_position_property():
    # <R(p) q, R(p') k> depends only on p - p' on every axis (exact angles, mode 1)
    q, k, qw, kw = qk_inputs(rows=1, heads=1, seed=7)
    ones = f32(np.ones(64))

    def rot(v, p):
        o, _ = oracle.qk_rmsnorm_rope3d(v, v, ones, ones, np.array([p], np.int32), SPLIT_T,
                                        angle_mode=1)
        return as_f64(o)[0, 0]

    d0 = rot(q, [3, 1, 4]) @ rot(k, [1, 5, 2])
    d1 = rot(q, [13, 21, 9]) @ rot(k, [11, 25, 7])
    assert abs(d0 - d1) <= 64 * 4 * 2 ** -24 * 4


def test_rope_composition():
    # R(p) R(p') = R(p + p'): rotating the (unit-RMS) output again is one rotation by the sum
    q, k, _, _ = qk_inputs(rows=4, heads=2, seed=9)
    ones = f32(np.ones(64))
    p1 = np.array([[1, 2, 3], [4, 5, 6], [0, 1, 0], [7, 0, 2]], np.int32)
    p2 = np.array([[2, 2, 1], [0, 3, 9], [5, 5, 5], [1, 1, 1]], np.int32)
    a, _ = oracle.qk_rmsnorm_rope3d(q, k, ones, ones, p1, SPLIT_T, eps=0.0, angle_mode=1)
    b, _ = oracle.qk_rmsnorm_rope3d(a, a, ones, ones, p2, SPLIT_T, eps=0.0, angle_mode=1)
    c, _ = oracle.qk_rmsnorm_rope3d(q, k, ones, ones, p1 + p2, SPLIT_T, eps=0.0, angle_mode=1)
    assert np.max(np.abs(as_f64(b) - as_f64(c))) < 2e-6


def test_rope_hand_value():
    # chunk t of size 4: pair 1 has frequency 10000^(-2/4) = 0.01, so t = 100 rotates it by
    # (almost exactly) 1 radian; a unit vector along the pair's first element goes to
    # (cos 1, sin 1) scaled by the RMS normalisation.
    Dh = 8
    v = np.zeros((1, 1, Dh), np.float32)
    v[0, 0, 2] = 1.0  # first element of pair 1 of the t chunk
    ones = f32(np.ones(Dh))
    o, _ = oracle.qk_rmsnorm_rope3d(v, v, ones, ones, np.array([[100, 0, 0]], np.int32),
                                    (4, 2, 2), eps=0.0)
    s = math.sqrt(Dh)  # rms of the input is 1/sqrt(8)
    ang = float(np.float32(100.0) * np.float32(0.01))
    assert abs(o[0, 0, 2] - s * math.cos(ang)) < 1e-6
    assert abs(o[0, 0, 3] - s * math.sin(ang)) < 1e-6  # counter-clockwise rotation
    assert np.all(o[0, 0, [0, 1, 4, 5, 6, 7]] == 0)


def test_rope_fp32_angle_vs_exact_angle_tiny():
    q, k, qw, kw = qk_inputs(rows=112, seed=11)
    pos = oracle.positions(112, 2, 6, 8, 16)
    a, b = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, pos, SPLIT_T, angle_mode=0)
    c, d = oracle.qk_rmsnorm_rope3d(q, k, qw, kw, pos, SPLIT_T, angle_mode=1)
    from tolerance import err_over_tol
    assert err_over_tol(a, c, "f32") <= 1.0 and err_over_tol(b, d, "f32") <= 1.0


# ----------------------------------------------------------------------------------
# fused gated residual + AdaLN, residual difference
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("xd,hd", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_fused_gated_adaln_equals_composition(xd, hd):
    conv = {"f32": f32, "bf16": bf16_bits}
    x = conv[xd](RNG.standard_normal((6, 64)))
    h = conv[hd](RNG.standard_normal((6, 64)))
    g = conv[xd](RNG.standard_normal((1, 64)) * 0.5)
    sh = conv[xd](RNG.standard_normal((1, 64)) * 0.1)
    sc = conv[xd](RNG.standard_normal((1, 64)) * 0.1)
    ydt = np.uint16
    x1, y1 = oracle.gated_residual_adaln(x, h, g, sh, sc, y_dtype=ydt)
    x2 = oracle.gated_residual(x, h, g)
    y2 = oracle.adaln_modulate(x2, sh, sc, y_dtype=ydt)
    assert np.array_equal(x1, x2) and np.array_equal(y1, y2)


def test_residual_l1():
    prev = f32(RNG.standard_normal((5, 16)))
    assert oracle.residual_l1(prev, prev)[0] == 0.0
    num, den = oracle.residual_l1(f32(2 * prev), prev)
    assert num == pytest.approx(den, rel=1e-12)
    assert den == pytest.approx(np.abs(as_f64(prev)).sum(), rel=1e-12)
    cur = f32(RNG.standard_normal((5, 16)))
    num, _ = oracle.residual_l1(cur, prev)
    assert num == pytest.approx(np.abs(as_f64(cur) - as_f64(prev)).sum(), rel=1e-12)


# ----------------------------------------------------------------------------------
# block-sparse attention router (SubBlock)
# ----------------------------------------------------------------------------------

def pair_mean_logits(q, k, block):
    """Average of q_a . k_b over every token pair (a in query block i, b in key
    block j), by explicit pairs -- no pooling -- for each head."""
    qf, kf = as_f64(q), as_f64(k)
    rows, heads, _ = qf.shape
    nb = (rows + block - 1) // block
    out = np.zeros((heads, nb, nb))
    for h in range(heads):
        logits = qf[:, h, :] @ kf[:, h, :].T          # every token pair
        for i in range(nb):
            for j in range(nb):
                out[h, i, j] = logits[i * block:(i + 1) * block, j * block:(j + 1) * block].mean()
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_subblock_score_is_mean_pair_logit(dtype):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((37, 2, 8))
    k = rng.standard_normal((37, 2, 8)) + 0.3
    if dtype == "f32":
        q, k = f32(q), f32(k)
    else:
        q, k = bf16_bits(q), bf16_bits(k)
    pq = oracle.subblock_pool(q, 10)                   # blocks of 10, 10, 10, 7
    pk = oracle.subblock_pool(k, 10)
    assert pq.shape == (2, 4, 8)
    s = oracle.subblock_scores(pq, pk)
    ref = pair_mean_logits(q, k, 10)
    assert np.abs(s - ref).max() <= 1e-12 * np.abs(ref).max()


def test_subblock_pool_of_constant_blocks():
    # every token of block b holds the value b + 1 (short last block included)
    x = np.zeros((23, 1, 4), np.float32)
    for r in range(23):
        x[r] = r // 8 + 1
    p = oracle.subblock_pool(x, 8)
    assert np.array_equal(p[0], np.repeat(np.array([[1.0], [2.0], [3.0]]), 4, axis=1))


def test_subblock_keep_closed_form():
    # nb - floor(sparsity * nb), from the tenth step on
    assert oracle.subblock_keep(978, 0.80, 10) == 978 - 782        # 782.4 skipped
    assert oracle.subblock_keep(978, 0.75, 10) == 978 - 733        # 733.5 skipped
    assert oracle.subblock_keep(1924, 0.80, 50) == 1924 - 1539     # 1539.2 skipped
    assert oracle.subblock_keep(1924, 0.75, 11) == 1924 - 1443     # 1443 exactly
    assert oracle.subblock_keep(978, 0.80, 9) == 978               # dense before step 10
    assert oracle.subblock_keep(978, 0.80, 1) == 978
    assert oracle.subblock_keep(32, 0.0, 10) == 32


def test_subblock_select_planted_ranking():
    rng = np.random.default_rng(3)
    nb = 40
    s = np.stack([rng.permutation(nb).astype(np.float64) for _ in range(6)]).reshape(2, 3, nb)
    kv = oracle.subblock_select(s, 7)
    for h in range(2):
        for i in range(3):
            want = np.sort(np.nonzero(s[h, i] >= nb - 7)[0])   # the 7 largest values 33..39
            assert np.array_equal(kv[h, i], want)


def test_subblock_select_matches_torch_topk():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((3, 5, 97))
    kv = oracle.subblock_select(s, 20)
    top = torch.topk(torch.tensor(s), 20, dim=-1).indices.sort(dim=-1).values.numpy()
    assert np.array_equal(kv, top.astype(np.int32))


def test_subblock_select_ties_take_lower_index():
    s = np.zeros((1, 2, 10))
    s[0, 1, :] = [1, 5, 5, 0, 5, 5, 2, 5, 0, 0]
    kv = oracle.subblock_select(s, 3)
    assert kv[0, 0].tolist() == [0, 1, 2]                 # all equal: lowest indices
    assert kv[0, 1].tolist() == [1, 2, 4]                 # five 5s tie for three places


def test_subblock_route_planted_blocks():
    # query tokens all e0; key block j tokens all alpha_j * e0, so the pair-mean
    # logit of every (i, j) is alpha_j.  The short last block has the largest
    # alpha: a sum (not mean) pooling or a full-block divisor would demote it.
    block, rows = 16, 16 * 5 + 3
    alpha = [0.25, 2.0, -1.0, 0.5, 1.0, 4.0]
    q = np.zeros((rows, 2, 128), np.float32)
    k = np.zeros((rows, 2, 128), np.float32)
    q[:, :, 0] = 1.0
    for r in range(rows):
        k[r, 0, 0] = alpha[r // block]
        k[r, 1, 0] = -alpha[r // block]                   # second head ranks in reverse
    kv, s = oracle.subblock_route(bf16_bits(q), bf16_bits(k), block, 0.5, 10)
    assert s.shape == (2, 6, 6) and kv.shape == (2, 6, 3)
    assert np.array_equal(s[0], np.tile(alpha, (6, 1)))
    for i in range(6):
        assert kv[0, i].tolist() == [1, 4, 5]             # 2.0, 1.0, 4.0
        assert kv[1, i].tolist() == [0, 2, 3]             # -0.25, 1.0, -0.5
    kv_dense, _ = oracle.subblock_route(bf16_bits(q), bf16_bits(k), block, 0.5, 9)
    assert kv_dense.shape == (2, 6, 6) and (kv_dense == np.arange(6)).all()
