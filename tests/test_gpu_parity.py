"""GPU parity: every libh3fused entry point against the CPU oracle on the same
seeded inputs, element by element, at sizes the oracle finishes in seconds
(several tiles plus a ragged tail) and, at the full 5 s / 10 s token shapes,
on sampled rows.  Tolerances by output type (tests/tolerance.py):
fp32 |err| <= 1e-6 + 1e-5 |ref|, bf16 |err| <= 2^-7 |ref| + 1e-3.
Integer work (positions) is compared bit for bit."""
import numpy as np
import pytest
import torch

import h3gen
import oracle
from gpu_util import DEV, dev_tensor, from_np, host, kind, rows_of, sample_rows, to_np
from tolerance import assert_close

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("video_diffusion_transformer_h3f_amd")

TINY = dict(T=2, H=6, W=8, A=16, D=256, heads=4, Dh=64, split=(16, 24, 24), F=512)
S5 = dict(T=31, H=48, W=84, A=128, D=5120, heads=40, Dh=128, split=(32, 48, 48), F=13824)
S10 = dict(S5, T=61, A=256)


def n_tokens(c):
    return c["T"] * c["H"] * c["W"] + c["A"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h3.lib()
    h3gen.dev_lib()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------------------------
# generator: device values are the host values, bit for bit
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_device_generator_matches_host(dtype):
    t = dev_tensor("x", 257, 520, dtype, row_stride=528)
    assert np.array_equal(to_np(t), host("x", 257, 520, dtype))
    t = dev_tensor("q_weight", 3, 128, dtype)
    assert np.array_equal(to_np(t), host("q_weight", 3, 128, dtype))


# ------------------------------------------------------------------------------------
# positions (integer, exact)
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [TINY, S5, S10], ids=["tiny", "5s", "10s"])
def test_positions_exact(cfg):
    n = n_tokens(cfg)
    pos = torch.empty(n, 3, dtype=torch.int32, device=DEV)
    rope = h3.make_rope(cfg["T"], cfg["H"], cfg["W"], cfg["A"], cfg["split"])
    h3.h3f_rope3d_positions(pos, rope)
    assert np.array_equal(to_np(pos), oracle.positions(n, cfg["T"], cfg["H"], cfg["W"], cfg["A"]))


def test_positions_offset_wraps():
    c = TINY
    n = 3 * n_tokens(c) + 5
    pos = torch.empty(n, 3, dtype=torch.int32, device=DEV)
    h3.h3f_rope3d_positions(pos, h3.make_rope(c["T"], c["H"], c["W"], c["A"], c["split"],
                                              token_offset=41))
    ref = oracle.positions(n, c["T"], c["H"], c["W"], c["A"], token_offset=41)
    assert np.array_equal(to_np(pos), ref)


# ------------------------------------------------------------------------------------
# gated residual
# ------------------------------------------------------------------------------------

GATED_CASES = [
    # (rows, hidden, x dtype, h dtype, groups, x row stride pad, h row stride pad)
    (112, 256, "f32", "f32", 1, 0, 0),
    (1001, 5120, "bf16", "bf16", 1, 0, 0),
    (777, 5120, "f32", "bf16", 1, 0, 0),
    (300, 3072, "bf16", "bf16", 3, 8, 16),
    (97, 136, "bf16", "bf16", 97, 0, 0),
    (1, 8, "bf16", "bf16", 1, 0, 0),
    (5, 4, "f32", "f32", 1, 4, 0),
]


@pytest.mark.parametrize("case", GATED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_gated_residual(case):
    rows, D, xd, hd, groups, xpad, hpad = case
    x = dev_tensor("x", rows, D, xd, row_stride=D + xpad)
    h = dev_tensor("h", rows, D, hd, row_stride=D + hpad)
    gate = dev_tensor("gate", groups, D, xd)
    rpg = -(-rows // groups)
    h3.h3f_gated_residual(x, h, gate, rows_per_group=rpg)
    ref = oracle.gated_residual(host("x", rows, D, xd), host("h", rows, D, hd),
                                host("gate", groups, D, xd), rows_per_group=rpg)
    assert_close(to_np(x), ref, kind(xd), "gated")


def test_gated_zero_gate_is_exact_identity():
    x = dev_tensor("x", 300, 5120, "bf16")
    before = to_np(x)
    h3.h3f_gated_residual(x, dev_tensor("h", 300, 5120, "bf16"),
                          torch.zeros(5120, dtype=torch.bfloat16, device=DEV))
    assert np.array_equal(to_np(x), before)


# ------------------------------------------------------------------------------------
# SwiGLU
# ------------------------------------------------------------------------------------

SWIGLU_CASES = [(112, 512, "f32"), (501, 13824, "bf16"), (64, 8320, "bf16"), (33, 1000, "bf16"),
                (7, 4, "f32"), (1, 8, "bf16")]


@pytest.mark.parametrize("case", SWIGLU_CASES, ids=lambda c: "x".join(map(str, c)))
def test_swiglu_packed(case):
    rows, F, dt = case
    gu = dev_tensor("gate_up", rows, 2 * F, dt)
    out = torch.empty(rows, F, dtype=gu.dtype, device=DEV)
    h3.h3f_swiglu(out, gu)
    ref = oracle.swiglu(host("gate_up", rows, 2 * F, dt))
    assert_close(to_np(out), ref, kind(dt), "swiglu")


def test_swiglu_separate_strided_and_in_place():
    rows, F = 129, 1024
    a = dev_tensor("gate_up", rows, F, "bf16", row_stride=F + 64)
    b = dev_tensor("h", rows, F, "bf16", row_stride=F + 8)
    ref_in = np.concatenate([host("gate_up", rows, F, "bf16"), host("h", rows, F, "bf16")], 1)
    ref = oracle.swiglu(ref_in)
    out = torch.empty(rows, F, dtype=torch.bfloat16, device=DEV)
    h3.h3f_swiglu(out, a, b)
    assert_close(to_np(out), ref, "bf16", "swiglu separate")
    h3.h3f_swiglu(a, a, b)  # in place over the gate operand
    assert_close(to_np(a), ref, "bf16", "swiglu in place")


def test_swiglu_extremes():
    a = torch.tensor([[0.0, 30.0, -30.0, -100.0, 100.0, 1e-3, -1e-3, 5.0]], device=DEV)
    b = torch.tensor([[3.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, -2.0]], device=DEV)
    out = torch.empty_like(a)
    h3.h3f_swiglu(out, a, b)
    ref = oracle.swiglu(np.concatenate([to_np(a), to_np(b)], 1))
    assert_close(to_np(out), ref, "f32", "swiglu extremes")
    assert to_np(out)[0, 0] == 0.0


# ------------------------------------------------------------------------------------
# AdaLN modulate
# ------------------------------------------------------------------------------------

ADALN_CASES = [
    # rows, hidden, x dtype, y dtype, groups
    (112, 256, "f32", "f32", 1),
    (1001, 5120, "bf16", "bf16", 1),
    (513, 5120, "f32", "bf16", 1),
    (300, 3072, "bf16", "bf16", 1),
    (300, 4096, "bf16", "bf16", 4),
    (200, 6144, "bf16", "bf16", 1),
    (65, 16384, "bf16", "bf16", 1),
    (65, 8192, "f32", "f32", 1),
    (65, 8192, "f32", "bf16", 1),
    (33, 8, "bf16", "bf16", 33),
    (17, 4, "f32", "f32", 1),
    (9, 1000, "bf16", "bf16", 1),
]


@pytest.mark.parametrize("case", ADALN_CASES, ids=lambda c: "x".join(map(str, c)))
def test_adaln(case):
    rows, D, xd, yd, groups = case
    x = dev_tensor("x", rows, D, xd)
    sh = dev_tensor("shift", groups, D, xd)
    sc = dev_tensor("scale", groups, D, xd)
    y = torch.empty(rows, D, dtype=torch.bfloat16 if yd == "bf16" else torch.float32, device=DEV)
    rpg = -(-rows // groups)
    h3.h3f_adaln_modulate(y, x, sh, sc, eps=1e-6, rows_per_group=rpg)
    ref = oracle.adaln_modulate(host("x", rows, D, xd), host("shift", groups, D, xd),
                                host("scale", groups, D, xd), eps=1e-6,
                                y_dtype=np.uint16 if yd == "bf16" else np.float32,
                                rows_per_group=rpg)
    assert_close(to_np(y), ref, kind(yd), "adaln")


ADALN_AFFINE_CASES = [
    # rows, hidden, x dtype, y dtype, groups
    (112, 256, "f32", "f32", 1),
    (1001, 5120, "bf16", "bf16", 1),    # modulation and gamma/beta staged in LDS
    (513, 5120, "f32", "bf16", 3),      # read through the caches
    (65, 16384, "bf16", "bf16", 1),     # too large to stage
    (300, 3072, "bf16", "bf16", 300),   # per-token modulation
    (17, 4, "f32", "f32", 1),
]


@pytest.mark.parametrize("case", ADALN_AFFINE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_adaln_affine(case):
    rows, D, xd, yd, groups = case
    x = dev_tensor("x", rows, D, xd)
    gm, bt = dev_tensor("ln_gamma", 1, D, xd).view(D), dev_tensor("ln_beta", 1, D, xd).view(D)
    sh = dev_tensor("shift", groups, D, xd)
    sc = dev_tensor("scale", groups, D, xd)
    y = torch.empty(rows, D, dtype=torch.bfloat16 if yd == "bf16" else torch.float32, device=DEV)
    rpg = -(-rows // groups)
    h3.h3f_adaln_affine_modulate(y, x, gm, bt, sh, sc, eps=1e-6, rows_per_group=rpg)
    ref = oracle.adaln_affine_modulate(host("x", rows, D, xd), host("ln_gamma", 1, D, xd),
                                       host("ln_beta", 1, D, xd), host("shift", groups, D, xd),
                                       host("scale", groups, D, xd), eps=1e-6,
                                       y_dtype=np.uint16 if yd == "bf16" else np.float32,
                                       rows_per_group=rpg)
    assert_close(to_np(y), ref, kind(yd), "adaln affine")


def test_adaln_affine_identity_parameters_match_plain_adaln():
    # gamma = 1, beta = 0: bit-identical to the plain operator
    rows, D = 257, 5120
    x = dev_tensor("x", rows, D, "bf16")
    sh, sc = dev_tensor("shift", 1, D, "bf16"), dev_tensor("scale", 1, D, "bf16")
    y0, y1 = torch.empty_like(x), torch.empty_like(x)
    h3.h3f_adaln_modulate(y0, x, sh, sc)
    h3.h3f_adaln_affine_modulate(y1, x, torch.ones(D, dtype=torch.bfloat16, device=DEV),
                                 torch.zeros(D, dtype=torch.bfloat16, device=DEV), sh, sc)
    assert torch.equal(y0, y1)


def test_adaln_in_place_strided_and_offset_rows():
    rows, D = 400, 5120
    x = dev_tensor("x", rows, D, "bf16", row_stride=D + 128)
    sh, sc = dev_tensor("shift", 1, D, "bf16"), dev_tensor("scale", 1, D, "bf16")
    ref = oracle.adaln_modulate(host("x", rows, D, "bf16"), host("shift", 1, D, "bf16"),
                                host("scale", 1, D, "bf16"))
    h3.h3f_adaln_modulate(x, x, sh, sc)
    assert_close(to_np(x), ref, "bf16", "adaln in place")


def test_adaln_constant_rows_give_shift():
    # hidden a power of two and a dyadic constant: the mean is exact, so the output is shift
    D = 1024
    x = torch.full((16, D), 0.375, dtype=torch.bfloat16, device=DEV)
    sh, sc = dev_tensor("shift", 1, D, "bf16"), dev_tensor("scale", 1, D, "bf16")
    y = torch.empty_like(x)
    h3.h3f_adaln_modulate(y, x, sh, sc)
    assert np.array_equal(to_np(y), np.broadcast_to(to_np(sh), (16, D)))


# ------------------------------------------------------------------------------------
# fused gated residual + AdaLN
# ------------------------------------------------------------------------------------

FUSED_CASES = [(112, 256, "f32", "f32", "f32"), (1001, 5120, "bf16", "bf16", "bf16"),
               (513, 5120, "f32", "bf16", "bf16"), (200, 3072, "f32", "f32", "bf16"),
               (64, 4096, "f32", "bf16", "f32"),
               # widest rows, and one row (the other wavefronts of its workgroup
               # only take part in the modulation staging)
               (65, 16384, "bf16", "bf16", "bf16"), (33, 8192, "f32", "f32", "f32"),
               (1, 5120, "bf16", "bf16", "bf16"), (3, 5120, "f32", "bf16", "bf16")]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_gated_residual_adaln(case):
    rows, D, xd, hd, yd = case
    x = dev_tensor("x", rows, D, xd)
    h = dev_tensor("h", rows, D, hd)
    gt, sh, sc = (dev_tensor(n, 1, D, xd) for n in ("gate", "shift", "scale"))
    y = torch.empty(rows, D, dtype=torch.bfloat16 if yd == "bf16" else torch.float32, device=DEV)
    h3.h3f_gated_residual_adaln(x, h, gt, sh, sc, y)
    rx, ry = oracle.gated_residual_adaln(
        host("x", rows, D, xd), host("h", rows, D, hd), *(host(n, 1, D, xd) for n in
                                                          ("gate", "shift", "scale")),
        y_dtype=np.uint16 if yd == "bf16" else np.float32)
    assert_close(to_np(x), rx, kind(xd), "fused x")
    assert_close(to_np(y), ry, kind(yd), "fused y")


# ------------------------------------------------------------------------------------
# QK RMSNorm + 3D RoPE
# ------------------------------------------------------------------------------------

def _qk_case(cfg, dtype, rows, offset=0, pairing=h3.H3F_ROPE_INTERLEAVED, packed=False,
             in_place=False, positions=False, audio_aligned=False):
    H, Dh = cfg["heads"], cfg["Dh"]
    if packed:
        qkv = torch.empty(rows, 3, H, Dh, dtype=torch.bfloat16 if dtype == "bf16" else
                          torch.float32, device=DEV)
        for i, n in enumerate(("q", "k", "v")):
            h3gen.fill_device(qkv.view(rows, 3 * H * Dh)[:, i * H * Dh:(i + 1) * H * Dh], n,
                              row0=offset)
        q, k = qkv[:, 0], qkv[:, 1]
    else:
        q = torch.empty(rows, H * Dh, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                        device=DEV)
        k = torch.empty_like(q)
        h3gen.fill_device(q, "q", row0=offset)
        h3gen.fill_device(k, "k", row0=offset)
        q, k = q.view(rows, H, Dh), k.view(rows, H, Dh)
    qw = dev_tensor("q_weight", 1, Dh, dtype).view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, dtype).view(Dh)
    ids = np.arange(offset, offset + rows)
    refq = host("q", ids, H * Dh, dtype).reshape(rows, H, Dh)
    refk = host("k", ids, H * Dh, dtype).reshape(rows, H, Dh)
    v_before = to_np(qkv[:, 2]) if packed else None
    pos_np = oracle.positions(rows, cfg["T"], cfg["H"], cfg["W"], cfg["A"], token_offset=offset)
    if audio_aligned:
        # the other reading of the audio axis: audio token k shares the time index of
        # the video frame it plays under, t = floor(k * T / n_audio), at h = w = 0
        n_video = cfg["T"] * cfg["H"] * cfg["W"]
        p = (offset + np.arange(rows)) % (n_video + cfg["A"])
        audio = p >= n_video
        pos_np[audio, 0] = (p[audio] - n_video) * cfg["T"] // cfg["A"]
        assert audio.any() and (pos_np[audio, 1:] == 0).all()
    pos_t = from_np(pos_np) if positions else None
    rope = h3.make_rope(cfg["T"], cfg["H"], cfg["W"], cfg["A"], cfg["split"],
                        token_offset=0 if positions else offset, positions=pos_t,
                        pairing=pairing)
    if in_place:
        qo, ko = q, k
    else:
        qo, ko = torch.empty(rows, H, Dh, dtype=q.dtype, device=DEV), torch.empty(
            rows, H, Dh, dtype=q.dtype, device=DEV)
    h3.h3f_qk_rmsnorm_rope3d(qo, ko, q, k, qw, kw, rope, eps=1e-6)
    rq, rk = oracle.qk_rmsnorm_rope3d(refq, refk, to_np(qw), to_np(kw), pos_np, cfg["split"],
                                      eps=1e-6, pairing=pairing)
    assert_close(to_np(qo), rq, kind(dtype), "q_out")
    assert_close(to_np(ko), rk, kind(dtype), "k_out")
    if packed:
        assert np.array_equal(to_np(qkv[:, 2]), v_before), "v must be untouched"


def test_qk_tiny_fp32():
    _qk_case(TINY, "f32", n_tokens(TINY))


def test_qk_tiny_fp32_offset_wrap():
    _qk_case(TINY, "f32", 2 * n_tokens(TINY) + 3, offset=50)


def test_qk_bf16_5s_head_layout_rows():
    _qk_case(S5, "bf16", 777)


def test_qk_bf16_audio_and_last_video_rows():
    # rows around the video/audio boundary of the 5 s grid (large t, h, w)
    n_video = S5["T"] * S5["H"] * S5["W"]
    _qk_case(S5, "bf16", 300, offset=n_video - 172)


def test_qk_fp32_large_positions():
    # 10 s grid, fp32 I/O: angles up to 255 rad for audio t, 83 for w
    c = dict(S10, Dh=128, heads=8)
    n_video = c["T"] * c["H"] * c["W"]
    _qk_case(c, "f32", 512, offset=n_video - 256)


def test_qk_packed_strided_in_place():
    _qk_case(S5, "bf16", 200, offset=12345, packed=True, in_place=True)


def test_qk_packed_strided_out_of_place():
    _qk_case(S5, "bf16", 200, offset=999, packed=True)


def test_qk_explicit_positions():
    _qk_case(S5, "bf16", 150, offset=124900, positions=True)


def test_qk_explicit_positions_audio_aligned_to_frames():
    # explicit positions carry a different audio placement through the same kernel
    n_video = S5["T"] * S5["H"] * S5["W"]
    _qk_case(S5, "bf16", 400, offset=n_video - 200, positions=True, audio_aligned=True)


def test_qk_half_split_pairing():
    c = dict(S5, heads=6)
    _qk_case(c, "bf16", 100, offset=5000, pairing=h3.H3F_ROPE_HALF_SPLIT)
    c2 = dict(TINY, split=(16, 16, 32))
    _qk_case(c2, "f32", 112, pairing=h3.H3F_ROPE_HALF_SPLIT)


def test_qk_other_head_dims():
    _qk_case(dict(TINY, Dh=64, split=(16, 24, 24), heads=3), "bf16", 50, offset=7)
    _qk_case(dict(TINY, Dh=256, split=(64, 96, 96), heads=5), "bf16", 40, offset=3)
    _qk_case(dict(TINY, Dh=32, split=(8, 8, 16), heads=2), "f32", 30)


def test_qk_head_dim_limits():
    # the largest heads the kernel takes (one head per wavefront: 64 lanes x 8 bf16)
    # and the smallest fp32 head (head_dim / 4 = 4 lanes per head, 16 heads per wavefront)
    _qk_case(dict(TINY, Dh=512, split=(128, 192, 192), heads=3), "bf16", 37, offset=11)
    _qk_case(dict(TINY, Dh=512, split=(128, 192, 192), heads=2), "bf16", 21, offset=90,
             pairing=h3.H3F_ROPE_HALF_SPLIT)
    _qk_case(dict(TINY, Dh=16, split=(4, 4, 8), heads=7), "f32", 45, offset=60)


# ------------------------------------------------------------------------------------
# full 5 s shapes (the measured workload), sampled rows
# ------------------------------------------------------------------------------------

def test_full_5s_shape_all_ops_sampled():
    c = S5
    N, D, F, H, Dh = n_tokens(c), c["D"], c["F"], c["heads"], c["Dh"]
    n_video = N - c["A"]
    idx = sample_rows(N, n_video)
    x = dev_tensor("x", N, D, "bf16")
    sh, sc, gt = (dev_tensor(n, 1, D, "bf16") for n in ("shift", "scale", "gate"))
    y = torch.empty_like(x)
    h3.h3f_adaln_modulate(y, x, sh, sc)
    ref_y = oracle.adaln_modulate(host("x", idx, D, "bf16"), host("shift", 1, D, "bf16"),
                                  host("scale", 1, D, "bf16"))
    assert_close(rows_of(y, idx), ref_y, "bf16", "adaln 5s")
    del y
    h = dev_tensor("h", N, D, "bf16")
    h3.h3f_gated_residual(x, h, gt)
    ref_x = oracle.gated_residual(host("x", idx, D, "bf16"), host("h", idx, D, "bf16"),
                                  host("gate", 1, D, "bf16"))
    assert_close(rows_of(x, idx), ref_x, "bf16", "gated 5s")
    del x, h
    gu = dev_tensor("gate_up", N, 2 * F, "bf16")
    act = torch.empty(N, F, dtype=torch.bfloat16, device=DEV)
    h3.h3f_swiglu(act, gu)
    ref_a = oracle.swiglu(host("gate_up", idx, 2 * F, "bf16"))
    assert_close(rows_of(act, idx), ref_a, "bf16", "swiglu 5s")
    del gu, act
    q = dev_tensor("q", N, H * Dh, "bf16").view(N, H, Dh)
    k = dev_tensor("k", N, H * Dh, "bf16").view(N, H, Dh)
    qw = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    h3.h3f_qk_rmsnorm_rope3d(qo, ko, q, k, qw, kw,
                             h3.make_rope(c["T"], c["H"], c["W"], c["A"], c["split"]))
    pos = oracle.positions(N, c["T"], c["H"], c["W"], c["A"])[idx]
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", idx, H * Dh, "bf16").reshape(-1, H, Dh),
                                      host("k", idx, H * Dh, "bf16").reshape(-1, H, Dh),
                                      to_np(qw), to_np(kw), pos, c["split"])
    assert_close(rows_of(qo, idx), rq, "bf16", "q 5s")
    assert_close(rows_of(ko, idx), rk, "bf16", "k 5s")


# ------------------------------------------------------------------------------------
# determinism, guard bands, no-op and error paths on the GPU
# ------------------------------------------------------------------------------------

def test_run_twice_bit_identical():
    D = 5120
    x = dev_tensor("x", 1000, D, "bf16")
    sh, sc = dev_tensor("shift", 1, D, "bf16"), dev_tensor("scale", 1, D, "bf16")
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    h3.h3f_adaln_modulate(y1, x, sh, sc)
    h3.h3f_adaln_modulate(y2, x, sh, sc)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_guard_bands_untouched():
    rows, D, pad = 300, 3072, 4096
    buf = torch.full((rows * D + 2 * pad,), -7.0, dtype=torch.bfloat16, device=DEV)
    y = buf[pad:pad + rows * D].view(rows, D)
    x = dev_tensor("x", rows, D, "bf16")
    sh, sc = dev_tensor("shift", 1, D, "bf16"), dev_tensor("scale", 1, D, "bf16")
    h3.h3f_adaln_modulate(y, x, sh, sc)
    b = to_np(buf.float())
    assert np.all(b[:pad] == -7.0) and np.all(b[pad + rows * D:] == -7.0)
    gu = dev_tensor("gate_up", rows, 2 * D, "bf16")
    h3.h3f_swiglu(y, gu)
    b = to_np(buf.float())
    assert np.all(b[:pad] == -7.0) and np.all(b[pad + rows * D:] == -7.0)


@pytest.mark.parametrize("rows", [1, 2, 5])
def test_fused_guard_rows_untouched(rows):
    # x and y sit inside larger buffers whose later rows the call must not touch:
    # the spare wavefronts of the last workgroup load the last row again for the
    # modulation staging but store nothing
    D, extra = 5120, 7
    xb = torch.full((rows + extra, D), -3.0, dtype=torch.bfloat16, device=DEV)
    yb = torch.full((rows + extra, D), -5.0, dtype=torch.bfloat16, device=DEV)
    h3gen.fill_device(xb[:rows], "x")
    h = dev_tensor("h", rows, D, "bf16")
    gt, sh, sc = (dev_tensor(n, 1, D, "bf16") for n in ("gate", "shift", "scale"))
    h3.h3f_gated_residual_adaln(xb[:rows], h, gt, sh, sc, yb[:rows])
    assert torch.all(xb[rows:] == -3.0) and torch.all(yb[rows:] == -5.0)
    rx, ry = oracle.gated_residual_adaln(
        host("x", rows, D, "bf16"), host("h", rows, D, "bf16"),
        *(host(n, 1, D, "bf16") for n in ("gate", "shift", "scale")), y_dtype=np.uint16)
    assert_close(to_np(xb[:rows]), rx, kind("bf16"), "fused x")
    assert_close(to_np(yb[:rows]), ry, kind("bf16"), "fused y")


def test_zero_rows_is_noop_and_errors_raise():
    x = torch.empty(0, 256, device=DEV)
    h3.h3f_gated_residual(x, torch.empty(0, 256, device=DEV), torch.zeros(256, device=DEV))
    a = torch.zeros(4, 12, device=DEV)  # hidden 12 not a multiple of 8 for bf16
    with pytest.raises(h3.H3FError) as e:
        h3.h3f_swiglu(a.bfloat16(), a.bfloat16(), a.bfloat16())
    assert e.value.name == "H3F_ERR_BAD_SHAPE"
    x = dev_tensor("x", 8, 256, "bf16")
    with pytest.raises(h3.H3FError) as e:
        h3.h3f_gated_residual(x, x, torch.zeros(256, dtype=torch.bfloat16, device=DEV))
    assert e.value.name == "H3F_ERR_ALIASING"


# ------------------------------------------------------------------------------------
# 10 s shape and the roofline sweep, sampled rows
# ------------------------------------------------------------------------------------

def _sampled_all_ops(c, every=97):
    N, D, F, H, Dh = n_tokens(c), c["D"], c["F"], c["heads"], c["Dh"]
    idx = sample_rows(N, N - c["A"], every=every)
    x = dev_tensor("x", N, D, "bf16")
    sh, sc, gt = (dev_tensor(n, 1, D, "bf16") for n in ("shift", "scale", "gate"))
    y = torch.empty_like(x)
    h3.h3f_adaln_modulate(y, x, sh, sc)
    assert_close(rows_of(y, idx), oracle.adaln_modulate(
        host("x", idx, D, "bf16"), host("shift", 1, D, "bf16"), host("scale", 1, D, "bf16")),
        "bf16", "adaln")
    del y
    h = dev_tensor("h", N, D, "bf16")
    h3.h3f_gated_residual(x, h, gt)
    assert_close(rows_of(x, idx), oracle.gated_residual(
        host("x", idx, D, "bf16"), host("h", idx, D, "bf16"), host("gate", 1, D, "bf16")),
        "bf16", "gated")
    del x, h
    gu = dev_tensor("gate_up", N, 2 * F, "bf16")
    act = torch.empty(N, F, dtype=torch.bfloat16, device=DEV)
    h3.h3f_swiglu(act, gu)
    assert_close(rows_of(act, idx), oracle.swiglu(host("gate_up", idx, 2 * F, "bf16")), "bf16",
                 "swiglu")
    del gu, act
    q = dev_tensor("q", N, H * Dh, "bf16").view(N, H, Dh)
    k = dev_tensor("k", N, H * Dh, "bf16").view(N, H, Dh)
    qw = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    h3.h3f_qk_rmsnorm_rope3d(qo, ko, q, k, qw, kw,
                             h3.make_rope(c["T"], c["H"], c["W"], c["A"], c["split"]))
    pos = oracle.positions(N, c["T"], c["H"], c["W"], c["A"])[idx]
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", idx, H * Dh, "bf16").reshape(-1, H, Dh),
                                      host("k", idx, H * Dh, "bf16").reshape(-1, H, Dh),
                                      to_np(qw), to_np(kw), pos, c["split"])
    assert_close(rows_of(qo, idx), rq, "bf16", "q")
    assert_close(rows_of(ko, idx), rk, "bf16", "k")


def test_full_10s_shape_all_ops_sampled():
    _sampled_all_ops(S10, every=211)


@pytest.mark.parametrize("D,F", [(3072, 8320), (4096, 11008), (6144, 16640)])
def test_sweep_shapes_all_ops_sampled(D, F):
    _sampled_all_ops(dict(T=8, H=48, W=84, A=512, D=D, heads=D // 128, Dh=128,
                          split=(32, 48, 48), F=F), every=389)


# ------------------------------------------------------------------------------------
# block epilogue chain: 10 s shape, fp32 residual stream, packed qkv, 50 steps
# ------------------------------------------------------------------------------------

def test_chain_10s_50_steps_sampled():
    c = S10
    N, D, F, H, Dh = n_tokens(c), c["D"], c["F"], c["heads"], c["Dh"]
    steps = 50
    x = dev_tensor("x", N, D, "f32")
    mods = {n: dev_tensor(n, 1, D, "f32") for n in
            ("shift", "scale", "gate", "shift2", "scale2", "gate2")}
    h1 = dev_tensor("h", N, D, "bf16")
    h2 = dev_tensor("h2", N, D, "bf16")
    gu = dev_tensor("gate_up", N, 2 * F, "bf16")
    qkv = torch.empty(N, 3, H, Dh, dtype=torch.bfloat16, device=DEV)
    flat = qkv.view(N, 3 * H * Dh)
    for i, n in enumerate(("q", "k", "v")):
        h3gen.fill_device(flat[:, i * H * Dh:(i + 1) * H * Dh], n)
    qw = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    y = torch.empty(N, D, dtype=torch.bfloat16, device=DEV)
    qo = torch.empty(N, H, Dh, dtype=torch.bfloat16, device=DEV)
    ko = torch.empty_like(qo)
    act = torch.empty(N, F, dtype=torch.bfloat16, device=DEV)
    rope = h3.make_rope(c["T"], c["H"], c["W"], c["A"], c["split"])
    for _ in range(steps):
        h3.h3f_adaln_modulate(y, x, mods["shift"], mods["scale"])
        h3.h3f_qk_rmsnorm_rope3d(qo, ko, qkv[:, 0], qkv[:, 1], qw, kw, rope)
        h3.h3f_gated_residual(x, h1, mods["gate"])
        h3.h3f_adaln_modulate(y, x, mods["shift2"], mods["scale2"])
        h3.h3f_swiglu(act, gu)
        h3.h3f_gated_residual(x, h2, mods["gate2"])
    torch.cuda.synchronize()

    idx = sample_rows(N, N - c["A"], every=1999, head=16, tail=16)
    hm = {n: host(n, 1, D, "f32") for n in mods}
    rx = host("x", idx, D, "f32")
    rh1, rh2 = host("h", idx, D, "bf16"), host("h2", idx, D, "bf16")
    for _ in range(steps):
        oracle.adaln_modulate(rx, hm["shift"], hm["scale"], y_dtype=np.uint16)
        rx = oracle.gated_residual(rx, rh1, hm["gate"])
        ry = oracle.adaln_modulate(rx, hm["shift2"], hm["scale2"], y_dtype=np.uint16)
        rx = oracle.gated_residual(rx, rh2, hm["gate2"])
    # x grows to ~ x0 + 50 (g1 h1 + g2 h2): std ~ 35; fp32 tolerance still applies
    assert_close(rows_of(x, idx), rx, "f32", "chain x after 50 steps")
    assert_close(rows_of(y, idx), ry, "bf16", "chain last adaln")
    assert_close(rows_of(act, idx), oracle.swiglu(host("gate_up", idx, 2 * F, "bf16")), "bf16",
                 "chain swiglu")
    pos = oracle.positions(N, c["T"], c["H"], c["W"], c["A"])[idx]
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", idx, H * Dh, "bf16").reshape(-1, H, Dh),
                                      host("k", idx, H * Dh, "bf16").reshape(-1, H, Dh),
                                      to_np(qw), to_np(kw), pos, c["split"])
    assert_close(rows_of(qo, idx), rq, "bf16", "chain q")
    assert_close(rows_of(ko, idx), rk, "bf16", "chain k")


# ------------------------------------------------------------------------------------
# residual difference (step-reuse test): a global reduction, compared as a whole
# ------------------------------------------------------------------------------------

# fp32 lane sums of 64 terms, a 6-level DPP tree and two fp32 workgroup levels before
# fp64: relative error below ~72 * 2^-24 of the sum of |terms|; 1e-5 leaves margin.
L1_RTOL = 1e-5


def _l1_check(rows, D, dt, rs_pad=0):
    cur = dev_tensor("x", rows, D, dt, row_stride=D + rs_pad)
    prev = dev_tensor("x_prev", rows, D, dt, row_stride=D + rs_pad)
    out = torch.zeros(3, dtype=torch.float64, device=DEV)
    h3.h3f_residual_l1(out, cur, prev)
    got = out.cpu().numpy()
    num, den = oracle.residual_l1(host("x", rows, D, dt), host("x_prev", rows, D, dt))
    assert abs(got[0] - num) <= L1_RTOL * num
    assert abs(got[1] - den) <= L1_RTOL * den
    assert abs(got[2] - num / den) <= 2 * L1_RTOL * (num / den)
    return out, cur, prev


@pytest.mark.parametrize("rows,D,dt,pad", [(112, 256, "f32", 0), (1001, 5120, "bf16", 0),
                                          (33, 1000, "bf16", 24), (3, 8, "bf16", 0)])
def test_residual_l1(rows, D, dt, pad):
    _l1_check(rows, D, dt, pad)


def test_residual_l1_full_5s_shape_deterministic_and_zero():
    out, cur, prev = _l1_check(n_tokens(S5), S5["D"], "bf16")
    out2 = torch.zeros(3, dtype=torch.float64, device=DEV)
    h3.h3f_residual_l1(out2, cur, prev)
    assert torch.equal(out, out2)  # bit-identical run to run
    h3.h3f_residual_l1(out2, prev, prev)
    assert out2[0].item() == 0.0 and out2[2].item() == 0.0
