"""GPU guard bands and invariants.

Guard bands: every output of every entry point is written inside a larger
buffer filled with a canary value -- before and after the tensor, and in the
gaps a padded row stride or head stride leaves between rows and heads -- and
after the call every canary must still be there.  The stores these checks
cover are the ones that rely on the hardware dropping out-of-range buffer
accesses (ragged row tails, head slots past the last head, spare wavefronts of
the last workgroup).

Invariants on the GPU's own outputs (the oracle's pins, re-checked on the
device):
  * RoPE at position 0 is the identity: with every position (0, 0, 0) the two
    pair layouts (interleaved and rotate-half) give bit-identical outputs, which
    match the oracle's RMSNorm alone;
  * audio tokens (h = w = 0) leave the h and w chunks unrotated: those chunks are
    bit-identical between the two pair layouts;
  * RoPE preserves the norm of every rotated pair: the GPU's per-pair norms at
    real positions equal its own norms at position 0 to within the output
    rounding;
  * gate = 0 leaves x bit-identical in the fused gated residual + AdaLN, whose y
    then equals the plain AdaLN of the same x bit for bit.
"""
import numpy as np
import pytest
import torch

import h3gen
import oracle
from gpu_util import DEV, dev_tensor, from_np, host, kind, to_np
from tolerance import as_f64, assert_close

pytestmark = pytest.mark.gpu

h3 = pytest.importorskip("video_diffusion_transformer_h3f_amd")

S5 = dict(T=31, H=48, W=84, A=128, D=5120, heads=40, Dh=128, split=(32, 48, 48), F=13824)
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
CANARY = -7.0  # exactly representable in bf16 and fp32; no operator output here equals it


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h3.lib()
    h3gen.dev_lib()
    yield
    torch.cuda.synchronize()


def guarded(rows, cols, dtype, row_stride=None, pad=4096):
    """A [rows, cols] view (row stride row_stride) inside a canary-filled buffer with
    `pad` canary elements before and after; returns (view, buffer, mask of the
    view's elements inside the buffer)."""
    rs = cols if row_stride is None else row_stride
    n = pad + (rows - 1) * rs + cols + pad if rows else 2 * pad
    buf = torch.full((n,), CANARY, dtype=TDT[dtype], device=DEV)
    view = buf[pad:pad + rows * rs].view(rows, rs)[:, :cols] if rows else buf[pad:pad]
    mask = np.zeros(n, dtype=bool)
    for r in range(rows):
        mask[pad + r * rs: pad + r * rs + cols] = True
    return view, buf, mask


def canaries_intact(buf, mask, what):
    b = as_f64(to_np(buf))
    bad = np.flatnonzero(~mask & (b != CANARY))
    assert bad.size == 0, f"{what}: {bad.size} canary elements overwritten (first at {bad[:5]})"


def filled(name, rows, cols, dtype, row_stride=None, seed=0):
    v, buf, mask = guarded(rows, cols, dtype, row_stride)
    h3gen.fill_device(v, name, seed=seed)
    return v, buf, mask


# ------------------------------------------------------------------------------------
# guard bands
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,D,xdt,hdt,pad", [
    (1, 5120, "bf16", "bf16", 0), (3, 5120, "bf16", "bf16", 8), (67, 1000, "f32", "f32", 12),
    (1001, 3072, "f32", "bf16", 4), (129, 8, "bf16", "bf16", 16),
])
def test_gated_residual_guards(rows, D, xdt, hdt, pad):
    x, xbuf, xmask = filled("x", rows, D, xdt, row_stride=D + pad)
    h = dev_tensor("h", rows, D, hdt)
    g = dev_tensor("gate", 1, D, xdt)
    h3.h3f_gated_residual(x, h, g)
    canaries_intact(xbuf, xmask, "gated x")
    ref = oracle.gated_residual(host("x", rows, D, xdt), host("h", rows, D, hdt),
                                host("gate", 1, D, xdt))
    assert_close(to_np(x), ref, kind(xdt), "gated x")


@pytest.mark.parametrize("rows,D,dt,pad", [(1, 5120, "bf16", 8), (5, 5120, "bf16", 0),
                                           (77, 1000, "f32", 4), (300, 3072, "bf16", 24)])
def test_adaln_and_swiglu_row_gaps(rows, D, dt, pad):
    y, ybuf, ymask = guarded(rows, D, dt, row_stride=D + pad)
    x = dev_tensor("x", rows, D, dt)
    sh, sc = dev_tensor("shift", 1, D, dt), dev_tensor("scale", 1, D, dt)
    h3.h3f_adaln_modulate(y, x, sh, sc)
    canaries_intact(ybuf, ymask, "adaln y")
    assert_close(to_np(y), oracle.adaln_modulate(host("x", rows, D, dt), host("shift", 1, D, dt),
                                                 host("scale", 1, D, dt)), kind(dt), "adaln y")
    out, obuf, omask = guarded(rows, D, dt, row_stride=D + pad)
    gu = dev_tensor("gate_up", rows, 2 * D, dt)
    h3.h3f_swiglu(out, gu)
    canaries_intact(obuf, omask, "swiglu out")
    assert_close(to_np(out), oracle.swiglu(host("gate_up", rows, 2 * D, dt)), kind(dt), "swiglu")


@pytest.mark.parametrize("rows,dt,pad", [(1, "bf16", 0), (3, "bf16", 8), (130, "f32", 4)])
def test_fused_gated_adaln_guards(rows, dt, pad):
    D = 5120 if dt == "bf16" else 2048
    x, xbuf, xmask = filled("x", rows, D, dt, row_stride=D + pad)
    y, ybuf, ymask = guarded(rows, D, dt, row_stride=D + pad)
    h = dev_tensor("h", rows, D, dt)
    gt, sh, sc = (dev_tensor(n, 1, D, dt) for n in ("gate", "shift", "scale"))
    h3.h3f_gated_residual_adaln(x, h, gt, sh, sc, y)
    canaries_intact(xbuf, xmask, "fused x")
    canaries_intact(ybuf, ymask, "fused y")
    rx, ry = oracle.gated_residual_adaln(host("x", rows, D, dt), host("h", rows, D, dt),
                                         *(host(n, 1, D, dt) for n in ("gate", "shift", "scale")))
    assert_close(to_np(x), rx, kind(dt), "fused x")
    assert_close(to_np(y), ry, kind(dt), "fused y")


def _qk_guarded(rows, heads, Dh, dt, split, head_pad, row_pad):
    """q_out / k_out as [rows, heads, Dh] views with padded head and row strides
    inside canary buffers; returns (views, buffers, masks)."""
    hs = Dh + head_pad
    rs = heads * hs + row_pad
    outs = []
    for _ in range(2):
        n = 2 * 4096 + rows * rs
        buf = torch.full((n,), CANARY, dtype=TDT[dt], device=DEV)
        view = buf[4096:4096 + rows * rs].as_strided((rows, heads, Dh), (rs, hs, 1))
        mask = np.zeros(n, dtype=bool)
        for r in range(rows):
            for hh in range(heads):
                s = 4096 + r * rs + hh * hs
                mask[s:s + Dh] = True
        outs.append((view, buf, mask))
    return outs


@pytest.mark.parametrize("rows,heads,Dh,dt,split,head_pad,row_pad", [
    (37, 5, 128, "bf16", (32, 48, 48), 0, 0),     # 5 heads: the second 4-head slot is ragged
    (37, 5, 128, "bf16", (32, 48, 48), 8, 16),    # padded head and row strides
    (19, 3, 64, "f32", (16, 24, 24), 4, 4),
    (11, 1, 256, "bf16", (64, 96, 96), 0, 8),
])
def test_qk_out_of_place_guards(rows, heads, Dh, dt, split, head_pad, row_pad):
    (qo, qbuf, qmask), (ko, kbuf, kmask) = _qk_guarded(rows, heads, Dh, dt, split, head_pad,
                                                       row_pad)
    q = dev_tensor("q", rows, heads * Dh, dt).view(rows, heads, Dh)
    k = dev_tensor("k", rows, heads * Dh, dt).view(rows, heads, Dh)
    qw, kw = dev_tensor("q_weight", 1, Dh, dt).view(Dh), dev_tensor("k_weight", 1, Dh, dt).view(Dh)
    T, Hg, W, A = 2, 3, 4, 5
    h3.h3f_qk_rmsnorm_rope3d(qo, ko, q, k, qw, kw, h3.make_rope(T, Hg, W, A, split,
                                                                 token_offset=7))
    canaries_intact(qbuf, qmask, "q_out")
    canaries_intact(kbuf, kmask, "k_out")
    pos = oracle.positions(rows, T, Hg, W, A, token_offset=7)
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", rows, heads * Dh, dt).reshape(rows, heads, Dh),
                                      host("k", rows, heads * Dh, dt).reshape(rows, heads, Dh),
                                      to_np(qw), to_np(kw), pos, split)
    assert_close(to_np(qo), rq, kind(dt), "q_out")
    assert_close(to_np(ko), rk, kind(dt), "k_out")


@pytest.mark.parametrize("heads,head_pad,row_pad", [(5, 0, 0), (5, 8, 16)])
def test_qk_pool_guards(heads, head_pad, row_pad):
    # the QK operator with the router's block pooling: same stores, plus the means
    rows, Dh, split, block = 4096 + 77, 128, (32, 48, 48), 128
    (qo, qbuf, qmask), (ko, kbuf, kmask) = _qk_guarded(rows, heads, Dh, "bf16", split, head_pad,
                                                       row_pad)
    q = dev_tensor("q", rows, heads * Dh, "bf16").view(rows, heads, Dh)
    k = dev_tensor("k", rows, heads * Dh, "bf16").view(rows, heads, Dh)
    qw = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    nb, keep, need = h3.h3f_subblock_plan(rows, heads, Dh, block, 0.8, 10)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    h3.h3f_qk_rmsnorm_rope3d_pool(qo, ko, q, k, qw, kw, h3.make_rope(31, 48, 84, 128, split),
                                  block, ws)
    canaries_intact(qbuf, qmask, "pooled q_out")
    canaries_intact(kbuf, kmask, "pooled k_out")
    pos = oracle.positions(rows, 31, 48, 84, 128)
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", rows, heads * Dh, "bf16").reshape(rows, heads, Dh),
                                      host("k", rows, heads * Dh, "bf16").reshape(rows, heads, Dh),
                                      to_np(qw), to_np(kw), pos, split)
    assert_close(to_np(qo), rq, "bf16", "pooled q_out")
    assert_close(to_np(ko), rk, "bf16", "pooled k_out")


@pytest.mark.parametrize("rows,heads", [(33, 5), (200, 40)])
def test_qk_packed_in_place_guards(rows, heads):
    Dh, split = 128, (32, 48, 48)
    n = rows * 3 * heads * Dh
    buf = torch.full((n + 2 * 4096,), CANARY, dtype=torch.bfloat16, device=DEV)
    qkv = buf[4096:4096 + n].view(rows, 3, heads, Dh)
    flat = qkv.view(rows, 3 * heads * Dh)
    for i, name in enumerate(("q", "k", "v")):
        h3gen.fill_device(flat[:, i * heads * Dh:(i + 1) * heads * Dh], name)
    before = to_np(buf)
    q, k = qkv[:, 0], qkv[:, 1]
    qw = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    h3.h3f_qk_rmsnorm_rope3d(q, k, q, k, qw, kw, h3.make_rope(31, 48, 84, 128, split))
    after = to_np(buf)
    # outside q and k (canaries and v) nothing changed, bit for bit
    qk_mask = np.zeros(buf.numel(), dtype=bool)
    for r in range(rows):
        s = 4096 + r * 3 * heads * Dh
        qk_mask[s:s + 2 * heads * Dh] = True
    assert np.array_equal(after[~qk_mask], before[~qk_mask]), "canaries or v changed"
    pos = oracle.positions(rows, 31, 48, 84, 128)
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", rows, heads * Dh, "bf16").reshape(rows, heads, Dh),
                                      host("k", rows, heads * Dh, "bf16").reshape(rows, heads, Dh),
                                      to_np(qw), to_np(kw), pos, split)
    assert_close(to_np(q), rq, "bf16", "q in place")
    assert_close(to_np(k), rk, "bf16", "k in place")



@pytest.mark.parametrize("kib", [1, 2, 5, 10])
@pytest.mark.parametrize("nbytes", [16, 4096 * 10 - 16, 3 * 40960 + 1008, 1 << 20])
def test_stream_fill_bursts_writes_exactly_its_bytes(kib, nbytes):
    # every 32-bit word of [0, nbytes) takes the value, nothing past it changes
    # (ragged last wavefront, a part-filled last workgroup, a single chunk)
    pad = 4096
    buf = torch.full((nbytes // 4 + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    view = buf[pad:pad + nbytes // 4]
    h3.h3f_stream_fill_bursts(view, kib, value=0x12345678)
    b = to_np(buf)
    assert (b[:pad] == 0x5A5A5A5A).all() and (b[pad + nbytes // 4:] == 0x5A5A5A5A).all()
    assert (b[pad:pad + nbytes // 4] == 0x12345678).all()


@pytest.mark.parametrize("rows,D,dt", [(1, 8, "bf16"), (1001, 5120, "bf16"), (67, 1000, "f32")])
def test_residual_l1_out_guards(rows, D, dt):
    buf = torch.full((16,), CANARY, dtype=torch.float64, device=DEV)
    out = buf[5:8]
    cur, prev = dev_tensor("x", rows, D, dt), dev_tensor("x_prev", rows, D, dt)
    h3.h3f_residual_l1(out, cur, prev)
    b = buf.cpu().numpy()
    assert (b[:5] == CANARY).all() and (b[8:] == CANARY).all()
    num, den = oracle.residual_l1(host("x", rows, D, dt), host("x_prev", rows, D, dt))
    assert abs(b[5] - num) <= 1e-5 * num and abs(b[6] - den) <= 1e-5 * den


@pytest.mark.parametrize("rows,heads,block", [(4096 + 77, 3, 128), (4096, 5, 3)])
@pytest.mark.parametrize("padded", [False, True], ids=["dense", "padded"])
def test_router_output_guards(rows, heads, block, padded):
    q = dev_tensor("q", rows, heads * 128, "bf16").view(rows, heads, 128)
    k = dev_tensor("k", rows, heads * 128, "bf16").view(rows, heads, 128)
    nb, keep, _ = h3.h3f_subblock_plan(rows, heads, 128, block, 0.8, 10)
    S = -(-nb // 32) * 32 + 3 if padded else nb  # rows of scores S floats apart
    pad = 1024
    kvbuf = torch.full((heads * nb * keep + 2 * pad,), -7, dtype=torch.int32, device=DEV)
    scbuf = torch.full((heads * nb * S + 2 * pad,), CANARY, dtype=torch.float32, device=DEV)
    kv = kvbuf[pad:pad + heads * nb * keep].view(heads, nb, keep)
    sc = scbuf[pad:pad + heads * nb * S].view(heads, nb, S)[:, :, :nb]
    h3.h3f_subblock_route(kv, sc, q, k, block, 0.8, 10)
    kb, sb = to_np(kvbuf), to_np(scbuf)
    assert (kb[:pad] == -7).all() and (kb[-pad:] == -7).all()
    assert (sb[:pad] == CANARY).all() and (sb[-pad:] == CANARY).all()
    rows_of_sc = sb[pad:-pad].reshape(heads, nb, S)
    assert (rows_of_sc[:, :, nb:] == CANARY).all()  # the pad columns of padded rows
    assert not (rows_of_sc[:, :, :nb] == CANARY).any()  # every score written
    kvm = kb[pad:-pad]
    assert kvm.min() >= 0 and kvm.max() < nb  # every kept-list entry written


# ------------------------------------------------------------------------------------
# invariants of the GPU's own outputs
# ------------------------------------------------------------------------------------

def _qk_run(q, k, qw, kw, split, positions=None, pairing=h3.H3F_ROPE_INTERLEAVED, grid=None):
    rows = q.shape[0]
    T, Hg, W, A = grid or (31, 48, 84, 128)
    rope = h3.make_rope(T, Hg, W, A, split, positions=positions, pairing=pairing)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    h3.h3f_qk_rmsnorm_rope3d(qo, ko, q, k, qw, kw, rope)
    return to_np(qo), to_np(ko)


@pytest.mark.parametrize("dt,Dh,split", [("bf16", 128, (32, 48, 48)), ("f32", 64, (16, 24, 24))])
def test_rope_position_zero_is_identity(dt, Dh, split):
    rows, heads = 96, 6
    q = dev_tensor("q", rows, heads * Dh, dt).view(rows, heads, Dh)
    k = dev_tensor("k", rows, heads * Dh, dt).view(rows, heads, Dh)
    qw, kw = dev_tensor("q_weight", 1, Dh, dt).view(Dh), dev_tensor("k_weight", 1, Dh, dt).view(Dh)
    zeros = torch.zeros(rows, 3, dtype=torch.int32, device=DEV)
    a = _qk_run(q, k, qw, kw, split, positions=zeros)
    b = _qk_run(q, k, qw, kw, split, positions=zeros, pairing=h3.H3F_ROPE_HALF_SPLIT)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # and that is the RMSNorm alone (the oracle at position 0)
    rq, rk = oracle.qk_rmsnorm_rope3d(host("q", rows, heads * Dh, dt).reshape(rows, heads, Dh),
                                      host("k", rows, heads * Dh, dt).reshape(rows, heads, Dh),
                                      to_np(qw), to_np(kw), np.zeros((rows, 3), np.int32), split)
    assert_close(a[0], rq, kind(dt), "q at position 0")
    assert_close(a[1], rk, kind(dt), "k at position 0")
    # video token 0 of the grid is position (0, 0, 0): same bits as the explicit zeros
    g = _qk_run(q, k, qw, kw, split)
    assert np.array_equal(g[0][0], a[0][0]) and np.array_equal(g[1][0], a[1][0])


def test_audio_tokens_leave_h_and_w_chunks_unrotated():
    # the last 128 rows of the 5 s sequence are audio tokens (t = k, h = w = 0)
    Dh, split, heads = 128, (32, 48, 48), 8
    N = 31 * 48 * 84 + 128
    rows = 300
    q = torch.empty(rows, heads * Dh, dtype=torch.bfloat16, device=DEV)
    k = torch.empty_like(q)
    h3gen.fill_device(q, "q", row0=N - rows)
    h3gen.fill_device(k, "k", row0=N - rows)
    q, k = q.view(rows, heads, Dh), k.view(rows, heads, Dh)
    qw = dev_tensor("q_weight", 1, Dh, "bf16").view(Dh)
    kw = dev_tensor("k_weight", 1, Dh, "bf16").view(Dh)
    pos = from_np(oracle.positions(N, 31, 48, 84, 128)[N - rows:])
    a = _qk_run(q, k, qw, kw, split, positions=pos)
    b = _qk_run(q, k, qw, kw, split, positions=pos, pairing=h3.H3F_ROPE_HALF_SPLIT)
    audio = slice(rows - 128, rows)
    for x, y in ((a[0], b[0]), (a[1], b[1])):
        assert np.array_equal(x[audio, :, 32:], y[audio, :, 32:]), "h/w chunks of audio rows"
        assert not np.array_equal(x[audio, :, :32], y[audio, :, :32])  # t chunk does rotate
        assert not np.array_equal(x[:100, :, 32:], y[:100, :, 32:])    # video rows rotate h, w


@pytest.mark.parametrize("dt,rtol", [("f32", 4e-7), ("bf16", 2 ** -7)])
def test_rope_preserves_pair_norms(dt, rtol):
    rows, heads, Dh, split = 64, 4, 128, (32, 48, 48)
    q = dev_tensor("q", rows, heads * Dh, dt).view(rows, heads, Dh)
    k = dev_tensor("k", rows, heads * Dh, dt).view(rows, heads, Dh)
    qw, kw = dev_tensor("q_weight", 1, Dh, dt).view(Dh), dev_tensor("k_weight", 1, Dh, dt).view(Dh)
    # large, varied positions: 10 s frames and the far corner of the grid
    pos_np = np.stack([np.arange(rows) % 61, (np.arange(rows) * 7) % 48,
                       (np.arange(rows) * 13) % 84], axis=1).astype(np.int32)
    pos_np[-1] = (60, 47, 83)
    zeros = torch.zeros(rows, 3, dtype=torch.int32, device=DEV)
    for pairing in (h3.H3F_ROPE_INTERLEAVED, h3.H3F_ROPE_HALF_SPLIT):
        rot = _qk_run(q, k, qw, kw, split, positions=from_np(pos_np), pairing=pairing)
        ref = _qk_run(q, k, qw, kw, split, positions=zeros, pairing=pairing)
        for r, z in zip(rot, ref):
            r, z = as_f64(r), as_f64(z)
            if pairing == h3.H3F_ROPE_INTERLEAVED:
                nr = np.hypot(r[..., 0::2], r[..., 1::2])
                nz = np.hypot(z[..., 0::2], z[..., 1::2])
            else:  # pairs (j, j + d_c/2) inside each chunk
                nr, nz = [], []
                o = 0
                for d in split:
                    h = d // 2
                    nr.append(np.hypot(r[..., o:o + h], r[..., o + h:o + d]))
                    nz.append(np.hypot(z[..., o:o + h], z[..., o + h:o + d]))
                    o += d
                nr, nz = np.concatenate(nr, -1), np.concatenate(nz, -1)
            # each stored component carries one output rounding (relative <= 2^-24
            # fp32, 2^-8 bf16 ulp / 2); the pair norm moves by at most that relative
            err = np.abs(nr - nz) / np.maximum(nz, 1e-30)
            assert float(err.max()) <= rtol, (dt, pairing, float(err.max()))


@pytest.mark.parametrize("rows,D,xdt,hdt", [(300, 5120, "bf16", "bf16"), (77, 2048, "f32", "bf16")])
def test_fused_gate_zero_is_identity(rows, D, xdt, hdt):
    x = dev_tensor("x", rows, D, xdt)
    x0 = to_np(x)
    h = dev_tensor("h", rows, D, hdt)
    g = torch.zeros(1, D, dtype=TDT[xdt], device=DEV)
    sh, sc = dev_tensor("shift", 1, D, xdt), dev_tensor("scale", 1, D, xdt)
    y = torch.empty(rows, D, dtype=torch.bfloat16, device=DEV)
    h3.h3f_gated_residual_adaln(x, h, g, sh, sc, y)
    assert np.array_equal(to_np(x), x0), "gate = 0 must leave x bit-identical"
    y_plain = torch.empty_like(y)
    h3.h3f_adaln_modulate(y_plain, x, sh, sc)
    assert np.array_equal(to_np(y), to_np(y_plain)), "y must be the plain AdaLN of x"
    assert_close(to_np(y), oracle.adaln_modulate(x0, host("shift", 1, D, xdt),
                                                 host("scale", 1, D, xdt), y_dtype=np.uint16),
                 "bf16", "fused y at gate 0")
