"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol include/h3fused.h declares, and rejects invalid arguments with the
documented status codes before any launch (no compute call is made here:
every call below fails validation, which is pure host logic)."""
import ctypes
import os
import re
import subprocess

import pytest

import video_diffusion_transformer_h3f_amd as h3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3fused.h")

OK, NULLP, SHAPE, STRIDE, MISAL, DTYPE, ALIAS, LAUNCH, UNSUP, WORKSPACE, BADVAL = range(11)
F32, BF16 = 0, 1


def declared():
    src = open(HEADER).read()
    return set(re.findall(r"^\s*(?:h3f_status_t|int|size_t|const char\s*\*)\s*(h3f_\w+)\s*\(",
                          src, re.M))


def test_header_declares_the_binding_exports():
    assert declared() == set(h3.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    L = h3.lib()
    for name in declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", h3.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (h3f_\w+)", out))
    assert declared() <= exported
    assert h3.abi_version() == 1


def test_status_strings():
    L = h3.lib()
    for s in range(11):
        assert L.h3f_status_string(s) != b"unknown status"
    assert L.h3f_status_string(99) == b"unknown status"


P = ctypes.c_void_p


def A(n):
    """A fake, never dereferenced device address, 16-byte aligned, far apart per n."""
    return P(0x10000000 * (n + 1))


L = None


@pytest.fixture(autouse=True, scope="module")
def _lib():
    global L
    L = h3.lib()


# --- gated residual -------------------------------------------------------------------

def gated(x=A(0), xd=BF16, xs=256, h=A(1), hd=BF16, hs=256, gate=A(2), gs=0, rpg=10, rows=10,
          hidden=256):
    return L.h3f_gated_residual(x, xd, xs, h, hd, hs, gate, gs, rpg, rows, hidden, None)


def test_gated_validation():
    assert gated(x=None, rows=0) == OK  # rows == 0 is a no-op before any check
    assert gated(x=None) == NULLP
    assert gated(h=None) == NULLP
    assert gated(gate=None) == NULLP
    assert gated(xd=7) == DTYPE
    assert gated(xd=BF16, hd=F32) == DTYPE
    assert gated(rows=-1) == SHAPE
    assert gated(hidden=0) == SHAPE
    assert gated(hidden=252) == SHAPE  # not a multiple of 8
    assert gated(rpg=0) == SHAPE
    assert gated(x=P(0x10000008)) == MISAL
    assert gated(xs=260) == STRIDE
    assert gated(xs=128) == STRIDE  # rows overlap
    assert gated(h=P(0x10000000 + 512)) == ALIAS  # h overlaps x
    assert gated(rows=2 ** 31) == UNSUP
    assert gated(rpg=5, gs=12) == STRIDE  # two groups, stride not a vector multiple
    assert gated(gate=P(0x10000000 + 64)) == ALIAS


# --- SwiGLU -----------------------------------------------------------------------------

def swiglu(out=A(0), os_=64, a=A(1), as_=128, b=P(0x20000000 + 128), bs=128, dt=BF16, rows=10,
           inner=64):
    return L.h3f_swiglu(out, os_, a, as_, b, bs, dt, rows, inner, None)


def test_swiglu_validation():
    assert swiglu(out=None, rows=0) == OK
    assert swiglu(out=None) == NULLP
    assert swiglu(b=None) == NULLP
    assert swiglu(dt=3) == DTYPE
    assert swiglu(inner=60) == SHAPE
    assert swiglu(inner=0) == SHAPE
    assert swiglu(a=P(0x20000004)) == MISAL
    assert swiglu(as_=132) == STRIDE
    assert swiglu(os_=32) == STRIDE
    assert swiglu(out=P(0x20000000 + 64)) == ALIAS   # out straddles a's row
    assert swiglu(out=P(0x20000000 + 144), os_=128) == ALIAS  # out shifted inside b's rows
    assert swiglu(dt=F32, inner=64, out=P(0x20000000 + 8)) == MISAL


# --- AdaLN --------------------------------------------------------------------------------

def adaln(y=A(0), yd=BF16, ys=512, x=A(1), xd=BF16, xs=512, sh=A(2), sc=A(3), gs=0, rpg=4,
          rows=4, hidden=512, eps=1e-6):
    return L.h3f_adaln_modulate(y, yd, ys, x, xd, xs, sh, sc, gs, rpg, rows, hidden,
                                ctypes.c_float(eps), None)


def test_adaln_validation():
    assert adaln(x=None, rows=0) == OK
    assert adaln(sc=None) == NULLP
    assert adaln(xd=BF16, yd=F32) == DTYPE
    assert adaln(hidden=516) == SHAPE
    assert adaln(hidden=16392, xs=16392, ys=16392) == UNSUP
    assert adaln(xd=F32, yd=F32, hidden=8196, xs=8196, ys=8196) == UNSUP
    assert adaln(sh=P(0x30000008)) == MISAL
    assert adaln(ys=500) == STRIDE
    assert adaln(y=P(0x20000000 + 16)) == ALIAS  # partial overlap with x
    assert adaln(y=A(1), yd=BF16, xd=BF16, ys=520) == ALIAS  # same base, other stride
    assert adaln(y=A(2)) == ALIAS  # y over shift


# --- fused gated + AdaLN -----------------------------------------------------------------------

def fused(x=A(0), xd=BF16, xs=512, h=A(1), hd=BF16, hs=512, g=A(2), sh=A(3), sc=A(4), gs=0,
          rpg=4, y=A(5), yd=BF16, ys=512, rows=4, hidden=512):
    return L.h3f_gated_residual_adaln(x, xd, xs, h, hd, hs, g, sh, sc, gs, rpg, y, yd, ys, rows,
                                      hidden, ctypes.c_float(1e-6), None)


def test_fused_validation():
    assert fused(y=None, rows=0) == OK
    assert fused(y=None) == NULLP
    assert fused(xd=BF16, hd=F32) == DTYPE
    assert fused(xd=BF16, yd=F32) == DTYPE
    assert fused(y=A(0)) == ALIAS  # y may not alias x in the fused form
    assert fused(y=A(1)) == ALIAS
    assert fused(hidden=20000, xs=20000, hs=20000, ys=20000) == UNSUP


# --- QK RMSNorm + RoPE -------------------------------------------------------------------------

def rope(**kw):
    r = h3.make_rope(31, 48, 84, 128, (32, 48, 48))
    for k, v in kw.items():
        setattr(r, k, v)
    return r


def qk(qo=A(0), qors=5120, qohs=128, ko=A(1), kors=5120, kohs=128, q=A(2), qrs=5120, qhs=128,
       k=A(3), krs=5120, khs=128, qw=A(4), kw=A(5), dt=BF16, rows=10, heads=40, hd=128, r=None):
    r = rope() if r is None else r
    return L.h3f_qk_rmsnorm_rope3d(qo, qors, qohs, ko, kors, kohs, q, qrs, qhs, k, krs, khs, qw, kw,
                                   dt, rows, heads, hd, ctypes.c_float(1e-6), ctypes.byref(r),
                                   None)


def test_qk_validation():
    assert qk(q=None, rows=0) == OK
    assert qk(kw=None) == NULLP
    assert L.h3f_qk_rmsnorm_rope3d(A(0), 5120, 128, A(1), 5120, 128, A(2), 5120, 128, A(3), 5120,
                                   128, A(4), A(5), BF16, 10, 40, 128, ctypes.c_float(1e-6), None,
                                   None) == NULLP
    assert qk(dt=5) == DTYPE
    assert qk(hd=124) == SHAPE  # not a multiple of 8
    assert qk(hd=120) == UNSUP  # 120 / 8 = 15 lanes: not a power of two
    assert qk(hd=96, qohs=96, kohs=96, qhs=96, khs=96) == UNSUP
    assert qk(hd=1024, r=rope(d_t=256, d_h=384, d_w=384)) == UNSUP
    assert qk(r=rope(d_t=30, d_h=50, d_w=48)) == SHAPE  # chunk not a multiple of 8
    assert qk(r=rope(d_t=32, d_h=48, d_w=40)) == SHAPE  # does not sum to head_dim
    assert qk(r=rope(pairing=2)) == UNSUP
    assert qk(r=rope(pairing=1, d_t=40, d_h=40, d_w=48)) == UNSUP  # half split needs 16 | d_c
    assert qk(r=rope(theta=0.0)) == SHAPE
    assert qk(r=rope(T=0)) == SHAPE
    assert qk(r=rope(token_offset=-1)) == SHAPE
    assert qk(q=P(0x30000002)) == MISAL
    assert qk(qhs=100) == STRIDE  # heads overlap
    assert qk(qrs=5000) == STRIDE  # rows overlap
    assert qk(qhs=132) == STRIDE  # not a vector multiple
    assert qk(qo=A(3)) == ALIAS  # q_out over k
    assert qk(ko=A(0)) == ALIAS  # k_out over q_out
    assert qk(qo=A(2), qohs=256, qors=20480, qhs=128, qrs=20480) == ALIAS  # same base, head strides differ
    assert qk(qo=A(4)) == ALIAS  # over a weight


def test_qk_valid_split_is_not_called():
    # a valid argument set would launch; make sure the helper above never does by keeping
    # one invalid field in every call (this test documents the convention)
    assert qk(r=rope(d_t=32, d_h=40, d_w=56), dt=9) == DTYPE


# --- positions, stream copy ---------------------------------------------------------------------

def test_positions_and_copy_validation():
    r = rope()
    assert L.h3f_rope3d_positions(None, 0, ctypes.byref(r), None) == OK
    assert L.h3f_rope3d_positions(None, 5, ctypes.byref(r), None) == NULLP
    assert L.h3f_rope3d_positions(A(0), 5, None, None) == NULLP
    assert L.h3f_rope3d_positions(P(0x10000002), 5, ctypes.byref(r), None) == MISAL
    bad = rope(H=0)
    assert L.h3f_rope3d_positions(A(0), 5, ctypes.byref(bad), None) == SHAPE
    assert L.h3f_rope3d_positions(A(0), -5, ctypes.byref(r), None) == SHAPE
    assert L.h3f_stream_copy(A(0), A(1), 0, None) == OK
    assert L.h3f_stream_copy(None, A(1), 16, None) == NULLP
    assert L.h3f_stream_copy(A(0), A(1), 17, None) == SHAPE
    assert L.h3f_stream_copy(A(0), P(0x10000000 + 32), 64, None) == ALIAS
    assert L.h3f_stream_copy(A(0), P(0x20000008), 64, None) == MISAL


def test_stream_read_and_fill_validation():
    # zero bytes is a no-op before any other check; the rest is rejected on the host
    assert L.h3f_stream_read(None, 0, 0, None, None) == OK
    assert L.h3f_stream_read(None, 16, 0, A(1), None) == NULLP
    assert L.h3f_stream_read(A(0), 16, 0, None, None) == NULLP
    assert L.h3f_stream_read(A(0), 17, 0, A(1), None) == SHAPE
    assert L.h3f_stream_read(A(0), -16, 1, A(1), None) == SHAPE
    assert L.h3f_stream_read(P(0x10000008), 64, 0, A(1), None) == MISAL
    assert L.h3f_stream_read(A(0), 64, 0, P(0x20000008), None) == MISAL
    # the sink inside the bytes read
    assert L.h3f_stream_read(P(0x10000000), 64, 1, P(0x10000000 + 32), None) == ALIAS
    assert L.h3f_stream_fill(None, 0, 7, None) == OK
    assert L.h3f_stream_fill(None, 16, 7, None) == NULLP
    assert L.h3f_stream_fill(A(0), 24, 7, None) == SHAPE
    assert L.h3f_stream_fill(P(0x10000004), 32, 7, None) == MISAL
    assert L.h3f_stream_fill_bursts(None, 0, 7, 10, None) == OK
    assert L.h3f_stream_fill_bursts(None, 16, 7, 10, None) == NULLP
    assert L.h3f_stream_fill_bursts(A(0), 24, 7, 10, None) == SHAPE
    assert L.h3f_stream_fill_bursts(A(0), -16, 7, 10, None) == SHAPE
    assert L.h3f_stream_fill_bursts(P(0x10000004), 32, 7, 10, None) == MISAL
    for k in (0, 3, 4, 11, -1):
        assert L.h3f_stream_fill_bursts(A(0), 1 << 20, 7, k, None) == UNSUP


def test_binding_fails_loudly_without_gpu_tensors():
    import torch

    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        h3.h3f_gated_residual(x, x, x[0])


# --- residual difference (step-reuse test) --------------------------------------------------

def test_residual_l1_validation():
    L.h3f_residual_l1_workspace_bytes.restype = ctypes.c_size_t
    need = L.h3f_residual_l1_workspace_bytes(125120, 5120, BF16)
    assert need > 0 and need % 16 == 0
    assert L.h3f_residual_l1_workspace_bytes(0, 5120, BF16) == 0
    assert L.h3f_residual_l1_workspace_bytes(4, 5121, BF16) == 0

    def l1(out=A(0), cur=A(1), cs=512, prev=A(2), ps=512, dt=BF16, rows=4, hidden=512, ws=A(3),
           wsb=1 << 20):
        return L.h3f_residual_l1(out, cur, cs, prev, ps, dt, rows, hidden, ws, wsb, None)

    assert l1(out=None) == NULLP
    assert l1(rows=0) == SHAPE
    assert l1(prev=None) == NULLP
    assert l1(dt=4) == DTYPE
    assert l1(hidden=500) == SHAPE
    assert l1(cur=P(0x20000008)) == MISAL
    assert l1(out=P(0x10000004)) == MISAL
    assert l1(cs=256) == STRIDE
    assert l1(ws=None) == WORKSPACE
    assert l1(wsb=8) == WORKSPACE
    assert l1(ws=P(0x40000008)) == WORKSPACE
    assert l1(ws=A(1)) == ALIAS
    assert l1(out=A(2)) == ALIAS


# --- block-sparse attention router ---------------------------------------------------------

def test_subblock_plan_sizes():
    # 5 s sequence: 125,120 tokens in blocks of 128 -> 978 blocks; sparsity 0.8 skips
    # floor(782.4) = 782 of them from the tenth step on
    assert h3.h3f_subblock_plan(125120, 40, 128, 128, 0.8, 10) == (978, 196, 2 * 40 * 978 * 128 * 4)
    assert h3.h3f_subblock_plan(125120, 40, 128, 128, 0.75, 50)[1] == 978 - 733
    assert h3.h3f_subblock_plan(125120, 40, 128, 128, 0.8, 9)[1] == 978
    assert h3.h3f_subblock_plan(246208, 40, 128, 128, 0.8, 10)[:2] == (1924, 1924 - 1539)
    # the largest sparsity below 1 still keeps one block
    assert h3.h3f_subblock_plan(4096, 1, 128, 1024, 1.0 - 2.0 ** -53, 10)[1] == 1


def test_subblock_plan_validation():
    def plan(rows=8192, heads=8, hd=128, block=128, sp=0.8, step=10):
        return L.h3f_subblock_plan(rows, heads, hd, block, sp, step, None, None, None)

    assert plan() == OK
    assert plan(rows=4095) == UNSUP            # sequence shorter than 4096 tokens
    assert plan(hd=64) == UNSUP                # head dimension other than 128
    assert plan(rows=8193 * 128, block=128) == UNSUP  # more than 8192 blocks
    assert plan(block=0) == SHAPE
    assert plan(heads=0) == SHAPE
    assert plan(sp=1.0) == BADVAL
    assert plan(sp=-0.01) == BADVAL
    assert plan(sp=float("nan")) == BADVAL
    assert plan(step=0) == BADVAL


def test_subblock_route_validation():
    # 4096 tokens x 8 heads x 128 (8 KB rows / 32 MB per tensor), 32 blocks of 128;
    # fake device addresses 256 MB apart: every call below fails validation.
    def route(kv=A(0), sc=A(1), ss=32, q=A(2), qrs=1024, qhs=128, k=A(3), krs=1024, khs=128,
              dt=BF16, rows=4096, heads=8, hd=128, block=128, sp=0.8, step=10, ws=A(4),
              wsb=1 << 20):
        return L.h3f_subblock_route(kv, sc, ss, q, qrs, qhs, k, krs, khs, dt, rows, heads, hd,
                                    block, sp, step, ws, wsb, None)

    assert route(kv=None) == NULLP
    assert route(sc=None) == NULLP
    assert route(k=None) == NULLP
    assert route(dt=3) == DTYPE
    assert route(dt=F32) == UNSUP              # the router runs on bf16 q / k only
    assert route(rows=2048) == UNSUP
    assert route(hd=64, qhs=64, khs=64) == UNSUP
    assert route(sp=1.5) == BADVAL
    assert route(q=P(0x30000008)) == MISAL
    assert route(kv=P(0x10000002)) == MISAL
    assert route(sc=P(0x20000004)) == MISAL          # scores take 16-byte stores
    assert route(qrs=(1 << 31) + 8) == UNSUP
    assert route(qrs=1020) == STRIDE
    assert route(khs=120) == STRIDE
    assert route(qrs=512) == STRIDE            # rows would overlap (8 heads x 128 > 512)
    assert route(ws=None) == WORKSPACE
    assert route(wsb=2 * 8 * 32 * 512 - 16) == WORKSPACE
    assert route(ws=P(0x50000008)) == WORKSPACE
    assert route(sc=A(2)) == ALIAS             # scores on top of q
    assert route(ws=P(0x10000000 + 64)) == ALIAS   # workspace inside kv_blocks
    assert route(kv=P(0x40000000 + 1024)) == ALIAS  # kv_blocks inside k
    # scores rows: at least n_blocks (32) floats apart, one head's matrix within
    # 32-bit offsets (2^32 - 16 bytes), padded rows part of the footprint
    assert route(ss=31) == STRIDE
    assert route(ss=0) == STRIDE
    assert route(ss=-32) == STRIDE
    assert route(ss=31, step=3) == STRIDE              # checked on dense steps too
    assert route(ss=(1 << 32) // 128) == UNSUP          # 32 x 2^25 floats = 2^32 bytes
    assert route(ss=1 << 62) == UNSUP                   # no overflow on the way
    # 256 rows 256 B apart: only the last row's 128 written bytes reach q (A(2))
    assert route(ss=64, sc=P(0x30000000 - 255 * 256 - 112)) == ALIAS


def test_qk_pool_validation():
    # the fused QK + router pooling: QK's own checks, then the router's
    # preconditions and its workspace (4096 tokens x 8 heads, 32 blocks of 128:
    # 2 x 8 x 32 x 128 x 4 = 256 KiB of block means)
    def qkp(qo=A(0), ko=A(1), q=A(2), k=A(3), qw=A(4), kw=A(5), dt=BF16, rows=4096, heads=8,
            hd=128, r=None, block=128, ws=A(6), wsb=1 << 18, qrs=1024):
        r = rope() if r is None else r
        return L.h3f_qk_rmsnorm_rope3d_pool(qo, 1024, 128, ko, 1024, 128, q, qrs, 128, k, 1024,
                                            128, qw, kw, dt, rows, heads, hd, ctypes.c_float(1e-6),
                                            ctypes.byref(r), block, ws, wsb, None)

    assert qkp(q=None) == NULLP
    assert qkp(rows=4095) == UNSUP            # the router's minimum sequence
    assert qkp(rows=0) == UNSUP               # not a no-op here
    assert qkp(hd=64) == UNSUP
    assert qkp(block=0) == SHAPE
    assert qkp(dt=F32) == UNSUP               # router input is bf16 only
    assert qkp(dt=3) == DTYPE
    assert qkp(r=rope(d_t=40)) == SHAPE         # 40 + 48 + 48 != head_dim
    assert qkp(ws=None) == WORKSPACE
    assert qkp(wsb=(1 << 18) - 16) == WORKSPACE
    assert qkp(ws=P(0x70000008)) == WORKSPACE
    assert qkp(ws=P(0x10000000 + 4096)) == ALIAS   # inside q_out
    assert qkp(qrs=1020) == STRIDE


def test_route_pooled_validation():
    def rp(kv=A(0), sc=A(1), ss=32, rows=4096, heads=8, hd=128, block=128, sp=0.8, step=10,
           ws=A(2), wsb=1 << 18):
        return L.h3f_subblock_route_pooled(kv, sc, ss, rows, heads, hd, block, sp, step, ws, wsb,
                                           None)

    assert rp(kv=None) == NULLP
    assert rp(sc=None) == NULLP
    assert rp(rows=100) == UNSUP
    assert rp(sp=1.0) == BADVAL
    assert rp(step=0) == BADVAL
    assert rp(sc=P(0x20000004)) == MISAL
    assert rp(ws=None) == WORKSPACE
    assert rp(wsb=(1 << 18) - 1) == WORKSPACE
    assert rp(ws=P(0x20000000 + 256)) == ALIAS     # workspace inside the scores
    assert rp(ss=16) == STRIDE
    assert rp(ss=16, step=2) == STRIDE
    assert rp(ss=(1 << 32) // 128) == UNSUP


def test_subblock_binding_checks_shapes_before_the_library():
    import torch

    q = torch.zeros(4096, 2, 128, dtype=torch.bfloat16)
    kv = torch.zeros(2, 32, 7, dtype=torch.int32)
    sc = torch.zeros(2, 32, 32)
    with pytest.raises(ValueError):
        h3.h3f_subblock_route(kv, sc, q, q, 128, 0.8, 10)


def test_absurd_strides_are_rejected_without_overflow():
    # strides whose footprints exceed 2^62 bytes: refused before any span arithmetic
    # could overflow (every value is a vector multiple, so only the size check can fire)
    big = 1 << 61
    assert gated(xs=big) == UNSUP
    assert gated(rpg=5, gs=big) == UNSUP
    assert swiglu(as_=big) == UNSUP
    assert adaln(xs=big) == UNSUP
    assert adaln(rpg=1, gs=big) == UNSUP
    assert fused(hs=big) == UNSUP
    assert qk(qhs=big) == UNSUP
    assert qk(krs=big) == UNSUP
    assert L.h3f_residual_l1(A(0), A(1), big, A(2), 512, BF16, 4, 512, A(3), 1 << 20,
                             None) == UNSUP


def test_adaln_affine_validation():
    def aff(y=A(0), yd=BF16, ys=512, x=A(1), xd=BF16, xs=512, gm=A(4), bt=P(0x50000000 + 4096),
            sh=A(2), sc=A(3), gs=0, rpg=8, rows=8, hidden=512):
        return L.h3f_adaln_affine_modulate(y, yd, ys, x, xd, xs, gm, bt, sh, sc, gs, rpg, rows,
                                           hidden, ctypes.c_float(1e-6), None)

    assert aff(gm=None, rows=0) == OK
    assert aff(gm=None) == NULLP
    assert aff(bt=None) == NULLP
    assert aff(xd=F32, yd=F32, hidden=16384) == UNSUP
    assert aff(gm=P(0x50000008)) == MISAL
    assert aff(bt=P(0x50000000 + 4100)) == MISAL
    assert aff(gm=P(0x10000000 + 64)) == ALIAS   # gamma inside y
    assert aff(bt=P(0x10000000 + 512)) == ALIAS  # beta inside y
    assert aff(yd=F32) == DTYPE
    assert aff(hidden=500) == SHAPE
