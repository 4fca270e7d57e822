"""Python binding of libh3fused (see include/h3fused.h): fused, memory-bound
per-token DiT operators and the block-sparse attention router, as hand-written
HIP kernels for gfx950 (MI355X).

Argument marshalling only.  Each function takes torch tensors that live on the
GPU (torch provides device memory and the current stream), passes their
pointers, strides and types to the C entry point of the same name, and raises
H3FError when the library rejects the call.  Every step of the computation runs
in the HIP kernels; there is no fallback of any kind: without the built library
every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libh3fused.so")

H3F_F32 = 0
H3F_BF16 = 1
H3F_ROPE_INTERLEAVED = 0
H3F_ROPE_HALF_SPLIT = 1

STATUS = {
    0: "H3F_OK", 1: "H3F_ERR_NULL_POINTER", 2: "H3F_ERR_BAD_SHAPE", 3: "H3F_ERR_BAD_STRIDE",
    4: "H3F_ERR_MISALIGNED", 5: "H3F_ERR_BAD_DTYPE", 6: "H3F_ERR_ALIASING", 7: "H3F_ERR_LAUNCH",
    8: "H3F_ERR_UNSUPPORTED", 9: "H3F_ERR_WORKSPACE", 10: "H3F_ERR_BAD_VALUE",
}

H3F_SUBBLOCK_FIRST_STEP = 10

EXPORTS = [
    "h3f_abi_version", "h3f_status_string", "h3f_rope3d_positions", "h3f_adaln_modulate",
    "h3f_gated_residual", "h3f_swiglu", "h3f_qk_rmsnorm_rope3d", "h3f_gated_residual_adaln",
    "h3f_stream_copy", "h3f_residual_l1_workspace_bytes", "h3f_residual_l1",
    "h3f_subblock_plan", "h3f_subblock_route", "h3f_adaln_affine_modulate",
    "h3f_qk_rmsnorm_rope3d_pool", "h3f_subblock_route_pooled", "h3f_stream_read",
    "h3f_stream_fill", "h3f_stream_fill_bursts", "h3f_residual_l1_noalloc",
    "h3f_residual_l1_noalloc_max_bytes",
]


class H3FError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = lib().h3f_status_string(status).decode()
        super().__init__(f"{fn}: {self.name} ({msg})")


class Rope3D(ctypes.Structure):
    """Mirror of h3f_rope3d_t."""
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("n_audio", ctypes.c_int32), ("d_t", ctypes.c_int32), ("d_h", ctypes.c_int32),
        ("d_w", ctypes.c_int32), ("pairing", ctypes.c_int32), ("theta", ctypes.c_double),
        ("token_offset", ctypes.c_int64), ("positions", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded libh3fused.so (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libh3fused.so is not built ({LIB_PATH}); run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f, st = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                              ctypes.c_int)
        L.h3f_abi_version.restype = ctypes.c_int
        L.h3f_status_string.argtypes = [st]
        L.h3f_status_string.restype = ctypes.c_char_p
        L.h3f_rope3d_positions.argtypes = [p, i64, ctypes.POINTER(Rope3D), p]
        L.h3f_adaln_modulate.argtypes = [p, st, i64, p, st, i64, p, p, i64, i64, i64, i64, f, p]
        L.h3f_adaln_affine_modulate.argtypes = [p, st, i64, p, st, i64, p, p, p, p, i64, i64,
                                                i64, i64, f, p]
        L.h3f_gated_residual.argtypes = [p, st, i64, p, st, i64, p, i64, i64, i64, i64, p]
        L.h3f_swiglu.argtypes = [p, i64, p, i64, p, i64, st, i64, i64, p]
        L.h3f_qk_rmsnorm_rope3d.argtypes = [p, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64,
                                            p, p, st, i64, i32, i32, f, ctypes.POINTER(Rope3D), p]
        L.h3f_gated_residual_adaln.argtypes = [p, st, i64, p, st, i64, p, p, p, i64, i64, p, st,
                                               i64, i64, i64, f, p]
        L.h3f_stream_copy.argtypes = [p, p, i64, p]
        L.h3f_stream_read.argtypes = [p, i64, i32, p, p]
        L.h3f_stream_fill.argtypes = [p, i64, ctypes.c_uint32, p]
        L.h3f_stream_fill_bursts.argtypes = [p, i64, ctypes.c_uint32, i32, p]
        L.h3f_residual_l1.argtypes = [p, p, i64, p, i64, st, i64, i64, p, ctypes.c_size_t, p]
        L.h3f_residual_l1_noalloc.argtypes = [p, p, i64, p, i64, st, i64, i64, p]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = st
        L.h3f_residual_l1_noalloc_max_bytes.argtypes = []
        L.h3f_residual_l1_noalloc_max_bytes.restype = ctypes.c_size_t
        L.h3f_residual_l1_workspace_bytes.argtypes = [i64, i64, st]
        L.h3f_residual_l1_workspace_bytes.restype = ctypes.c_size_t
        L.h3f_subblock_plan.argtypes = [i64, i32, i32, i32, ctypes.c_double, i32,
                                        ctypes.POINTER(i32), ctypes.POINTER(i32),
                                        ctypes.POINTER(ctypes.c_size_t)]
        L.h3f_subblock_route.argtypes = [p, p, i64, p, i64, i64, p, i64, i64, st, i64, i32, i32,
                                         i32, ctypes.c_double, i32, p, ctypes.c_size_t, p]
        L.h3f_qk_rmsnorm_rope3d_pool.argtypes = [p, i64, i64, p, i64, i64, p, i64, i64, p, i64,
                                                 i64, p, p, st, i64, i32, i32, f,
                                                 ctypes.POINTER(Rope3D), i32, p, ctypes.c_size_t,
                                                 p]
        L.h3f_subblock_route_pooled.argtypes = [p, p, i64, i64, i32, i32, i32, ctypes.c_double,
                                                i32, p, ctypes.c_size_t, p]
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().h3f_abi_version()


# ---------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------

def _dtype(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return H3F_F32
    if t.dtype == torch.bfloat16:
        return H3F_BF16
    raise TypeError(f"libh3fused takes float32 or bfloat16 tensors, got {t.dtype}")


def _dev(*ts):
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libh3fused operates on GPU tensors only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors of a call must be on one device")
    return dev


def _stream(dev, stream):
    import torch

    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check(fn, status):
    if status != 0:
        raise H3FError(fn, status)


def _rows2d(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D tensor with unit inner stride")
    return t.shape[0], t.shape[1], t.stride(0)


def _mod(v, hidden, name):
    """Modulation vector(s): [hidden] or [groups, hidden] -> (groups, group stride)."""
    if v.dim() == 1:
        v2 = v.view(1, -1)
    else:
        v2 = v
    if v2.dim() != 2 or v2.shape[1] != hidden or v2.stride(1) != 1:
        raise ValueError(f"{name}: expected [hidden] or [groups, hidden] with unit inner stride")
    return v2.shape[0], v2.stride(0)


def _rows_per_group(rows, groups, rows_per_group):
    """Rows per modulation group.  The library reads group ceil(rows / rpg) - 1 as
    its last one, so the tensors must hold at least that many groups."""
    if rows_per_group is not None:
        rpg = int(rows_per_group)
        if rpg < 1:
            raise ValueError("rows_per_group must be >= 1")
    elif groups == 1:
        rpg = max(rows, 1)
    elif rows % groups:
        raise ValueError("rows_per_group is needed when rows is not a multiple of the group count")
    else:
        rpg = rows // groups
    if rows > 0 and -(-rows // rpg) > groups:
        raise ValueError(f"{rows} rows at {rpg} rows per group need {-(-rows // rpg)} modulation "
                         f"groups; the modulation tensors hold {groups}")
    return rpg


def _same_dtype(ref, name_ref, *named):
    """Modulation vectors and LayerNorm weights are read in the type of the stream
    tensor they act on."""
    for t, n in named:
        if t.dtype != ref.dtype:
            raise TypeError(f"{n} must have {name_ref}'s dtype ({ref.dtype}), got {t.dtype}")


# ---------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------

def h3f_rope3d_positions(pos, rope: Rope3D, stream=None):
    """pos: int32 [rows, 3] GPU tensor, filled with (t, h, w) of each row."""
    import torch

    if pos.dtype != torch.int32 or pos.dim() != 2 or pos.shape[1] != 3 or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 [rows, 3] tensor")
    dev = _dev(pos)
    _check("h3f_rope3d_positions", lib().h3f_rope3d_positions(
        _ptr(pos), pos.shape[0], ctypes.byref(rope), _stream(dev, stream)))
    return pos


def h3f_adaln_modulate(y, x, shift, scale, eps: float = 1e-6, rows_per_group=None, stream=None):
    """y[r] = LN(x[r]) * (1 + scale[g]) + shift[g]; y may be x itself."""
    dev = _dev(y, x, shift, scale)
    rows, hidden, xs = _rows2d(x, "x")
    yr, yh, ys = _rows2d(y, "y")
    if (yr, yh) != (rows, hidden):
        raise ValueError("y and x shapes differ")
    groups, gs = _mod(shift, hidden, "shift")
    g2, gs2 = _mod(scale, hidden, "scale")
    if (groups, gs) != (g2, gs2):
        raise ValueError("shift and scale must share shape and strides")
    _same_dtype(x, "x", (shift, "shift"), (scale, "scale"))
    rpg = _rows_per_group(rows, groups, rows_per_group)
    _check("h3f_adaln_modulate", lib().h3f_adaln_modulate(
        _ptr(y), _dtype(y), ys, _ptr(x), _dtype(x), xs, _ptr(shift), _ptr(scale), gs, rpg, rows,
        hidden, eps, _stream(dev, stream)))
    return y


def h3f_adaln_affine_modulate(y, x, gamma, beta, shift, scale, eps: float = 1e-6,
                              rows_per_group=None, stream=None):
    """y[r] = (LN(x[r]) * gamma + beta) * (1 + scale[g]) + shift[g]; gamma, beta [hidden]."""
    dev = _dev(y, x, gamma, beta, shift, scale)
    rows, hidden, xs = _rows2d(x, "x")
    yr, yh, ys = _rows2d(y, "y")
    if (yr, yh) != (rows, hidden):
        raise ValueError("y and x shapes differ")
    for v, n in ((gamma, "gamma"), (beta, "beta")):
        if v.numel() != hidden or not v.is_contiguous():
            raise ValueError(f"{n}: expected a contiguous [hidden] tensor")
    groups, gs = _mod(shift, hidden, "shift")
    g2, gs2 = _mod(scale, hidden, "scale")
    if (groups, gs) != (g2, gs2):
        raise ValueError("shift and scale must share shape and strides")
    _same_dtype(x, "x", (shift, "shift"), (scale, "scale"), (gamma, "gamma"), (beta, "beta"))
    rpg = _rows_per_group(rows, groups, rows_per_group)
    _check("h3f_adaln_affine_modulate", lib().h3f_adaln_affine_modulate(
        _ptr(y), _dtype(y), ys, _ptr(x), _dtype(x), xs, _ptr(gamma), _ptr(beta), _ptr(shift),
        _ptr(scale), gs, rpg, rows, hidden, eps, _stream(dev, stream)))
    return y


def h3f_gated_residual(x, h, gate, rows_per_group=None, stream=None):
    """x[r] += gate[g] * h[r], in place."""
    dev = _dev(x, h, gate)
    rows, hidden, xs = _rows2d(x, "x")
    hr, hh, hs = _rows2d(h, "h")
    if (hr, hh) != (rows, hidden):
        raise ValueError("h and x shapes differ")
    groups, gs = _mod(gate, hidden, "gate")
    _same_dtype(x, "x", (gate, "gate"))
    rpg = _rows_per_group(rows, groups, rows_per_group)
    _check("h3f_gated_residual", lib().h3f_gated_residual(
        _ptr(x), _dtype(x), xs, _ptr(h), _dtype(h), hs, _ptr(gate), gs, rpg, rows, hidden,
        _stream(dev, stream)))
    return x


def h3f_swiglu(out, a, b=None, stream=None):
    """out = silu(a) * b.  With b None, `a` is the packed [rows, 2*inner] gate/up
    tensor whose first half is the gate and second half the up projection."""
    if b is None:
        inner2 = a.shape[-1]
        if inner2 % 2:
            raise ValueError("packed gate/up width must be even")
        a, b = a[:, : inner2 // 2], a[:, inner2 // 2:]
    dev = _dev(out, a, b)
    rows, inner, os_ = _rows2d(out, "out")
    ar, ai, as_ = _rows2d(a, "a")
    br, bi, bs = _rows2d(b, "b")
    if (ar, ai) != (rows, inner) or (br, bi) != (rows, inner):
        raise ValueError("out, a, b shapes differ")
    if not (out.dtype == a.dtype == b.dtype):
        raise TypeError("out, a, b must share a dtype")
    _check("h3f_swiglu", lib().h3f_swiglu(
        _ptr(out), os_, _ptr(a), as_, _ptr(b), bs, _dtype(out), rows, inner,
        _stream(dev, stream)))
    return out


def make_rope(T, H, W, n_audio, split, theta=10000.0, token_offset=0, positions=None,
              pairing=H3F_ROPE_INTERLEAVED) -> Rope3D:
    """Token grid and RoPE parameters.  `positions`, when given, is a contiguous int32
    [rows, 3] GPU tensor of (t, h, w) per row; the returned struct keeps a reference
    to it, and the QK calls check it against their rows and device."""
    import torch

    r = Rope3D()
    r.T, r.H, r.W, r.n_audio = int(T), int(H), int(W), int(n_audio)
    r.d_t, r.d_h, r.d_w = (int(s) for s in split)
    r.pairing = int(pairing)
    r.theta = float(theta)
    r.token_offset = int(token_offset)
    if positions is not None:
        if (positions.dtype != torch.int32 or positions.dim() != 2 or positions.shape[1] != 3
                or not positions.is_contiguous()):
            raise ValueError("positions must be a contiguous int32 [rows, 3] tensor")
        if not positions.is_cuda:
            raise ValueError("positions must be a GPU tensor")
    r.positions = None if positions is None else positions.data_ptr()
    r.positions_tensor = positions  # keeps the array alive as long as the struct
    return r


def _check_rope(rope: Rope3D, rows: int, dev):
    pos = getattr(rope, "positions_tensor", None)
    if rope.positions and pos is None:
        raise ValueError("rope.positions was set outside make_rope; pass positions to make_rope")
    if pos is not None:
        if pos.shape[0] < rows:
            raise ValueError(f"rope positions hold {pos.shape[0]} rows; the call has {rows}")
        if pos.device != dev:
            raise ValueError("rope positions must be on the device of q and k")


def _heads3d(t, name):
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name}: expected [rows, heads, head_dim] with unit inner stride")
    return t.shape, t.stride(0), t.stride(1)


def _qk_args(q_out, k_out, q, k, q_weight, k_weight):
    shp, qrs, qhs = _heads3d(q, "q")
    kshp, krs, khs = _heads3d(k, "k")
    qoshp, qors, qohs = _heads3d(q_out, "q_out")
    koshp, kors, kohs = _heads3d(k_out, "k_out")
    if not (shp == kshp == qoshp == koshp):
        raise ValueError("q, k, q_out, k_out shapes differ")
    rows, heads, head_dim = shp
    for w, n in ((q_weight, "q_weight"), (k_weight, "k_weight")):
        if w.numel() != head_dim or not w.is_contiguous():
            raise ValueError(f"{n}: expected a contiguous [head_dim] tensor")
    dt = _dtype(q)
    for t in (k, q_out, k_out, q_weight, k_weight):
        if _dtype(t) != dt:
            raise TypeError("all qk tensors must share one dtype")
    return (_ptr(q_out), qors, qohs, _ptr(k_out), kors, kohs, _ptr(q), qrs, qhs, _ptr(k), krs,
            khs, _ptr(q_weight), _ptr(k_weight), dt, rows, heads, head_dim)


def h3f_qk_rmsnorm_rope3d_pool(q_out, k_out, q, k, q_weight, k_weight, rope: Rope3D,
                               block: int, workspace, eps: float = 1e-6, stream=None):
    """h3f_qk_rmsnorm_rope3d that also writes the router's block means of q_out and
    k_out into `workspace` (uint8 GPU tensor of at least the bytes h3f_subblock_plan
    gives for the same rows, heads, head_dim and block)."""
    dev = _dev(q_out, k_out, q, k, q_weight, k_weight, workspace)
    args = _qk_args(q_out, k_out, q, k, q_weight, k_weight)
    _check_rope(rope, q.shape[0], dev)
    _check("h3f_qk_rmsnorm_rope3d_pool", lib().h3f_qk_rmsnorm_rope3d_pool(
        *args, eps, ctypes.byref(rope), block, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev, stream)))
    return q_out, k_out


def _route_outputs(kv_blocks, scores, heads, nb, keep):
    """Checks the router's outputs and returns the row stride of scores in floats:
    kv_blocks int32 [heads, nb, keep] contiguous; scores float32 [heads, nb, nb]
    whose rows are evenly spaced, dense or the first nb columns of a contiguous
    [heads, nb, S] buffer (S a multiple of 32 lets the kernel write whole lines)."""
    import torch

    if kv_blocks.dtype != torch.int32 or scores.dtype != torch.float32:
        raise TypeError("kv_blocks must be int32 and scores float32")
    if tuple(kv_blocks.shape) != (heads, nb, keep) or tuple(scores.shape) != (heads, nb, nb):
        raise ValueError(f"kv_blocks must be [{heads}, {nb}, {keep}] and scores [{heads}, {nb}, {nb}]")
    if not kv_blocks.is_contiguous():
        raise ValueError("kv_blocks must be contiguous")
    s0, s1, s2 = scores.stride()
    if s2 != 1 or s1 < nb or (heads > 1 and s0 != nb * s1):
        raise ValueError("scores rows must be evenly spaced: strides (nb * S, S, 1) with S >= nb")
    return s1


def scores_view(heads: int, n_blocks: int, device, pad_to: int = 32):
    """A float32 [heads, n_blocks, n_blocks] view for the router's scores whose rows
    are padded to a multiple of pad_to floats (32: 128-byte rows, each line of
    scores written whole).  The pad columns are never written."""
    import torch

    s = -(-n_blocks // pad_to) * pad_to
    return torch.empty(heads, n_blocks, s, dtype=torch.float32, device=device)[:, :, :n_blocks]


def h3f_subblock_route_pooled(kv_blocks, scores, rows: int, heads: int, block: int,
                              sparsity: float, step: int, workspace, stream=None):
    """Router score + selection from the block means h3f_qk_rmsnorm_rope3d_pool wrote
    into `workspace`; kv_blocks / scores as for h3f_subblock_route."""
    dev = _dev(kv_blocks, scores, workspace)
    nb, keep, _ = h3f_subblock_plan(rows, heads, 128, block, sparsity, step)
    srs = _route_outputs(kv_blocks, scores, heads, nb, keep)
    _check("h3f_subblock_route_pooled", lib().h3f_subblock_route_pooled(
        _ptr(kv_blocks), _ptr(scores), srs, rows, heads, 128, block, float(sparsity), step,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev, stream)))
    return kv_blocks, scores


def h3f_qk_rmsnorm_rope3d(q_out, k_out, q, k, q_weight, k_weight, rope: Rope3D,
                          eps: float = 1e-6, stream=None):
    """Per-head RMSNorm of q and k, then 3D RoPE.  Tensors are [rows, heads, head_dim]
    views (any row / head strides); q_out / k_out may be q / k themselves."""
    dev = _dev(q_out, k_out, q, k, q_weight, k_weight)
    shp, qrs, qhs = _heads3d(q, "q")
    kshp, krs, khs = _heads3d(k, "k")
    qoshp, qors, qohs = _heads3d(q_out, "q_out")
    koshp, kors, kohs = _heads3d(k_out, "k_out")
    if not (shp == kshp == qoshp == koshp):
        raise ValueError("q, k, q_out, k_out shapes differ")
    rows, heads, head_dim = shp
    for w, n in ((q_weight, "q_weight"), (k_weight, "k_weight")):
        if w.numel() != head_dim or not w.is_contiguous():
            raise ValueError(f"{n}: expected a contiguous [head_dim] tensor")
    dt = _dtype(q)
    for t in (k, q_out, k_out, q_weight, k_weight):
        if _dtype(t) != dt:
            raise TypeError("all qk tensors must share one dtype")
    _check_rope(rope, rows, dev)
    _check("h3f_qk_rmsnorm_rope3d", lib().h3f_qk_rmsnorm_rope3d(
        _ptr(q_out), qors, qohs, _ptr(k_out), kors, kohs, _ptr(q), qrs, qhs, _ptr(k), krs, khs,
        _ptr(q_weight), _ptr(k_weight), dt, rows, heads, head_dim, eps, ctypes.byref(rope),
        _stream(dev, stream)))
    return q_out, k_out


def h3f_gated_residual_adaln(x, h, gate, shift, scale, y, eps: float = 1e-6,
                             rows_per_group=None, stream=None):
    """x[r] += gate[g] * h[r] (in place), then y[r] = AdaLN(x[r]; shift[g], scale[g])."""
    dev = _dev(x, h, gate, shift, scale, y)
    rows, hidden, xs = _rows2d(x, "x")
    hr, hh, hs = _rows2d(h, "h")
    yr, yh, ys = _rows2d(y, "y")
    if (hr, hh) != (rows, hidden) or (yr, yh) != (rows, hidden):
        raise ValueError("x, h, y shapes differ")
    shapes = [_mod(v, hidden, n) for v, n in ((gate, "gate"), (shift, "shift"), (scale, "scale"))]
    if len(set(shapes)) != 1:
        raise ValueError("gate, shift and scale must share shape and strides")
    groups, gs = shapes[0]
    _same_dtype(x, "x", (gate, "gate"), (shift, "shift"), (scale, "scale"))
    rpg = _rows_per_group(rows, groups, rows_per_group)
    _check("h3f_gated_residual_adaln", lib().h3f_gated_residual_adaln(
        _ptr(x), _dtype(x), xs, _ptr(h), _dtype(h), hs, _ptr(gate), _ptr(shift), _ptr(scale), gs,
        rpg, _ptr(y), _dtype(y), ys, rows, hidden, eps, _stream(dev, stream)))
    return x, y


def h3f_residual_l1_workspace_bytes(rows: int, hidden: int, dtype) -> int:
    """Workspace bytes h3f_residual_l1 needs for a [rows, hidden] tensor of dtype."""
    import torch

    dt = H3F_BF16 if dtype == torch.bfloat16 else H3F_F32
    return int(lib().h3f_residual_l1_workspace_bytes(rows, hidden, dt))


def h3f_residual_l1(out, cur, prev, workspace=None, stream=None):
    """out (float64 [3] on the GPU) = (sum|cur - prev|, sum|prev|, ratio).
    workspace: uint8 GPU tensor of at least h3f_residual_l1_workspace_bytes();
    allocated here (torch) when None."""
    import torch

    dev = _dev(out, cur, prev)
    if out.dtype != torch.float64 or out.numel() < 3 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float64 tensor of >= 3 elements")
    rows, hidden, cs = _rows2d(cur, "cur")
    pr, ph, ps = _rows2d(prev, "prev")
    if (pr, ph) != (rows, hidden) or cur.dtype != prev.dtype:
        raise ValueError("cur and prev must share shape and dtype")
    need = h3f_residual_l1_workspace_bytes(rows, hidden, cur.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check("h3f_residual_l1", lib().h3f_residual_l1(
        _ptr(out), _ptr(cur), cs, _ptr(prev), ps, _dtype(cur), rows, hidden, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev, stream)))
    return out


def h3f_residual_l1_noalloc(out, cur, prev, stream=None):
    """h3f_residual_l1 with the library's own device scratch instead of a workspace
    (no allocation of any kind; for callers that cannot allocate).  Calls that
    overlap on one GPU share that scratch and race."""
    import torch

    dev = _dev(out, cur, prev)
    if out.dtype != torch.float64 or out.numel() < 3 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float64 tensor of >= 3 elements")
    rows, hidden, cs = _rows2d(cur, "cur")
    pr, ph, ps = _rows2d(prev, "prev")
    if (pr, ph) != (rows, hidden) or cur.dtype != prev.dtype:
        raise ValueError("cur and prev must share shape and dtype")
    _check("h3f_residual_l1_noalloc", lib().h3f_residual_l1_noalloc(
        _ptr(out), _ptr(cur), cs, _ptr(prev), ps, _dtype(cur), rows, hidden,
        _stream(dev, stream)))
    return out


def h3f_residual_l1_noalloc_max_bytes() -> int:
    """Bytes of the device scratch behind h3f_residual_l1_noalloc; calls whose
    h3f_residual_l1_workspace_bytes() exceeds it are rejected."""
    return int(lib().h3f_residual_l1_noalloc_max_bytes())


def h3f_subblock_plan(rows: int, heads: int, head_dim: int, block: int, sparsity: float,
                      step: int):
    """(n_blocks, keep, workspace_bytes) of one router call (host-only)."""
    nb, keep, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
    _check("h3f_subblock_plan", lib().h3f_subblock_plan(
        rows, heads, head_dim, block, float(sparsity), step, ctypes.byref(nb), ctypes.byref(keep),
        ctypes.byref(ws)))
    return nb.value, keep.value, ws.value


def h3f_subblock_route(kv_blocks, scores, q, k, block: int, sparsity: float, step: int,
                       workspace=None, stream=None):
    """Block-sparse attention router.  q, k: bf16 [rows, heads, head_dim] views;
    kv_blocks: int32 [heads, n_blocks, keep], contiguous; scores: float32 [heads,
    n_blocks, n_blocks], dense or padded rows (scores_view); sizes from
    h3f_subblock_plan.  workspace: uint8 GPU tensor of at least the planned bytes;
    allocated here (torch) when None."""
    import torch

    dev = _dev(kv_blocks, scores, q, k)
    shp, qrs, qhs = _heads3d(q, "q")
    kshp, krs, khs = _heads3d(k, "k")
    if shp != kshp:
        raise ValueError("q and k shapes differ")
    rows, heads, head_dim = shp
    nb, keep, need = h3f_subblock_plan(rows, heads, head_dim, block, sparsity, step)
    srs = _route_outputs(kv_blocks, scores, heads, nb, keep)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check("h3f_subblock_route", lib().h3f_subblock_route(
        _ptr(kv_blocks), _ptr(scores), srs, _ptr(q), qrs, qhs, _ptr(k), krs, khs, _dtype(q), rows,
        heads, head_dim, block, float(sparsity), step, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev, stream)))
    return kv_blocks, scores


def h3f_stream_copy(dst, src, stream=None):
    """Byte copy src -> dst (measurement helper); both contiguous, same byte size."""
    dev = _dev(dst, src)
    nb = src.numel() * src.element_size()
    if not (dst.is_contiguous() and src.is_contiguous()) or dst.numel() * dst.element_size() != nb:
        raise ValueError("dst and src must be contiguous with equal byte sizes")
    _check("h3f_stream_copy", lib().h3f_stream_copy(_ptr(dst), _ptr(src), nb,
                                                    _stream(dev, stream)))
    return dst


def h3f_stream_read(src, sink, cached: bool = False, stream=None):
    """Read all of src (contiguous) once (measurement helper); sink: >= 16-byte
    GPU tensor that is written only if the loaded data folds to a fixed value."""
    dev = _dev(src, sink)
    if not (src.is_contiguous() and sink.is_contiguous()) or sink.numel() * sink.element_size() < 16:
        raise ValueError("src must be contiguous and sink a contiguous tensor of >= 16 bytes")
    _check("h3f_stream_read", lib().h3f_stream_read(
        _ptr(src), src.numel() * src.element_size(), 1 if cached else 0, _ptr(sink),
        _stream(dev, stream)))
    return src


def h3f_stream_fill_bursts(dst, kib_per_wavefront: int, value: int = 0, stream=None):
    """h3f_stream_fill with each wavefront writing its own kib_per_wavefront KiB
    (1, 2, 5 or 10) before it ends (measurement helper)."""
    dev = _dev(dst)
    if not dst.is_contiguous():
        raise ValueError("dst must be contiguous")
    _check("h3f_stream_fill_bursts", lib().h3f_stream_fill_bursts(
        _ptr(dst), dst.numel() * dst.element_size(), int(value) & 0xFFFFFFFF,
        int(kib_per_wavefront), _stream(dev, stream)))
    return dst


def h3f_stream_fill(dst, value: int = 0, stream=None):
    """Write the 32-bit pattern `value` over all of dst (contiguous; measurement helper)."""
    dev = _dev(dst)
    if not dst.is_contiguous():
        raise ValueError("dst must be contiguous")
    _check("h3f_stream_fill", lib().h3f_stream_fill(
        _ptr(dst), dst.numel() * dst.element_size(), int(value) & 0xFFFFFFFF,
        _stream(dev, stream)))
    return dst
